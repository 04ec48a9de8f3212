/*
 * fa.h -- exact, IO-aware tiled softmax attention for AMD Instinct MI355X
 * (gfx950): the C ABI of libfa.so.
 *
 * The library computes exact softmax attention (FlashAttention; tensortonic
 * "FlashAttention" sections 3-7, ai-engineering wiki "Trick: Numerical
 * Stability with Softmax") without ever writing the N x N score or weight
 * matrix to device memory:
 *
 *     O_i = sum_j softmax_j(scale * <q_i, k_j>) v_j      over allowed keys j
 *     L_i = m_i + ln(l_i)                                (row log-sum-exp)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Element types: q, k, v, o, dout, dq, dk, dv are bfloat16 (raw 16-bit
 *    storage, round-to-nearest-even on output) -- or IEEE fp16 for the *_f16
 *    variants at the end; lse is float32.  Arithmetic is 16-bit x 16-bit
 *    products with float32 accumulation.
 *  - Dense layout: [B, H, N, D] row-major, contiguous (tensortonic section 9:
 *    [batch, heads, tokens, head_width]); lse is [B, H, N].  Q, K and V have
 *    the same length N, except in fa_fwd_qk and fa_fwd_splitkv.
 *  - Causal masking (causal = 1) lets query i read keys j <= i (a token reads
 *    itself and the past, never the future: tensortonic section 1).
 *  - softmax_scale multiplies the float32 dot product q_i . k_j before the
 *    softmax (tensortonic section 6 divides by sqrt(head width); pass
 *    1/sqrt(D) for that).  It must be finite and > 0.
 *  - Inputs must be finite: every element of q, k, v (and of o, lse and dout
 *    passed to a backward entry) must be a finite number, and the scaled
 *    scores must stay within float32 range.  The forward kernels are compiled
 *    on that assumption (their maxima skip NaN handling), so a NaN or
 *    infinite input yields unspecified output: it is not guaranteed to
 *    propagate as NaN.  Masked positions use -infinity internally, never
 *    NaN, and rows that read no key produce O = 0 and L = -infinity.
 *  - L is in natural-log units of the scaled scores: L_i = ln sum_j
 *    exp(scale * q_i . k_j) over the allowed keys (tensortonic section 7).
 *  - Supported head widths: D = 64 and D = 128.
 *  - Pointers are device pointers owned by the caller, 16-byte aligned.  The
 *    library never allocates, frees or keeps them after the call returns.
 *  - Every call is asynchronous on `stream` (0 = the null stream) and never
 *    synchronises; results are valid once the caller has synchronised the
 *    stream.  Calls on different streams touching disjoint outputs may run
 *    concurrently.
 *  - Errors: every argument check completes before any HIP call, so a
 *    rejected call has no side effect.  After validation the only error is
 *    FA_ERR_LAUNCH (the launch itself failed).  Faults inside a kernel surface
 *    at the caller's next synchronisation, as for any HIP kernel.
 *  - Per (batch, head) slice of N rows, (N + 256) * D * 2 bytes must stay
 *    below 2 GiB (the kernels address one slice with 32-bit offsets, and may
 *    address up to one tile past its end; 256 rows of headroom cover that):
 *    N <= 8388351 at D = 128, 16776959 at D = 64.  Larger slices return
 *    FA_ERR_TOO_LARGE.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same definition as the HIP runtime's, so this header needs no HIP include. */
typedef struct ihipStream_t* hipStream_t;

enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL = 1,        /* a required pointer is NULL                     */
    FA_ERR_SHAPE = 2,       /* B, H, N, nseq, total or max_seqlen out of range */
    FA_ERR_UNSUPPORTED = 3, /* D not in {64, 128}, or causal not in {0, 1}     */
    FA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                */
    FA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required         */
    FA_ERR_LAUNCH = 6,      /* a kernel launch failed (HIP error)              */
    FA_ERR_ARG = 7,         /* softmax_scale not finite or not > 0, a negative
                               num_splits, or dropout_p outside [0, 1)        */
    FA_ERR_TOO_LARGE = 8,   /* a (batch, head) slice exceeds 2 GiB             */
    FA_ERR_SCRATCH = 9      /* fa_bwd_noalloc: B * H * N above its static
                               scratch (2^21 query rows)                      */
};

/*
 * Forward pass, dense batch.
 *
 * Computes O = softmax(scale * Q K^T (masked)) V and the row log-sum-exp L
 * with the query-first tiled schedule of tensortonic section 6: each work
 * unit keeps one query tile on chip, streams the key/value tiles past it,
 * keeps a running maximum m, denominator l and unnormalised accumulator u per
 * query row (section 5), rescales by exp(m_old - m_new) when the maximum
 * grows, and writes O = u / l and L = m + ln l once at the end.  Under causal
 * masking, key tiles wholly in the future are skipped and the element mask is
 * applied only on tiles that cross the diagonal (section 6).
 *
 *   q, k, v   in   bf16 [B, H, N, D]
 *   o         out  bf16 [B, H, N, D]   (fully overwritten)
 *   lse       out  fp32 [B, H, N]      (may be NULL when not needed)
 *   B, H, N   >= 1;  D in {64, 128};  causal in {0, 1}
 *
 * Returns FA_OK or an fa_status code.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int D, float softmax_scale, int causal,
           hipStream_t stream);

/*
 * Forward pass with Nq queries against Nk keys (chunked prefill, or queries
 * against a longer key/value sequence).  tensortonic section 9 notes that
 * the square causal mask is not right for every unequal-length layout; here
 * the queries are the LAST Nq positions of the Nk-long sequence, so under the
 * causal mask query i reads keys j <= i + Nk - Nq (the mask aligned
 * bottom-right; Nq = Nk is the square mask of fa_fwd).  When Nq > Nk the
 * first Nq - Nk queries read no key: their O rows are 0 and L is -inf.
 *
 *   q         in   bf16 [B, H, Nq, D]
 *   k, v      in   bf16 [B, H, Nk, D]
 *   o         out  bf16 [B, H, Nq, D]  (fully overwritten)
 *   lse       out  fp32 [B, H, Nq]     (may be NULL)
 *   B, H, Nq, Nk >= 1;  D in {64, 128};  causal in {0, 1}
 *
 * Same schedule, conventions and status codes as fa_fwd.
 */
int fa_fwd_qk(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int Nq, int Nk, int D, float softmax_scale, int causal,
              hipStream_t stream);

/*
 * Bytes of device workspace fa_fwd_splitkv needs for these sizes and this
 * num_splits (0 when it will not split, or when fa_fwd_splitkv would reject
 * the sizes).  It holds each key range's normalised partial O_s and L_s
 * (float32) until the merge, L = ln sum_s exp(L_s) (tensortonic section 5's
 * running rescale applied to whole key ranges).
 */
size_t fa_fwd_splitkv_workspace_size(int B, int H, int Nq, int Nk, int D, int num_splits);

/*
 * Decoding-shaped forward: few queries against a long key/value sequence
 * (tensortonic section 8: a cached generation step has one new query and a
 * long run of past keys and values, a different workload that needs kernels
 * suited to its shape).  The keys of every (batch, head) are split into
 * ranges handled by separate workgroups, so a handful of query rows still
 * fill the GPU; each range yields its normalised partial O_s and L_s, and a
 * second kernel combines them exactly: L = ln sum_s exp(L_s) and
 * O = sum_s exp(L_s - L) O_s (the running-softmax rescale of section 5
 * applied to whole ranges).  The result is that of fa_fwd_qk on the same
 * arguments, up to rounding.
 *
 *   q, k, v, o, lse, B, H, Nq, Nk, D, causal   as for fa_fwd_qk
 *   num_splits  0 = choose automatically; > 0 = that many ranges, at most
 *               one per 64 keys.  With one range no workspace is used.
 *               Nq <= 32 runs a decoding kernel (one workgroup per range and
 *               head, its four waves streaming 32-key blocks; automatic
 *               choice: about 256 workgroups, ranges of at least 512 keys).
 *               Larger Nq runs the forward tiles over each range (automatic
 *               choice: about 512 workgroups, ranges of at least 256 keys).
 *   workspace   device memory of fa_fwd_splitkv_workspace_size(B, H, Nq, Nk,
 *               D, num_splits) bytes (may be NULL when that is 0); contents
 *               on entry ignored, on exit unspecified
 *
 * Returns FA_OK or an fa_status code (FA_ERR_WORKSPACE when the workspace is
 * missing or short).
 */
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   void* workspace, size_t workspace_bytes, int B, int H, int Nq, int Nk,
                   int D, float softmax_scale, int causal, int num_splits,
                   hipStream_t stream);

/*
 * Forward pass over packed variable-length sequences (nexusofnerds
 * "FlashAttention": variable-length packing; padding would otherwise waste
 * work).  nseq sequences are concatenated along the token axis; sequence b
 * owns packed tokens [cu_seqlens[b], cu_seqlens[b+1]).  Each sequence attends
 * only to itself, with causal positions relative to its own start.
 *
 *   q, k, v     in   bf16 [H, total, D]
 *   o           out  bf16 [H, total, D]  (rows of every sequence overwritten)
 *   lse         out  fp32 [H, total]     (may be NULL)
 *   cu_seqlens  in   DEVICE int32 [nseq + 1]: cu[0] = 0, non-decreasing,
 *                    cu[nseq] = total.  Zero-length sequences are allowed.
 *   max_seqlen  host int >= every sequence length (sizes the launch grid so
 *                    no device-to-host copy is needed).  Rows of a sequence
 *                    longer than max_seqlen are not written.
 *   nseq, total, max_seqlen, H >= 1;  D in {64, 128}
 *
 * The offsets cannot be checked on the host; the kernels clamp them to
 * [0, total] so malformed offsets never cause out-of-range accesses (their
 * results are then unspecified).
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o,
                  float* lse, const int32_t* cu_seqlens, int nseq, int total,
                  int max_seqlen, int H, int D, float softmax_scale,
                  int causal, hipStream_t stream);

/*
 * Bytes of device workspace fa_bwd needs for these sizes (0 if fa_bwd would
 * reject the sizes).  tensortonic section 7: the backward pass rebuilds each
 * weight as exp(s_ij - L_i) from the row statistic L saved by the forward
 * pass; the workspace holds that statistic per query row in the form the
 * kernels use, -L_i * log2(e), and the row sum D_i = <dO_i, O_i> of the
 * softmax gradient, as two float32 [B, H, N] regions each padded to 256
 * bytes.
 */
size_t fa_bwd_workspace_size(int B, int H, int N, int D);

/*
 * Backward pass, dense batch (tensortonic section 7): reloads query and key
 * tiles, recomputes each score tile, rebuilds its weights as
 * exp(s_ij - L_i) from the saved row log-sum-exp, and accumulates the
 * gradients of sum(dout * O) with respect to q, k and v; the N x N weights
 * are never stored.  There is no dropout.
 *
 *   q, k, v, o, dout   in   bf16 [B, H, N, D]; o and lse must come from
 *                           fa_fwd on the same q, k, v, scale and causal
 *   lse                in   fp32 [B, H, N]
 *   dq, dk, dv         out  bf16 [B, H, N, D] (fully overwritten)
 *   workspace          scratch device memory of at least
 *                      fa_bwd_workspace_size(B, H, N, D) bytes; contents on
 *                      entry are ignored, on exit unspecified
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const float* lse, const void* dout, void* dq, void* dk, void* dv,
           void* workspace, size_t workspace_bytes, int B, int H, int N, int D,
           float softmax_scale, int causal, hipStream_t stream);

/*
 * Backward pass without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, result and status codes
 * as fa_bwd, minus workspace and workspace_bytes; the call allocates nothing.
 * The workspace lives instead in a static device array of the library, 16 MiB
 * on every GPU the library runs on, held until the process ends: it serves
 * B * H * N <= 2^21 query rows (for example B2 H32 N32768); larger sizes
 * return FA_ERR_SCRATCH before any HIP call.  Every call on one GPU shares
 * that GPU's array (the kernels write every value of it they read before
 * reading it, so nothing carries over from the previous call), so calls
 * that may overlap on one GPU (different streams, or another thread) race
 * and must be serialised by the caller.  The array's device address is
 * looked up on the first call on each device.
 */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                   int H, int N, int D, float softmax_scale, int causal, hipStream_t stream);

/*
 * Backward pass over packed variable-length sequences: the gradients of
 * fa_fwd_varlen, computed as fa_bwd computes them for each sequence on its
 * own (tensortonic section 7 for the recomputation; the causal mask and the
 * sequence bounds are those of fa_fwd_varlen, so no gradient flows between
 * sequences).  There is no dropout.
 *
 *   q, k, v, o, dout   in   bf16 [H, total, D], tokens packed along the token
 *                           axis as for fa_fwd_varlen; o and lse must come
 *                           from fa_fwd_varlen on the same q, k, v,
 *                           cu_seqlens, scale and causal
 *   lse                in   fp32 [H, total]
 *   dq, dk, dv         out  bf16 [H, total, D] (rows of every sequence
 *                           overwritten)
 *   cu_seqlens         in   DEVICE int32 [nseq + 1] with the contract of
 *                           fa_fwd_varlen (clamped to [0, total] in the
 *                           kernels, so malformed offsets never cause
 *                           out-of-range accesses)
 *   max_seqlen         host int >= every sequence length (sizes the grid;
 *                           rows of a longer sequence are not written)
 *   nseq, total, max_seqlen, H >= 1;  D in {64, 128}
 *   workspace          scratch device memory of at least
 *                      fa_bwd_workspace_size(1, H, total, D) bytes (one row
 *                      per packed token and head); contents on entry are
 *                      ignored, on exit unspecified
 *
 * Status codes are those of fa_fwd_varlen and fa_bwd.
 */
int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                  const float* lse, const void* dout, void* dq, void* dk, void* dv,
                  const int32_t* cu_seqlens, int nseq, int total, int max_seqlen,
                  void* workspace, size_t workspace_bytes, int H, int D,
                  float softmax_scale, int causal, hipStream_t stream);

/*
 * Attention dropout (tensortonic section 7: with dropout enabled the
 * backward pass must reproduce the forward pass's drop decisions from saved
 * generator state, never draw a new mask).  After the softmax each weight
 * P_ij is kept with probability 1 - p' and scaled by 1 / (1 - p'), or set to
 * zero; O uses the dropped weights while lse stays the log-sum-exp of all
 * allowed scores.  The decisions are a pure function of (seed, offset, head,
 * query, key): the counter-based generator Philox4x32-10 (Salmon et al.,
 * SC 2011) with counter (key / 4, query / 4, b * H + h, offset mod 2^32) and
 * key seed; byte key % 4 of output word query % 4 is compared with
 * T = min(255, round(256 * dropout_p)) and the weight kept iff it is >= T,
 * so p' = T / 256 (dropout_p is rounded to a multiple of 1/256).  Passing the
 * same seed and offset to fa_bwd_dropout replays the forward's mask; no mask
 * is stored.
 *
 *   dropout_p   in [0, 1); T = 0 (dropout_p < 1/512) is attention without
 *               dropout.  Otherwise FA_ERR_ARG.
 *   seed        64-bit generator key
 *   offset      generator counter offset (low 32 bits used); advance it per
 *               call to draw fresh masks under one seed
 *
 * Other arguments, layouts and status codes are those of fa_fwd and fa_bwd.
 *
 * The packed variants (fa_fwd_varlen_dropout, fa_bwd_varlen_dropout) apply
 * the same rule to each sequence b of head h of a packed batch, with
 * counter (key / 4, query / 4, b * H + h, offset mod 2^32), query and key
 * counted from the sequence start; their other arguments are those of
 * fa_fwd_varlen and fa_bwd_varlen.
 */
int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int H, int N, int D, float softmax_scale, int causal, float dropout_p,
                   uint64_t seed, uint64_t offset, hipStream_t stream);
int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dout, void* dq, void* dk, void* dv,
                   void* workspace, size_t workspace_bytes, int B, int H, int N, int D,
                   float softmax_scale, int causal, float dropout_p, uint64_t seed,
                   uint64_t offset, hipStream_t stream);
int fa_fwd_varlen_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                          const int32_t* cu_seqlens, int nseq, int total, int max_seqlen,
                          int H, int D, float softmax_scale, int causal, float dropout_p,
                          uint64_t seed, uint64_t offset, hipStream_t stream);
int fa_bwd_varlen_dropout(const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* dout, void* dq, void* dk, void* dv,
                          const int32_t* cu_seqlens, int nseq, int total, int max_seqlen,
                          void* workspace, size_t workspace_bytes, int H, int D,
                          float softmax_scale, int causal, float dropout_p, uint64_t seed,
                          uint64_t offset, hipStream_t stream);

/*
 * FP16 variants (nexusofnerds "What is FlashAttention?": the kernels run in
 * mixed precision with BF16 or FP16 inputs).  Each has the contract of the
 * function without the suffix, with every 16-bit tensor (q, k, v, o, dout,
 * dq, dk, dv) in IEEE binary16 instead of bfloat16; the scores, softmax
 * statistics, accumulators, lse and workspaces stay fp32, and the 16-bit
 * results are rounded to nearest-even.  The workspace sizes are those of
 * fa_fwd_splitkv_workspace_size and fa_bwd_workspace_size.
 */
int fa_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse, int B,
               int H, int N, int D, float softmax_scale, int causal, hipStream_t stream);
int fa_bwd_varlen_f16(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      const int32_t* cu_seqlens, int nseq, int total, int max_seqlen,
                      void* workspace, size_t workspace_bytes, int H, int D,
                      float softmax_scale, int causal, hipStream_t stream);
int fa_fwd_qk_f16(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                  int H, int Nq, int Nk, int D, float softmax_scale, int causal,
                  hipStream_t stream);
int fa_fwd_splitkv_f16(const void* q, const void* k, const void* v, void* o, float* lse,
                       void* workspace, size_t workspace_bytes, int B, int H, int Nq,
                       int Nk, int D, float softmax_scale, int causal, int num_splits,
                       hipStream_t stream);
int fa_fwd_varlen_f16(const void* q, const void* k, const void* v, void* o, float* lse,
                      const int32_t* cu_seqlens, int nseq, int total, int max_seqlen,
                      int H, int D, float softmax_scale, int causal, hipStream_t stream);
int fa_bwd_f16(const void* q, const void* k, const void* v, const void* o, const float* lse,
               const void* dout, void* dq, void* dk, void* dv, void* workspace,
               size_t workspace_bytes, int B, int H, int N, int D, float softmax_scale,
               int causal, hipStream_t stream);
int fa_fwd_dropout_f16(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int N, int D, float softmax_scale, int causal,
                       float dropout_p, uint64_t seed, uint64_t offset, hipStream_t stream);
int fa_bwd_dropout_f16(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dout, void* dq, void* dk, void* dv,
                       void* workspace, size_t workspace_bytes, int B, int H, int N, int D,
                       float softmax_scale, int causal, float dropout_p, uint64_t seed,
                       uint64_t offset, hipStream_t stream);
int fa_fwd_varlen_dropout_f16(const void* q, const void* k, const void* v, void* o,
                              float* lse, const int32_t* cu_seqlens, int nseq, int total,
                              int max_seqlen, int H, int D, float softmax_scale, int causal,
                              float dropout_p, uint64_t seed, uint64_t offset,
                              hipStream_t stream);
int fa_bwd_varlen_dropout_f16(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, void* dq, void* dk,
                              void* dv, const int32_t* cu_seqlens, int nseq, int total,
                              int max_seqlen, void* workspace, size_t workspace_bytes, int H,
                              int D, float softmax_scale, int causal, float dropout_p,
                              uint64_t seed, uint64_t offset, hipStream_t stream);

/*
 * Static, human-readable name of a status code (never NULL; "unknown fa
 * status" for a value outside enum fa_status).  A library convention for
 * error reporting, not part of the method the pages describe.
 */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
