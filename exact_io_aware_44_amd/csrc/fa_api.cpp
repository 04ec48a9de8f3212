// fa_api.cpp -- the C ABI declared in include/fa.h: argument validation
// (completed before any HIP call, so every rejection is side-effect free and
// testable without a GPU), then dispatch to the kernel launchers.
#include "fa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "fa_launch.hpp"

namespace {

constexpr int64_t kMaxSliceBytes = (int64_t)1 << 31;  // 32-bit offsets per slice

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_common(int H, int D, float scale, int causal) {
    if (H < 1) return FA_ERR_SHAPE;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
    if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
    if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_ARG;
    return FA_OK;
}

int check_slice(int64_t tokens, int D) {
    // the kernels also address up to one tile past the end; keep headroom
    return (tokens + 256) * D * 2 < kMaxSliceBytes ? FA_OK : FA_ERR_TOO_LARGE;
}

int validate_fwd(const void* q, const void* k, const void* v, const void* o,
                 const float* lse, int B, int H, int N, int D, float scale,
                 int causal) {
    if (!q || !k || !v || !o) return FA_ERR_NULL;
    if (B < 1 || N < 1) return FA_ERR_SHAPE;
    if (int rc = check_common(H, D, scale, causal)) return rc;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
        (lse && !aligned16(lse)))
        return FA_ERR_ALIGN;
    if (B > 65535 || H > 65535) return FA_ERR_SHAPE;  // grid y / z limits
    return check_slice(N, D);
}

// Two fp32 values per query row (D_i = dO_i . O_i and -L_i log2 e), stored
// as two [B, H, N] regions, each padded to 256 bytes.
size_t workspace_bytes(int B, int H, int N) {
    const size_t rows = (size_t)B * H * N;
    return 2 * ((rows * sizeof(float) + 255) & ~(size_t)255);
}

// Up to this many queries per (batch, head), fa_fwd_splitkv runs the decoding
// kernel (all queries of a head in one wave's lanes).
constexpr int kDecodeMaxQ = 32;

// Key-range splits for fa_fwd_splitkv: the requested count (0 = automatic:
// for the decoding kernel about 256 workgroups, one per CU, each range at
// least 512 keys; otherwise about 512 workgroups, two per CU, each range at
// least 256 keys; more ranges only add merge traffic and shorter streams),
// clamped to one 64-key tile per range, then rounded so every range but the
// last holds a whole number of tiles and none is empty.
struct Splits {
    int count;
    int chunk;  // keys per range
};
// All arithmetic is in int64: the sizes come straight from the caller.
Splits pick_splits(int B, int H, int Nq, int Nk, int requested) {
    const int64_t nq = Nq, nk = Nk;
    const int64_t units = (int64_t)B * H * ((nq + 127) / 128);
    int64_t s = requested;
    if (s == 0 && nq <= kDecodeMaxQ) {
        // decoding kernel: one workgroup per CU (256 of them), each range at
        // least 512 keys so every wave streams several blocks
        s = std::min<int64_t>(128, (256 + units - 1) / units);
        s = std::min<int64_t>(s, std::max<int64_t>(1, (nk + 511) / 512));
    } else if (s == 0) {
        s = std::min<int64_t>(128, (512 + units - 1) / units);
        s = std::min<int64_t>(s, std::max<int64_t>(1, (nk + 255) / 256));
    }
    s = std::max<int64_t>(1, std::min<int64_t>(s, (nk + 63) / 64));
    const int64_t chunk = ((nk + s - 1) / s + 63) / 64 * 64;
    return Splits{(int)((nk + chunk - 1) / chunk), (int)chunk};
}
// Partial O then partial L, fp32, each region padded to 256 bytes.  The
// sizes are already validated (B, H <= 65535, one slice below 2 GiB, at most
// one range per 64 keys), so the products stay far below 2^64.
size_t splitkv_bytes(int B, int H, int Nq, int D, int splits) {
    if (splits <= 1) return 0;
    const size_t rows = (size_t)B * H * Nq * splits;
    return 4 * (((rows * D + 63) & ~(size_t)63) + ((rows + 63) & ~(size_t)63));
}

// ---- the entry points, parameterised by the element type (bf16 / fp16) ----

// Drop threshold T = min(255, round(256 p)) and the kept-weight scale, or an
// error for p outside [0, 1).
int make_dropout(float p, uint64_t seed, uint64_t offset, fa::Dropout& d) {
    if (!std::isfinite(p) || p < 0.f || !(p < 1.f)) return FA_ERR_ARG;
    const double t = std::floor((double)p * 256.0 + 0.5);
    d.thresh = t > 255.0 ? 255u : (uint32_t)t;
    d.inv_keep = (float)(256.0 / (256.0 - d.thresh));
    d.seed_lo = (uint32_t)seed;
    d.seed_hi = (uint32_t)(seed >> 32);
    d.offset = (uint32_t)offset;
    return FA_OK;
}

int fwd_impl(bool f16, const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int N, int D, float softmax_scale, int causal,
             hipStream_t stream, const fa::Dropout* drop = nullptr) {
    if (int rc = validate_fwd(q, k, v, o, lse, B, H, N, D, softmax_scale, causal))
        return rc;
    fa::FwdArgs a{q, k, v, o, lse, nullptr, B, H, N, N, D, softmax_scale, causal != 0, N};
    if (drop) a.drop = *drop;
    a.f16 = f16;
    return fa::launch_fwd(a, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fwd_qk_impl(bool f16, const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int Nq, int Nk, int D, float softmax_scale, int causal,
                hipStream_t stream) {
    if (int rc = validate_fwd(q, k, v, o, lse, B, H, Nq, D, softmax_scale, causal))
        return rc;
    if (Nk < 1) return FA_ERR_SHAPE;
    if (int rc = check_slice(Nk, D)) return rc;
    fa::FwdArgs a{q, k, v, o, lse, nullptr, B, H, Nq, Nq, D, softmax_scale, causal != 0, Nk};
    a.f16 = f16;
    return fa::launch_fwd(a, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fwd_splitkv_impl(bool f16, const void* q, const void* k, const void* v, void* o,
                     float* lse, void* workspace, size_t ws_bytes, int B, int H, int Nq,
                     int Nk, int D, float softmax_scale, int causal, int num_splits,
                     hipStream_t stream) {
    if (int rc = validate_fwd(q, k, v, o, lse, B, H, Nq, D, softmax_scale, causal))
        return rc;
    if (Nk < 1) return FA_ERR_SHAPE;
    if (num_splits < 0) return FA_ERR_ARG;
    if (int rc = check_slice(Nk, D)) return rc;
    if (int rc = check_slice(2 * (int64_t)Nq, D)) return rc;  // fp32 partial rows
    const Splits sp = pick_splits(B, H, Nq, Nk, num_splits);
    fa::FwdArgs a{q, k, v, o, lse, nullptr, B, H, Nq, Nq, D, softmax_scale, causal != 0, Nk};
    if (sp.count > 1) {
        if (!workspace || ws_bytes < splitkv_bytes(B, H, Nq, D, sp.count))
            return FA_ERR_WORKSPACE;
        if (!aligned16(workspace)) return FA_ERR_ALIGN;
        a.splits = sp.count;
        a.chunk = sp.chunk;
        a.part = static_cast<float*>(workspace);
    }
    a.f16 = f16;
    a.decode = Nq <= kDecodeMaxQ;
    return fa::launch_fwd(a, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fwd_varlen_impl(bool f16, const void* q, const void* k, const void* v, void* o,
                    float* lse, const int32_t* cu_seqlens, int nseq, int total,
                    int max_seqlen, int H, int D, float softmax_scale, int causal,
                    hipStream_t stream, const fa::Dropout* drop = nullptr) {
    if (!q || !k || !v || !o || !cu_seqlens) return FA_ERR_NULL;
    if (nseq < 1 || total < 1 || max_seqlen < 1 || nseq > 65535) return FA_ERR_SHAPE;
    if (int rc = check_common(H, D, softmax_scale, causal)) return rc;
    if (H > 65535) return FA_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
        (lse && !aligned16(lse)) || (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u))
        return FA_ERR_ALIGN;
    if (int rc = check_slice(total, D)) return rc;
    if (max_seqlen > total) max_seqlen = total;  // no sequence is longer than total
    fa::FwdArgs a{q, k, v, o, lse, cu_seqlens, nseq, H, total, max_seqlen, D,
                  softmax_scale, causal != 0, total};
    if (drop) a.drop = *drop;
    a.f16 = f16;
    return fa::launch_fwd(a, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int bwd_impl(bool f16, const void* q, const void* k, const void* v, const void* o,
             const float* lse, const void* dout, void* dq, void* dk, void* dv,
             void* workspace, size_t ws_bytes, int B, int H, int N, int D,
             float softmax_scale, int causal, hipStream_t stream,
             const fa::Dropout* drop = nullptr) {
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
    if (B < 1 || N < 1) return FA_ERR_SHAPE;
    if (int rc = check_common(H, D, softmax_scale, causal)) return rc;
    if (B > 65535 || H > 65535) return FA_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
        !aligned16(lse) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) ||
        !aligned16(dv))
        return FA_ERR_ALIGN;
    if (int rc = check_slice(N, D)) return rc;
    if (!workspace || ws_bytes < workspace_bytes(B, H, N)) return FA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA_ERR_ALIGN;
    fa::BwdArgs a{q, k, v, o, lse, dout, dq, dk, dv, static_cast<float*>(workspace),
                  B, H, N, D, softmax_scale, causal != 0};
    if (drop) a.drop = *drop;
    a.f16 = f16;
    return fa::launch_bwd(a, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// fa_bwd without a workspace argument: the workspace lives in the library's
// static device scratch (fa::kBwdScratchBytes per device).
int bwd_noalloc_impl(const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                     int H, int N, int D, float softmax_scale, int causal,
                     hipStream_t stream) {
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
    if (B < 1 || N < 1) return FA_ERR_SHAPE;
    if (int rc = check_common(H, D, softmax_scale, causal)) return rc;
    if (B > 65535 || H > 65535) return FA_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
        !aligned16(lse) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) ||
        !aligned16(dv))
        return FA_ERR_ALIGN;
    if (int rc = check_slice(N, D)) return rc;
    if (workspace_bytes(B, H, N) > fa::kBwdScratchBytes) return FA_ERR_SCRATCH;
    float* ws = nullptr;
    if (fa::bwd_scratch(&ws) != hipSuccess) return FA_ERR_LAUNCH;
    fa::BwdArgs a{q, k, v, o, lse, dout, dq, dk, dv, ws, B, H, N, D, softmax_scale,
                  causal != 0};
    return fa::launch_bwd(a, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int bwd_varlen_impl(bool f16, const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv,
                    const int32_t* cu_seqlens, int nseq, int total, int max_seqlen,
                    void* workspace, size_t ws_bytes, int H, int D, float softmax_scale,
                    int causal, hipStream_t stream, const fa::Dropout* drop = nullptr) {
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !cu_seqlens)
        return FA_ERR_NULL;
    if (nseq < 1 || total < 1 || max_seqlen < 1 || nseq > 65535) return FA_ERR_SHAPE;
    if (int rc = check_common(H, D, softmax_scale, causal)) return rc;
    if (H > 65535) return FA_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
        !aligned16(lse) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) ||
        !aligned16(dv) || (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u))
        return FA_ERR_ALIGN;
    if (int rc = check_slice(total, D)) return rc;
    // the workspace holds one row per packed token of every head
    if (!workspace || ws_bytes < workspace_bytes(1, H, total)) return FA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA_ERR_ALIGN;
    if (max_seqlen > total) max_seqlen = total;  // no sequence is longer than total
    fa::BwdArgs a{q, k, v, o, lse, dout, dq, dk, dv, static_cast<float*>(workspace),
                  nseq, H, total, D, softmax_scale, causal != 0};
    a.f16 = f16;
    a.cu = cu_seqlens;
    a.max_seqlen = max_seqlen;
    if (drop) a.drop = *drop;
    return fa::launch_bwd(a, stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {


const char* fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "FA_OK";
        case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
        case FA_ERR_SHAPE: return "FA_ERR_SHAPE: a size argument is out of range";
        case FA_ERR_UNSUPPORTED:
            return "FA_ERR_UNSUPPORTED: head width must be 64 or 128 and causal 0 or 1";
        case FA_ERR_ALIGN: return "FA_ERR_ALIGN: pointers must be 16-byte aligned";
        case FA_ERR_WORKSPACE:
            return "FA_ERR_WORKSPACE: workspace is NULL or smaller than the size its "
                   "*_workspace_size function returns";
        case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: a kernel launch failed";
        case FA_ERR_ARG:
            return "FA_ERR_ARG: softmax_scale must be finite and > 0, num_splits >= 0, "
                   "dropout_p in [0, 1)";
        case FA_ERR_TOO_LARGE:
            return "FA_ERR_TOO_LARGE: one (batch, head) slice exceeds 2 GiB";
        case FA_ERR_SCRATCH:
            return "FA_ERR_SCRATCH: B * H * N exceeds the 2^21 query rows of "
                   "fa_bwd_noalloc's static scratch";
        default: return "unknown fa status";
    }
}

size_t fa_fwd_splitkv_workspace_size(int B, int H, int Nq, int Nk, int D, int num_splits) {
    // sizes fa_fwd_splitkv would reject need no workspace
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || num_splits < 0 || (D != 64 && D != 128) ||
        B > 65535 || H > 65535 || check_slice(Nk, D) || check_slice(2 * (int64_t)Nq, D))
        return 0;
    return splitkv_bytes(B, H, Nq, D, pick_splits(B, H, Nq, Nk, num_splits).count);
}

size_t fa_bwd_workspace_size(int B, int H, int N, int D) {
    // sizes fa_bwd would reject need no workspace
    if (B < 1 || H < 1 || N < 1 || (D != 64 && D != 128) || B > 65535 || H > 65535 ||
        check_slice(N, D))
        return 0;
    return workspace_bytes(B, H, N);
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
           int N, int D, float softmax_scale, int causal, hipStream_t stream) {
    return fwd_impl(false, q, k, v, o, lse, B, H, N, D, softmax_scale, causal, stream);
}
int fa_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse, int B,
               int H, int N, int D, float softmax_scale, int causal, hipStream_t stream) {
    return fwd_impl(true, q, k, v, o, lse, B, H, N, D, softmax_scale, causal, stream);
}

int fa_fwd_qk(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
              int Nq, int Nk, int D, float softmax_scale, int causal, hipStream_t stream) {
    return fwd_qk_impl(false, q, k, v, o, lse, B, H, Nq, Nk, D, softmax_scale, causal,
                       stream);
}
int fa_fwd_qk_f16(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                  int H, int Nq, int Nk, int D, float softmax_scale, int causal,
                  hipStream_t stream) {
    return fwd_qk_impl(true, q, k, v, o, lse, B, H, Nq, Nk, D, softmax_scale, causal,
                       stream);
}

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   void* workspace, size_t ws_bytes, int B, int H, int Nq, int Nk, int D,
                   float softmax_scale, int causal, int num_splits, hipStream_t stream) {
    return fwd_splitkv_impl(false, q, k, v, o, lse, workspace, ws_bytes, B, H, Nq, Nk, D,
                            softmax_scale, causal, num_splits, stream);
}
int fa_fwd_splitkv_f16(const void* q, const void* k, const void* v, void* o, float* lse,
                       void* workspace, size_t ws_bytes, int B, int H, int Nq, int Nk,
                       int D, float softmax_scale, int causal, int num_splits,
                       hipStream_t stream) {
    return fwd_splitkv_impl(true, q, k, v, o, lse, workspace, ws_bytes, B, H, Nq, Nk, D,
                            softmax_scale, causal, num_splits, stream);
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int32_t* cu_seqlens, int nseq, int total, int max_seqlen, int H,
                  int D, float softmax_scale, int causal, hipStream_t stream) {
    return fwd_varlen_impl(false, q, k, v, o, lse, cu_seqlens, nseq, total, max_seqlen, H,
                           D, softmax_scale, causal, stream);
}
int fa_fwd_varlen_f16(const void* q, const void* k, const void* v, void* o, float* lse,
                      const int32_t* cu_seqlens, int nseq, int total, int max_seqlen, int H,
                      int D, float softmax_scale, int causal, hipStream_t stream) {
    return fwd_varlen_impl(true, q, k, v, o, lse, cu_seqlens, nseq, total, max_seqlen, H,
                           D, softmax_scale, causal, stream);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, void* workspace,
           size_t ws_bytes, int B, int H, int N, int D, float softmax_scale, int causal,
           hipStream_t stream) {
    return bwd_impl(false, q, k, v, o, lse, dout, dq, dk, dv, workspace, ws_bytes, B, H, N,
                    D, softmax_scale, causal, stream);
}
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
                   int H, int N, int D, float softmax_scale, int causal, hipStream_t stream) {
    return bwd_noalloc_impl(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, D, softmax_scale,
                            causal, stream);
}
int fa_bwd_f16(const void* q, const void* k, const void* v, const void* o, const float* lse,
               const void* dout, void* dq, void* dk, void* dv, void* workspace,
               size_t ws_bytes, int B, int H, int N, int D, float softmax_scale, int causal,
               hipStream_t stream) {
    return bwd_impl(true, q, k, v, o, lse, dout, dq, dk, dv, workspace, ws_bytes, B, H, N,
                    D, softmax_scale, causal, stream);
}

int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                  const float* lse, const void* dout, void* dq, void* dk, void* dv,
                  const int32_t* cu_seqlens, int nseq, int total, int max_seqlen,
                  void* workspace, size_t ws_bytes, int H, int D, float softmax_scale,
                  int causal, hipStream_t stream) {
    return bwd_varlen_impl(false, q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens, nseq, total,
                           max_seqlen, workspace, ws_bytes, H, D, softmax_scale, causal,
                           stream);
}
int fa_bwd_varlen_f16(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      const int32_t* cu_seqlens, int nseq, int total, int max_seqlen,
                      void* workspace, size_t ws_bytes, int H, int D, float softmax_scale,
                      int causal, hipStream_t stream) {
    return bwd_varlen_impl(true, q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens, nseq, total,
                           max_seqlen, workspace, ws_bytes, H, D, softmax_scale, causal,
                           stream);
}

#define FA_DROPOUT_ENTRIES(SUFFIX, F16)                                                   \
    int fa_fwd_dropout##SUFFIX(const void* q, const void* k, const void* v, void* o,      \
                               float* lse, int B, int H, int N, int D,                    \
                               float softmax_scale, int causal, float dropout_p,          \
                               uint64_t seed, uint64_t offset, hipStream_t stream) {      \
        fa::Dropout d{};                                                                   \
        if (int rc = make_dropout(dropout_p, seed, offset, d)) return rc;                  \
        return fwd_impl(F16, q, k, v, o, lse, B, H, N, D, softmax_scale, causal, stream,  \
                        &d);                                                               \
    }                                                                                      \
    int fa_bwd_dropout##SUFFIX(const void* q, const void* k, const void* v, const void* o, \
                               const float* lse, const void* dout, void* dq, void* dk,    \
                               void* dv, void* workspace, size_t ws_bytes, int B, int H,  \
                               int N, int D, float softmax_scale, int causal,             \
                               float dropout_p, uint64_t seed, uint64_t offset,           \
                               hipStream_t stream) {                                       \
        fa::Dropout d{};                                                                   \
        if (int rc = make_dropout(dropout_p, seed, offset, d)) return rc;                  \
        return bwd_impl(F16, q, k, v, o, lse, dout, dq, dk, dv, workspace, ws_bytes, B, H,  \
                        N, D, softmax_scale, causal, stream, &d);                          \
    }                                                                                      \
    int fa_fwd_varlen_dropout##SUFFIX(                                                     \
        const void* q, const void* k, const void* v, void* o, float* lse,                  \
        const int32_t* cu_seqlens, int nseq, int total, int max_seqlen, int H, int D,      \
        float softmax_scale, int causal, float dropout_p, uint64_t seed, uint64_t offset,  \
        hipStream_t stream) {                                                              \
        fa::Dropout d{};                                                                   \
        if (int rc = make_dropout(dropout_p, seed, offset, d)) return rc;                  \
        return fwd_varlen_impl(F16, q, k, v, o, lse, cu_seqlens, nseq, total, max_seqlen,  \
                               H, D, softmax_scale, causal, stream, &d);                   \
    }                                                                                      \
    int fa_bwd_varlen_dropout##SUFFIX(                                                     \
        const void* q, const void* k, const void* v, const void* o, const float* lse,      \
        const void* dout, void* dq, void* dk, void* dv, const int32_t* cu_seqlens,         \
        int nseq, int total, int max_seqlen, void* workspace, size_t ws_bytes, int H,      \
        int D, float softmax_scale, int causal, float dropout_p, uint64_t seed,            \
        uint64_t offset, hipStream_t stream) {                                             \
        fa::Dropout d{};                                                                   \
        if (int rc = make_dropout(dropout_p, seed, offset, d)) return rc;                  \
        return bwd_varlen_impl(F16, q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens, nseq,   \
                               total, max_seqlen, workspace, ws_bytes, H, D,               \
                               softmax_scale, causal, stream, &d);                         \
    }
FA_DROPOUT_ENTRIES(, false)
FA_DROPOUT_ENTRIES(_f16, true)
#undef FA_DROPOUT_ENTRIES

}  // extern "C"
