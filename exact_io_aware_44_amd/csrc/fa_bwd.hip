// fa_bwd.hip -- backward pass of exact tiled softmax attention for gfx950.
//
// The forward pass saved only O and the row log-sum-exp L (tensortonic
// "FlashAttention" section 7).  Each kernel here reloads query and key tiles,
// recomputes a score tile and rebuilds its weights as P_ij = exp(s_ij - L_i);
// no N x N matrix is stored.  With dP_ij = dO_i . v_j and
// D_i = sum_j P_ij dP_ij = dO_i . O_i, the gradients of sum(dO * O) are
//
//     dS_ij = P_ij (dP_ij - D_i)
//     dV_j  = sum_i P_ij dO_i
//     dK_j  = scale * sum_i dS_ij q_i
//     dQ_i  = scale * sum_j dS_ij k_j
//
// (the chain rule through the softmax; the pages state only the weight
// reconstruction and that each tile contributes to dQ, dK and dV).
//
// Two launches, no atomics, deterministic:
//   1. dq:    one unit per 128-query tile keeps Q and dO in registers and
//             streams key tiles (K, V) through LDS: S^T, P^T, dP^T, dS^T,
//             dQ += dS K.  Each unit first forms D_i = dO_i . O_i from the
//             saved bf16 O and -L_i log2 e for its rows, and also writes
//             them to the workspace.
//   2. dkdv:  one unit per key tile keeps its keys' V (and K) on chip and
//             streams query tiles (Q, dO, -L log2 e, D) through LDS: S, P,
//             dV += P^T dO, dP = dO V^T, dS, dK += dS^T Q.  dkdv64_kernel
//             (64 keys per wave) runs it; the dropout replay uses
//             dkdv_kernel (32 keys per wave), whose registers leave room
//             for the generator.
// Recomputing S and dP in the dq pass costs two extra products out of seven
// but avoids a cross-unit reduction of dQ.
//
// Register layouts follow fa_device.hpp: with the score tile in the
// [query][key] orientation each lane holds one key and 16 queries of a 32x32
// block, which is exactly the B operand of the products contracted over
// queries (dV^T = dO^T P, dK^T = Q^T dS); their A operands (dO^T, Q^T) are
// transpose reads of the row-major LDS tiles.  The dq pass mirrors the
// forward kernel (lane = query).
#include <mutex>
#include <type_traits>

#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

struct BwdParams {
    const bf16* q;
    const bf16* k;
    const bf16* v;
    const bf16* o;
    const float* lse;
    const bf16* dout;
    bf16* dq;
    bf16* dk;
    bf16* dv;
    float* dd;     // [B, H, N]  D_i = dO_i . O_i
    float* nl2;    // [B, H, N]  -L_i * log2(e)
    const int32_t* cu;  // packed sequences: offsets [nseq + 1] (varlen only)
    int H, N;      // N: tokens per sequence (dense) or packed total (varlen)
    int per_head;  // dK/dV units per (batch, head): key tiles, or pairs if causal
    float c;       // scale * log2(e)
    float scale;
    Dropout drop;  // the forward's drop decisions, replayed
};

// Direct global -> LDS load of one dword per lane (lane i writes M0 + 4*i).
__device__ __forceinline__ void load4_lds(Buf b, uint32_t off, void* lds_wave_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(b.r, (FA_LDS void*)lds_wave_base, 4, off, 0,
                                             0, 0);
}
// Rows of the (batch, head) slice a unit works on.  Dense: N rows from
// head * N.  Packed (varlen, [H, total, D], batch = sequence): the rows of
// sequence b = head / H in head h's plane, [cu[b], cu[b+1]) clamped to
// [0, total]; positions, and so the causal mask, count from the sequence
// start and no key outside it is read.
template <bool VARLEN>
__device__ __forceinline__ void slice_rows(const BwdParams& p, int head, int& n,
                                           int64_t& row0) {
    if constexpr (VARLEN) {
        const int b = head / p.H, h = head - b * p.H;
        int s = p.cu[b], e = p.cu[b + 1];
        s = min(max(s, 0), p.N);
        e = min(max(e, s), p.N);
        n = e - s;
        row0 = (int64_t)h * p.N + s;
    } else {
        n = p.N;
        row0 = (int64_t)head * p.N;
    }
}

// s_waitcnt vmcnt(0) lgkmcnt(0): this wave's loads (global and LDS) are done.
__device__ __forceinline__ void wait_vmem_lds() { __builtin_amdgcn_s_waitcnt(0x0070); }

// Writes a wave's 32 rows of a transposed accumulator to rows base ..
// base + 31 of dst, times `scale`.  In the accumulator a lane holds 8-byte
// pieces of one row (lane: row l32, columns 32e + 8(r/4) + 4hi + r%4 of
// acc[e], register r); stored directly, each store instruction would write 32
// rows in 16-byte pieces.  The rows are staged in st (32 x (D + 8) elements,
// this wave's own LDS region; the 16-byte row padding spreads the 8-byte
// writes over the banks) and written back as whole rows, 16 bytes per lane,
// with the non-temporal hint (nothing in the pass reads them again).
template <typename E, int D>
__device__ __forceinline__ void store_rows(bf16* st, const f32x16* acc, float scale, Buf dst,
                                           int base, int lane) {
    constexpr int OSTR = D + 8, CPR = D / 8, RPI = 64 / CPR;
    const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int e = 0; e < D / 32; ++e)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
            *reinterpret_cast<u32x2*>(st + l32 * OSTR + 32 * e + 8 * r4 + 4 * hi) =
                pack4<E>(acc[e][4 * r4] * scale, acc[e][4 * r4 + 1] * scale,
                         acc[e][4 * r4 + 2] * scale, acc[e][4 * r4 + 3] * scale);
    // the wave reads rows other lanes wrote: its writes land first
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int t = 0; t < 32 / RPI; ++t) {
        const int i = RPI * t + lane / CPR, c = lane % CPR;
        const u32x4 w = *reinterpret_cast<const u32x4*>(st + i * OSTR + 8 * c);
        store16_nt(dst, ((uint32_t)(base + i) * D + 8 * c) * 2, w);
    }
    // reads done before the region is written again
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------------------
// dK, dV (dropout replay): unit = (batch, head, 128-key tile); wave w owns
//    keys 32w..32w+31 of the tile.  K and V (the B operands of S and dP)
//    stay in VGPRs, the dK^T, dV^T accumulators in AGPRs, while 64-query
//    stages of Q, dO, -L log2 e and D stream through double-buffered LDS.
// ---------------------------------------------------------------------------
template <int D>
struct KvTile {
    static constexpr int BK = 128;                 // keys per unit
    static constexpr int BQ = 64;                  // queries per streamed stage
    static constexpr int THREADS = 256;
    static constexpr int CPR = D / 8;              // 16-byte chunks per row
    static constexpr int T_ELEMS = BQ * D;         // one Q or dO stage
    static constexpr int LPW = BQ * CPR / 64 / 4;  // 1 KiB loads per wave per tile
    static constexpr int RPL = 64 / CPR;           // rows per 1 KiB load
    static constexpr int DS = D / 16;              // MFMA k-steps across the head width
    static constexpr int DB = D / 32;              // 32-wide blocks of the head width
};

// Q / dO stages are stored with unpadded rows and the 16-byte chunk index of
// row r XORed with qd_swz(r).  Both read patterns are then free of bank
// conflicts (64 banks): a quarter-wave ds_read_b128 of one chunk in 16
// consecutive rows sees 16 distinct XORs, and a half-wave transpose read of 4
// chunks in 4 consecutive rows sees the 4 rows in 4 distinct chunk groups.
template <int D>
__device__ __forceinline__ int qd_swz(int r) {
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3))
                    : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}
template <int D>
__device__ __forceinline__ int qd_off(int r, int chunk) {  // element offset
    return r * D + ((chunk ^ qd_swz<D>(r)) << 3);
}

// acc += A * B on v_mfma_f32_32x32x16_bf16 with acc held in AGPRs (the
// compiler would otherwise keep it in VGPRs, which the dK/dV kernel needs for
// K, V and the score tiles).  Hazards the compiler cannot see through the asm:
//  - a VALU write of a or b needs two wait states before the MFMA reads it:
//    the s_nop 1;
//  - back-to-back accumulation into the same registers is interlocked;
//  - reading acc after the last MFMA needs the wait of mfma_acc_drain.
template <typename E>
__device__ __forceinline__ void mfma_acc(f32x16& acc, bf16x8 a, bf16x8 b) {
    if constexpr (__is_same(E, f16))
        asm("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    else
        asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Wait states between the last MFMA into an accumulator and any read of it
// (a 16-pass MFMA result needs at most 18).
__device__ __forceinline__ void mfma_acc_drain(f32x16& a, f32x16& b) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(a), "+a"(b));
}

template <typename E, int D, bool CAUSAL, bool DROP, bool VARLEN>
__global__ __launch_bounds__(256, 1) void dkdv_kernel(BwdParams p) {
    using T = KvTile<D>;
    // one LDS object per buffer, selected statically, so the compiler can tell
    // the stage being read from the one a DMA is filling
    __shared__ __attribute__((aligned(16))) bf16 q_lds0[T::T_ELEMS];
    __shared__ __attribute__((aligned(16))) bf16 q_lds1[T::T_ELEMS];
    __shared__ __attribute__((aligned(16))) bf16 do_lds0[T::T_ELEMS];
    __shared__ __attribute__((aligned(16))) bf16 do_lds1[T::T_ELEMS];
    __shared__ __attribute__((aligned(16))) float f_lds0[2 * T::BQ];  // -L log2 e, then D
    __shared__ __attribute__((aligned(16))) float f_lds1[2 * T::BQ];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5;
    const int g = lane >> 4, i16 = lane & 15;
    int head, uidx;
    unit_of(blockIdx.x, gridDim.x, p.per_head, head, uidx);
    int n;
    int64_t row0;
    slice_rows<VARLEN>(p, head, n, row0);
    const int nkt = (n + T::BK - 1) / T::BK;
    // key tiles of this unit: under causal masking a heavy one (many queries
    // follow it) and the matching light one, so all units carry equal work
    int kt0, kt1;
    if (!unit_tiles(CAUSAL, false, uidx, nkt, kt0, kt1)) return;

    const uint32_t bytes = (uint32_t)n * D * 2;
    const Buf qb = make_buf(p.q + row0 * D, bytes);
    const Buf kb = make_buf(p.k + row0 * D, bytes);
    const Buf vb = make_buf(p.v + row0 * D, bytes);
    const Buf dob = make_buf(p.dout + row0 * D, bytes);
    const Buf nlb = make_buf(p.nl2 + row0, (uint32_t)n * 4);
    const Buf ddb = make_buf(p.dd + row0, (uint32_t)n * 4);
    const Buf dkb = make_buf(p.dk + row0 * D, bytes);
    const Buf dvb = make_buf(p.dv + row0 * D, bytes);

    // ---- stage movement: wave w issues the 1 KiB loads w*LPW .. w*LPW+LPW-1
    //      of each tile; lane -> LDS slot is fixed, the global chunk it
    //      fetches carries the swizzle ----
    uint32_t qoff[T::LPW];
#pragma unroll
    for (int x = 0; x < T::LPW; ++x) {
        const int L = wave * T::LPW + x;
        const int r = L * T::RPL + lane / T::CPR;
        const int pc = lane % T::CPR;
        qoff[x] = (uint32_t)(r * D + ((pc ^ qd_swz<D>(r)) << 3)) * 2;
    }
    auto load_stage = [&](int q0, bf16* __restrict__ qd, bf16* __restrict__ dod,
                          float* __restrict__ fd) __attribute__((always_inline)) {
#pragma unroll
        for (int x = 0; x < T::LPW; ++x) {
            const int L = wave * T::LPW + x;
            load16_lds(qb, qoff[x] + (uint32_t)q0 * D * 2, qd + 512 * L);
            load16_lds(dob, qoff[x] + (uint32_t)q0 * D * 2, dod + 512 * L);
        }
        if (wave == 0) load4_lds(nlb, (uint32_t)(q0 + lane) * 4, fd);
        if (wave == 1) load4_lds(ddb, (uint32_t)(q0 + lane) * 4, fd + T::BQ);
    };

    bf16x8 kreg[T::DS], vreg[T::DS];
    f32x16 dk[T::DB], dv[T::DB];
    int kw0 = 0, kj = 0;

    // S = Q K^T and dP = dO V^T for the 32-query block b of a stage; lane:
    // key kj, local queries 32b + 8(r/4) + 4hi + r%4 (register r).
    auto scores = [&](const bf16* __restrict__ qs, const bf16* __restrict__ dos, int b,
                      f32x16& s, f32x16& dp) __attribute__((always_inline)) {
        s = f32x16{};
        dp = f32x16{};
#pragma unroll
        for (int ss = 0; ss < T::DS; ++ss) {
            const int off = qd_off<D>(32 * b + l32, 2 * ss + hi);
            s = mfma32<E>(lds_read16(qs + off), kreg[ss], s);
            dp = mfma32<E>(lds_read16(dos + off), vreg[ss], dp);
        }
    };
    // Dropout decisions of one 32-query block for this lane's key: word a
    // holds group a (queries qb0 + 8a + 4hi + x in byte x).  The four lanes
    // of a quad (keys j0 .. j0+3) need the same four generator calls, one per
    // group: lane t makes the call of group t and the quad trades columns.
    auto drop_words = [&](int qb0) __attribute__((always_inline)) {
        const int t = kj & 3;
        const u32x4 mine = dropout_block(p.drop, head, qb0 + 8 * t + 4 * hi, kj);
        // column t ^ d of this lane's call goes to quad lane t ^ d
        return quad_share(t, u32x4{block_column(mine, t), block_column(mine, t ^ 1),
                                   block_column(mine, t ^ 2), block_column(mine, t ^ 3)});
    };
    // P = exp2(S c - L log2 e) and dS = P (dP - D), rounded to bf16 in the
    // B-operand order of the two 16-query k-steps; MASK zeroes the weights
    // of keys after their query (tiles on the causal diagonal only).  Under
    // dropout dw holds the block's decisions as drop_words returns them.
    auto weights_group = [&](const float* __restrict__ fs, int qb0, int b, const f32x16& s,
                             const f32x16& dp, float* pf, float* sf, int a, const u32x4& dw,
                             auto mask_tag) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int tm = kj - qb0 - 4 * hi;  // masked where tm > local query offset
        {
            const f32x4 nl = *reinterpret_cast<const f32x4*>(fs + 32 * b + 8 * a + 4 * hi);
            const f32x4 dd =
                *reinterpret_cast<const f32x4*>(fs + T::BQ + 32 * b + 8 * a + 4 * hi);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int r = 4 * a + x;
                float pv = exp2_fast(__builtin_fmaf(s[r], p.c, nl[x]));
                if (MASK) pv = tm > 8 * a + x ? 0.f : pv;
                if constexpr (DROP) {
                    // dV takes the kept weights P Z, dS = P (dP Z - D)
                    const float z = dropout_keep(dw[a], x, p.drop.thresh)
                                        ? p.drop.inv_keep : 0.f;
                    pf[r] = pv * z;
                    sf[r] = pv * (dp[r] * z - dd[x]);
                } else {
                    pf[r] = pv;
                    sf[r] = pv * (dp[r] - dd[x]);
                }
            }
        }
    };
    auto weights = [&](const float* __restrict__ fs, int qb0, int b, const f32x16& s,
                       const f32x16& dp, bf16x8* pb, bf16x8* sb, auto mask_tag)
                       __attribute__((always_inline)) {
        float pf[16], sf[16];
        u32x4 dw{};
        if constexpr (DROP) dw = drop_words(qb0);
#pragma unroll
        for (int a = 0; a < 4; ++a) weights_group(fs, qb0, b, s, dp, pf, sf, a, dw, mask_tag);
        pb[0] = pack8<E>(pf);
        pb[1] = pack8<E>(pf + 8);
        sb[0] = pack8<E>(sf);
        sb[1] = pack8<E>(sf + 8);
    };
    // dV^T += dO^T P and dK^T += Q^T dS; dO^T and Q^T by transpose reads,
    // their query order matching the B operands'.
    auto accumulate = [&](const bf16* __restrict__ qs, const bf16* __restrict__ dos, int b,
                          const bf16x8* pb, const bf16x8* sb) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < T::DB; ++e)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int rr = 32 * b + 16 * t + 4 * hi + (i16 >> 2);
                const int cc = 4 * e + 2 * (g & 1) + ((i16 & 3) >> 1);
                const int o0 = qd_off<D>(rr, cc) + 4 * (i16 & 1);
                const int o1 = qd_off<D>(rr + 8, cc) + 4 * (i16 & 1);
                const bf16x8 doT = cat(lds_read_tr(dos + o0), lds_read_tr(dos + o1));
                mfma_acc<E>(dv[e], doT, pb[t]);
                const bf16x8 qT = cat(lds_read_tr(qs + o0), lds_read_tr(qs + o1));
                mfma_acc<E>(dk[e], qT, sb[t]);
            }
    };
    using True = std::true_type;
    using False = std::false_type;

    // One 64-query stage.  MASKED: a stage on the causal diagonal of this
    // wave's keys (blocks wholly before the keys are skipped, the rest
    // masked, block by block); otherwise a software-pipelined pass over both
    // blocks (see below).
    auto step = [&](int qt, bool more, const bf16* __restrict__ qs,
                    const bf16* __restrict__ dos, const float* __restrict__ fs,
                    bf16* __restrict__ qn, bf16* __restrict__ don, float* __restrict__ fn,
                    auto mask_tag) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(mask_tag)::value;
        if (more) load_stage((qt + 1) * T::BQ, qn, don, fn);
        const int q0 = qt * T::BQ;
        f32x16 s0, dp0;
        bf16x8 pb0[2], sb0[2];
        if constexpr (!MASKED) {
            // Software pipeline of the stage: every MFMA operand is read from
            // LDS PF MFMAs ahead; block 0's weights run beside block 1's
            // score MFMAs, block 1's weights beside block 0's dV/dK MFMAs.
            constexpr int PF = 6;
            f32x16 s1, dp1;
            bf16x8 pb1[2], sb1[2];
            // phase 1: S and dP of both blocks (i: block i / 2DS, k-step
            // (i % 2DS) / 2, S when even, dP when odd)
            constexpr int NSC = 4 * T::DS;
            auto sc_fetch = [&](int i) {
                const int b = i / (2 * T::DS), ss = (i % (2 * T::DS)) >> 1;
                return lds_read16(((i & 1) ? dos : qs) + qd_off<D>(32 * b + l32, 2 * ss + hi));
            };
            s0 = dp0 = s1 = dp1 = f32x16{};
            bf16x8 op[NSC];
#pragma unroll
            for (int i = 0; i < PF; ++i) op[i] = sc_fetch(i);
#pragma unroll
            for (int i = 0; i < NSC; ++i) {
                if (i + PF < NSC) op[i + PF] = sc_fetch(i + PF);
                const int b = i / (2 * T::DS), ss = (i % (2 * T::DS)) >> 1;
                if (b == 0) {
                    if (i & 1) dp0 = mfma32<E>(op[i], vreg[ss], dp0);
                    else s0 = mfma32<E>(op[i], kreg[ss], s0);
                } else {
                    if (i & 1) dp1 = mfma32<E>(op[i], vreg[ss], dp1);
                    else s1 = mfma32<E>(op[i], kreg[ss], s1);
                }
            }
            weights(fs, q0, 0, s0, dp0, pb0, sb0, False{});
            // phases 2 and 3: dV^T += dO^T P and dK^T += Q^T dS per block
            // (j: d-block j / 4, k-step (j / 2) % 2, dV when even, dK when
            // odd); transpose operands PF ahead
            constexpr int NAC = 4 * T::DB;
            auto ac_fetch = [&](int b, int j) {
                const int e = j >> 2, t = (j >> 1) & 1;
                const int rr = 32 * b + 16 * t + 4 * hi + (i16 >> 2);
                const int cc = 4 * e + 2 * (g & 1) + ((i16 & 3) >> 1);
                const bf16* src = (j & 1) ? qs : dos;
                return cat(lds_read_tr(src + qd_off<D>(rr, cc) + 4 * (i16 & 1)),
                           lds_read_tr(src + qd_off<D>(rr + 8, cc) + 4 * (i16 & 1)));
            };
            float pf1[16], sf1[16];
            u32x4 dw1{};
            if constexpr (DROP) dw1 = drop_words(q0 + 32);
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const bf16x8* pb = b ? pb1 : pb0;
                const bf16x8* sb = b ? sb1 : sb0;
                bf16x8 ao[NAC];
#pragma unroll
                for (int j = 0; j < PF; ++j) ao[j] = ac_fetch(b, j);
#pragma unroll
                for (int j = 0; j < NAC; ++j) {
                    if (j + PF < NAC) ao[j + PF] = ac_fetch(b, j + PF);
                    const int e = j >> 2, t = (j >> 1) & 1;
                    if (j & 1) mfma_acc<E>(dk[e], ao[j], sb[t]);
                    else mfma_acc<E>(dv[e], ao[j], pb[t]);
                    // block 1's weights: its four groups of 4 queries spread
                    // evenly over block 0's MFMAs
                    constexpr int GAP = NAC / 4;
                    if (b == 0 && j % GAP == GAP - 1)
                        weights_group(fs, q0 + 32, 1, s1, dp1, pf1, sf1, j / GAP, dw1, False{});
                }
                if (b == 0) {
                    pb1[0] = pack8<E>(pf1);
                    pb1[1] = pack8<E>(pf1 + 8);
                    sb1[0] = pack8<E>(sf1);
                    sb1[1] = pack8<E>(sf1 + 8);
                }
            }
        } else {
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int qb0 = q0 + 32 * b;
                if (qb0 + 31 < kw0) continue;  // every query precedes our keys
                scores(qs, dos, b, s0, dp0);
                weights(fs, qb0, b, s0, dp0, pb0, sb0, True{});
                accumulate(qs, dos, b, pb0, sb0);
            }
        }
        wait_vmem_lds();  // next stage landed; this stage's reads are done
        barrier_only();
    };
    auto run_stage = [&](int qt, int qt_begin, int nqt, auto mask_tag)
                         __attribute__((always_inline)) {
        const bool more = qt + 1 < nqt;
        const bool odd = (qt - qt_begin) & 1;
        step(qt, more, odd ? q_lds1 : q_lds0, odd ? do_lds1 : do_lds0, odd ? f_lds1 : f_lds0,
             odd ? q_lds0 : q_lds1, odd ? do_lds0 : do_lds1, odd ? f_lds0 : f_lds1, mask_tag);
    };

    for (int rep = 0; rep < 2; ++rep) {
        const int kt = rep == 0 ? kt0 : kt1;
        if (kt < 0) break;
        const int k0u = kt * T::BK;
        kw0 = k0u + 32 * wave;
        kj = kw0 + l32;
#pragma unroll
        for (int s = 0; s < T::DS; ++s) {
            const uint32_t off = ((uint32_t)kj * D + 16 * s + 8 * hi) * 2;
            kreg[s] = __builtin_bit_cast(bf16x8, load16(kb, off));
            vreg[s] = __builtin_bit_cast(bf16x8, load16(vb, off));
        }
#pragma unroll
        for (int e = 0; e < T::DB; ++e) {
            dv[e] = f32x16{};
            dk[e] = f32x16{};
        }
        // under causal masking queries before the key tile see none of it
        const int qt_begin = CAUSAL ? k0u / T::BQ : 0;
        const int nqt = (n + T::BQ - 1) / T::BQ;
        load_stage(qt_begin * T::BQ, q_lds0, do_lds0, f_lds0);
        wait_vmem_lds();
        barrier_only();
        // The first two stages hold the diagonal of every wave's keys (a
        // wave's 32 keys start at most 96 past the tile start); separate
        // loops keep the straight-line interior loop free of the masked
        // variant, and the accumulators in one register assignment.
        int qt = qt_begin;
        if (CAUSAL) {
            const int diag_end = min(nqt, qt_begin + 2);
            for (; qt < diag_end; ++qt) run_stage(qt, qt_begin, nqt, True{});
        }
        // two interior stages per trip, so each reads and fills statically
        // known LDS buffers and its operand addresses are a per-lane offset
        // plus a constant (the stage parity is even here: 0 or 2 diagonal
        // stages ran)
        if (((qt - qt_begin) & 1) == 0) {
            for (; qt + 1 < nqt; qt += 2) {
                step(qt, true, q_lds0, do_lds0, f_lds0, q_lds1, do_lds1, f_lds1, False{});
                step(qt + 1, qt + 2 < nqt, q_lds1, do_lds1, f_lds1, q_lds0, do_lds0, f_lds0,
                     False{});
            }
        }
        for (; qt < nqt; ++qt) run_stage(qt, qt_begin, nqt, False{});
#pragma unroll
        for (int e = 0; e < T::DB; ++e) mfma_acc_drain(dv[e], dk[e]);
        // dV[kj][d] = acc, dK[kj][d] = scale * acc, through a Q/dO stage
        // buffer of this wave's own (all waves are past the last stage's
        // barrier, so none reads them any more)
        static_assert(32 * (D + 8) <= T::T_ELEMS, "a wave's rows fit in one stage buffer");
        bf16* const st = wave == 0 ? q_lds0 : wave == 1 ? q_lds1 : wave == 2 ? do_lds0 : do_lds1;
        store_rows<E, D>(st, dv, 1.f, dvb, kw0, lane);
        store_rows<E, D>(st, dk, p.scale, dkb, kw0, lane);
        // the second key tile's first stage refills these buffers
        if (rep == 0 && kt1 >= 0) barrier_only();
    }
}

// ---------------------------------------------------------------------------
// 2b. dK, dV with 64 keys per wave: unit = (batch, head, 256-key tile), wave
//     w owning keys 64w .. 64w + 63.  Each Q or dO operand read from LDS
//     (rows for S and dP, transpose reads for dV and dK) feeds two MFMAs,
//     one per 32-key block of the wave, where dkdv_kernel's 32 keys per wave
//     use each read once: fewer LDS instructions per MFMA, which is what
//     bounds dkdv_kernel (its stage time is about the sum of its MFMA, LDS
//     and VALU time).  V of the 64 keys stays in VGPRs (64), K in a padded
//     LDS tile loaded once per key tile, and the dK^T and dV^T accumulators
//     fill all 256 AGPRs, so a SIMD holds one wave.
//     A 32-query block runs four phases, each operand requested PF operands
//     ahead: S MFMAs; dP MFMAs with the weights P = exp2(S c - L log2 e)
//     computed beside them; dV MFMAs with dS = P (dP - D) beside them; dK
//     MFMAs.  V is held negated and the dP accumulators start at D, so they
//     end at D - dP and dS is one multiply (and a sign) per element.
// ---------------------------------------------------------------------------
template <int D>
struct Kv64Tile {
    static constexpr int WK = 64;                  // keys per wave
    static constexpr int BK = 4 * WK;              // keys per unit
    static constexpr int BQ = 64;                  // queries per streamed stage
    static constexpr int CPR = D / 8;              // 16-byte chunks per row
    static constexpr int T_ELEMS = BQ * D;         // one Q or dO stage
    static constexpr int LPW = BQ * CPR / 64 / 4;  // 1 KiB loads per wave per stage
    static constexpr int RPL = 64 / CPR;           // rows per 1 KiB load
    static constexpr int DS = D / 16;              // MFMA k-steps across the head width
    static constexpr int DB = D / 32;              // 32-wide blocks of the head width
    // K tile: row pitch padded by one 16-byte chunk, so the rows a
    // quarter-wave reads with ds_read_b128 spread over the banks
    static constexpr int KSTR = D + 8;
    static constexpr int KCH = KSTR / 8;           // chunk slots per padded row
    static constexpr int K_LOADS = WK * KCH / 64;  // 1 KiB loads per wave (own keys)
};

template <typename E, int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(256, 1) void dkdv64_kernel(BwdParams p) {
    using T = Kv64Tile<D>;
    static_assert(T::WK * T::KCH % 64 == 0, "whole 1 KiB loads per wave");
    // One LDS object, so every buffer is the same base plus a constant that
    // fits a ds_read's immediate offset (separate objects would each need
    // their own address registers).  The accesses of each stage go through
    // __restrict__ pointers, which tells the compiler that the stage being
    // read and the one a DMA is filling do not overlap.
    // Layout: the two f buffers (fp32 -L log2 e, then D), the four stage
    // buffers, then the K tile, whose reads take their base from a register
    // (it starts past the 64 KiB an immediate offset reaches).
    constexpr int S_OFF = 2 * (4 * T::BQ);              // two f buffers, in bf16 units
    constexpr int K_OFF = S_OFF + 4 * T::T_ELEMS;
    __shared__ __attribute__((aligned(16))) bf16 smem[K_OFF + T::BK * T::KSTR];
    float* const f_lds0 = reinterpret_cast<float*>(smem);
    float* const f_lds1 = f_lds0 + 2 * T::BQ;
    bf16* const q_lds0 = smem + S_OFF;
    bf16* const q_lds1 = smem + S_OFF + T::T_ELEMS;
    bf16* const do_lds0 = smem + S_OFF + 2 * T::T_ELEMS;
    bf16* const do_lds1 = smem + S_OFF + 3 * T::T_ELEMS;
    bf16* const k_lds = smem + K_OFF;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5;
    const int g = lane >> 4, i16 = lane & 15;
    int head, uidx;
    unit_of(blockIdx.x, gridDim.x, p.per_head, head, uidx);
    int n;
    int64_t row0;
    slice_rows<VARLEN>(p, head, n, row0);
    const int nkt = (n + T::BK - 1) / T::BK;
    int kt0, kt1;
    if (!unit_tiles(CAUSAL, false, uidx, nkt, kt0, kt1)) return;

    const uint32_t bytes = (uint32_t)n * D * 2;
    const Buf qb = make_buf(p.q + row0 * D, bytes);
    const Buf kb = make_buf(p.k + row0 * D, bytes);
    const Buf vb = make_buf(p.v + row0 * D, bytes);
    const Buf dob = make_buf(p.dout + row0 * D, bytes);
    const Buf nlb = make_buf(p.nl2 + row0, (uint32_t)n * 4);
    const Buf ddb = make_buf(p.dd + row0, (uint32_t)n * 4);
    const Buf dkb = make_buf(p.dk + row0 * D, bytes);
    const Buf dvb = make_buf(p.dv + row0 * D, bytes);

    // stage movement as in dkdv_kernel: wave w issues the 1 KiB loads
    // w*LPW .. w*LPW+LPW-1 of each stage; the global chunk a lane fetches
    // carries the swizzle
    uint32_t qoff[T::LPW];
#pragma unroll
    for (int x = 0; x < T::LPW; ++x) {
        const int L = wave * T::LPW + x;
        const int r = L * T::RPL + lane / T::CPR;
        const int pc = lane % T::CPR;
        qoff[x] = (uint32_t)(r * D + ((pc ^ qd_swz<D>(r)) << 3)) * 2;
    }
    auto load_stage = [&](int q0, bf16* __restrict__ qd, bf16* __restrict__ dod,
                          float* __restrict__ fd) __attribute__((always_inline)) {
#pragma unroll
        for (int x = 0; x < T::LPW; ++x) {
            const int L = wave * T::LPW + x;
            load16_lds(qb, qoff[x] + (uint32_t)q0 * D * 2, qd + 512 * L);
            load16_lds(dob, qoff[x] + (uint32_t)q0 * D * 2, dod + 512 * L);
        }
        if (wave == 0) load4_lds(nlb, (uint32_t)(q0 + lane) * 4, fd);
        if (wave == 1) load4_lds(ddb, (uint32_t)(q0 + lane) * 4, fd + T::BQ);
    };

    bf16x8 vreg[2][T::DS];               // [32-key block][k-step]
    f32x16 dk[2][T::DB], dv[2][T::DB];      // [32-key block][32-wide d block]
    int kw0 = 0;

    // Per-lane LDS element offsets, computed once.  The swizzle depends on
    // the row mod 16 only, so query block qb and k-step t of a transpose
    // read add (32 qb + 16 t) * D, a constant the reads take as their
    // immediate offset (with the buffer's place in smem) instead of each
    // combination holding an address register.
    int row_off[T::DS];      // Q / dO rows, k-step ss, query block 0
#pragma unroll
    for (int ss = 0; ss < T::DS; ++ss) row_off[ss] = qd_off<D>(l32, 2 * ss + hi);
    int tr_off[T::DB][2];    // dO^T / Q^T, d-block e, rows +0 / +8, k-step 0
#pragma unroll
    for (int e = 0; e < T::DB; ++e) {
        const int rr = 4 * hi + (i16 >> 2);
        const int cc = 4 * e + 2 * (g & 1) + ((i16 & 3) >> 1);
        tr_off[e][0] = qd_off<D>(rr, cc) + 4 * (i16 & 1);
        tr_off[e][1] = qd_off<D>(rr + 8, cc) + 4 * (i16 & 1);
    }
    // K^T rows of key block 0, k-step 0, as an element offset from smem;
    // hidden from the optimiser so it stays one register (block and k-step
    // are immediates)
    int k_off = K_OFF + (T::WK * wave + l32) * T::KSTR + 8 * hi;
    asm volatile("" : "+v"(k_off));

    // NQB (1 or 2) consecutive 32-query blocks, the first being local block
    // qb0 of the stage (queries qg0 ..), as one stream of steps, so operand
    // requests run ahead across the block boundary.  Step i of a block:
    // operand i in [0, NS) Q rows (S, with the two K^T operands of the
    // step); [NS, 2NS) dO rows (dP); [2NS, 2NS + NA) dO^T (dV); [2NS + NA,
    // NOP) Q^T (dK); each feeds the MFMAs of both key blocks.  MASK: weights
    // of keys after their query are zero (the wave's diagonal stage).
    auto qrun = [&](const bf16* __restrict__ qs, const bf16* __restrict__ dos,
                    const float* __restrict__ fs, int qb0, int qg0, auto nqb_tag,
                    auto mask_tag) __attribute__((always_inline)) {
        constexpr int NQB = decltype(nqb_tag)::value;
        constexpr bool MASK = decltype(mask_tag)::value;
        constexpr int NS = T::DS, NA = 2 * T::DB, NOP = 2 * NS + 2 * NA;
        constexpr int NT = NQB * NOP;  // steps of the stream
        constexpr int PF = 5;          // operand read distance, in steps (10 MFMAs)
        auto fetch = [&](int st) -> bf16x8 {
            const int qb = qb0 + st / NOP, i = st % NOP;
            if (i < 2 * NS) {
                const int ss = i % NS;
                return lds_read16((i < NS ? qs : dos) + 32 * qb * D + row_off[ss]);
            }
            const int j = (i - 2 * NS) % NA;
            const int e = j % T::DB, t = j / T::DB;
            const bf16* src = (i < 2 * NS + NA ? dos : qs) + (32 * qb + 16 * t) * D;
            return cat(lds_read_tr(src + tr_off[e][0]), lds_read_tr(src + tr_off[e][1]));
        };
        // K^T operands of an S step (rows of this wave's keys in the K tile,
        // both key blocks), requested with the step's Q operand
        auto kfetch = [&](int st, bf16x8 (&kk)[2]) {
            const bf16* kr = smem + k_off + 16 * (st % NOP);
            kk[0] = lds_read16(kr);
            kk[1] = lds_read16(kr + 32 * T::KSTR);
        };
        auto is_s = [](int st) { return st % NOP < NS; };
        f32x16 s[2], dp[2];
        bf16x8 pb[2][2], sb[2][2];  // [key block][16-query k-step]
        f32x4 nl{};
        // weights of group a (4 queries) of key block kb of stream block
        // blk, in place in s: P = exp2(S c - L log2 e); keys after their
        // query get zero
        auto p_group = [&](int blk, int kb, int a) __attribute__((always_inline)) {
            if (kb == 0)
                nl = *reinterpret_cast<const f32x4*>(fs + 32 * (qb0 + blk) + 8 * a + 4 * hi);
            // masked: tm > query offset in the block
            const int tm = kw0 + 32 * kb + l32 - (qg0 + 32 * blk) - 4 * hi;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int r = 4 * a + x;
                float pv = exp2_fast(__builtin_fmaf(s[kb][r], p.c, nl[x]));
                if (MASK) pv = tm > 8 * a + x ? 0.f : pv;
                s[kb][r] = pv;
            }
        };
        // dS = P (dP - D) of group a of key block kb, in place in dp, which
        // holds D - dP
        auto ds_group = [&](int kb, int a) __attribute__((always_inline)) {
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int r = 4 * a + x;
                dp[kb][r] = -(s[kb][r] * dp[kb][r]);
            }
        };
        // D of the queries of stream block blk in the accumulator layout
        // (register 4a + x: query 8a + 4hi + x): the value both dP
        // accumulators start from.  With V negated they accumulate D - dP,
        // which saves the subtraction per element.
        auto dinit = [&](int blk) __attribute__((always_inline)) {
            f32x16 d;
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(fs + T::BQ + 32 * (qb0 + blk) +
                                                                8 * a + 4 * hi);
#pragma unroll
                for (int x = 0; x < 4; ++x) d[4 * a + x] = v[x];
            }
            return d;
        };
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 op[NT], kop[NT][2];
#pragma unroll
        for (int st = 0; st < PF; ++st) {
            op[st] = fetch(st);
            if (is_s(st)) kfetch(st, kop[st]);
        }
        // VALU groups spread over the dP and dV phases (8 groups each)
#pragma clang loop unroll(full)
        for (int st = 0; st < NT; ++st) {
            const int i = st % NOP;
            if (st + PF < NT) {
                op[st + PF] = fetch(st + PF);
                if (is_s(st + PF)) kfetch(st + PF, kop[st + PF]);
            }
            const int blk = st / NOP;
            if (i == 0) s[0] = s[1] = f32x16{};  // a new block
            if (i < NS) {
                s[0] = mfma32<E>(op[st], kop[st][0], s[0]);
                s[1] = mfma32<E>(op[st], kop[st][1], s[1]);
            } else if (i < 2 * NS) {
                const int ss = i - NS;
                if (ss == 0) {
                    const f32x16 d = dinit(blk);
                    dp[0] = mfma32<E>(op[st], vreg[0][ss], d);
                    dp[1] = mfma32<E>(op[st], vreg[1][ss], d);
                } else {
                    dp[0] = mfma32<E>(op[st], vreg[0][ss], dp[0]);
                    dp[1] = mfma32<E>(op[st], vreg[1][ss], dp[1]);
                }
                constexpr int PER = 8 / NS;  // groups per step
#pragma unroll
                for (int k = 0; k < PER; ++k) {
                    const int gi = ss * PER + k;  // a-major: (a, kb)
                    p_group(blk, gi & 1, gi >> 1);
                }
                if (i == 2 * NS - 1) {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        pb[kb][0] = pack8<E>(s[kb], 0);
                        pb[kb][1] = pack8<E>(s[kb], 8);
                    }
                }
            } else if (i < 2 * NS + NA) {
                // k-step t outer, d-block e inner: an accumulator recurs
                // every 2 DB MFMAs
                const int j = i - 2 * NS, e = j % T::DB, t = j / T::DB;
                mfma_acc<E>(dv[0][e], op[st], pb[0][t]);
                mfma_acc<E>(dv[1][e], op[st], pb[1][t]);
                constexpr int PER = 8 / NA;
#pragma unroll
                for (int k = 0; k < PER; ++k) {
                    const int gi = j * PER + k;
                    ds_group(gi & 1, gi >> 1);
                }
                if (i == 2 * NS + NA - 1) {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        sb[kb][0] = pack8<E>(dp[kb], 0);
                        sb[kb][1] = pack8<E>(dp[kb], 8);
                    }
                }
            } else {
                const int j = i - 2 * NS - NA, e = j % T::DB, t = j / T::DB;
                mfma_acc<E>(dk[0][e], op[st], sb[0][t]);
                mfma_acc<E>(dk[1][e], op[st], sb[1][t]);
            }
            // keep this order: the operand reads PF steps ahead, the step's
            // two MFMAs, then its share of the VALU work
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    using True = std::true_type;
    using False = std::false_type;

    // One 64-query stage.  DIAG: one of the unit's first four stages, where
    // a wave's 64 keys may follow some or all of the stage's queries (blocks
    // wholly before the keys are skipped, the others masked: past the
    // wave's diagonal the mask keeps every weight).
    auto stage = [&](int qt, int qt_next, const bf16* __restrict__ qs,
                     const bf16* __restrict__ dos, const float* __restrict__ fs,
                     bf16* __restrict__ qn, bf16* __restrict__ don, float* __restrict__ fn,
                     auto diag_tag) __attribute__((always_inline)) {
        constexpr bool DIAG = decltype(diag_tag)::value;
        if (qt_next >= 0) load_stage(qt_next * T::BQ, qn, don, fn);
        const int q0 = qt * T::BQ;
        using One = std::integral_constant<int, 1>;
        using Two = std::integral_constant<int, 2>;
        if (DIAG) {
            // block by block; blocks whose queries all precede our keys are
            // skipped
            if (q0 + 31 >= kw0) qrun(qs, dos, fs, 0, q0, One{}, True{});
            if (q0 + 63 >= kw0) qrun(qs, dos, fs, 1, q0 + 32, One{}, True{});
        } else {
            qrun(qs, dos, fs, 0, q0, Two{}, False{});
        }
        wait_vmem_lds();  // next stage landed; this stage's reads are done
        barrier_only();
    };

    for (int rep = 0; rep < 2; ++rep) {
        const int kt = rep == 0 ? kt0 : kt1;
        if (kt < 0) break;
        const int k0u = kt * T::BK;
        kw0 = k0u + T::WK * wave;
        // the lane index is hidden from the optimiser here, so the per-lane
        // offsets of the loads below are computed per key tile instead of
        // being hoisted out of this loop and held (spilled) across it
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int s = 0; s < T::DS; ++s) {
                const uint32_t off =
                    ((uint32_t)(kw0 + 32 * kb2 + (ln & 31)) * D + 16 * s + 8 * (ln >> 5)) * 2;
                // negated (sign bit of each 16-bit element): see dinit
                vreg[kb2][s] = __builtin_bit_cast(
                    bf16x8, load16(vb, off) ^ u32x4{0x80008000u, 0x80008000u, 0x80008000u,
                                                    0x80008000u});
            }
        // this wave's 64 K rows -> its region of the K tile (pad slots fetch
        // nothing and write zeros); the wait and barrier below cover them
#pragma unroll
        for (int t = 0; t < T::K_LOADS; ++t) {
            const int P = 64 * t + ln, r = P / T::KCH, c = P % T::KCH;
            const uint32_t off = c < T::CPR ? ((uint32_t)(kw0 + r) * D + 8 * c) * 2 : kOutOfRange;
            load16_lds(kb, off, k_lds + T::WK * wave * T::KSTR + 512 * t);
        }
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int e = 0; e < T::DB; ++e) {
                dv[kb2][e] = f32x16{};
                dk[kb2][e] = f32x16{};
            }
        // under causal masking queries before the key tile see none of it
        const int qt_begin = CAUSAL ? k0u / T::BQ : 0;
        const int nqt = (n + T::BQ - 1) / T::BQ;
        // the tile's 256 keys span its first four stages; each wave's
        // diagonal is one of them
        const int ndiag = CAUSAL ? min(nqt - qt_begin, T::BK / T::BQ) : 0;
        // Walk order.  The diagonal stages come first.  The other stages of
        // a unit's first key tile (the one with more queries) then run from
        // the last query stage down, and those of its second tile from the
        // diagonal up, so the units of a head that run together read the
        // same Q/dO stage at the same time: at step i past the diagonal the
        // first tiles are all at stage nqt - 1 - i, and a second tile (its
        // partner's stages done) at the same stage for every pair.
        const bool desc = CAUSAL && rep == 0;
        auto qt_of = [&](int i) {
            return desc && i >= ndiag ? nqt - 1 - (i - ndiag) : qt_begin + i;
        };
        const int ns = nqt - qt_begin;
        auto qt_next = [&](int i) { return i + 1 < ns ? qt_of(i + 1) : -1; };
        load_stage(qt_begin * T::BQ, q_lds0, do_lds0, f_lds0);
        wait_vmem_lds();
        barrier_only();
        int i = 0;
        for (; i < ndiag; ++i) {
            const bool odd = i & 1;
            stage(qt_begin + i, qt_next(i), odd ? q_lds1 : q_lds0, odd ? do_lds1 : do_lds0,
                  odd ? f_lds1 : f_lds0, odd ? q_lds0 : q_lds1, odd ? do_lds0 : do_lds1,
                  odd ? f_lds0 : f_lds1, True{});
        }
        // two stages per trip, so each reads and fills statically known LDS
        // buffers (the parity is even here: 0 or 4 diagonal stages ran)
        for (; i + 1 < ns; i += 2) {
            stage(qt_of(i), qt_next(i), q_lds0, do_lds0, f_lds0, q_lds1, do_lds1, f_lds1,
                  False{});
            stage(qt_of(i + 1), qt_next(i + 1), q_lds1, do_lds1, f_lds1, q_lds0, do_lds0, f_lds0,
                  False{});
        }
        if (i < ns) {
            const bool odd = i & 1;
            stage(qt_of(i), -1, odd ? q_lds1 : q_lds0, odd ? do_lds1 : do_lds0,
                  odd ? f_lds1 : f_lds0, odd ? q_lds0 : q_lds1, odd ? do_lds0 : do_lds1,
                  odd ? f_lds0 : f_lds1, False{});
        }
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int e = 0; e < T::DB; ++e) mfma_acc_drain(dv[kb2][e], dk[kb2][e]);
        // dV[kj][d] = acc, dK[kj][d] = scale * acc, through a stage buffer of
        // this wave's own (every wave is past the last stage's barrier)
        static_assert(32 * (D + 8) <= T::T_ELEMS, "a wave's rows fit in one stage buffer");
        bf16* const st = wave == 0 ? q_lds0 : wave == 1 ? q_lds1 : wave == 2 ? do_lds0 : do_lds1;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
            store_rows<E, D>(st, dv[kb2], 1.f, dvb, kw0 + 32 * kb2, lane);
            store_rows<E, D>(st, dk[kb2], p.scale, dkb, kw0 + 32 * kb2, lane);
        }
        // the second key tile's first stage refills these buffers
        if (rep == 0 && kt1 >= 0) barrier_only();
    }
}

// ---------------------------------------------------------------------------
// dQ: unit = (batch, head, 128-query tile); wave w owns queries
//    32w..32w+31 of the tile and keeps them (Q, dO as B operands) and their
//    dQ^T accumulator in VGPRs while 64-key stages of K and V stream through
//    double-buffered LDS.  Scores are taken transposed, S^T = K Q^T, so each
//    lane holds one query and its L and D are scalars.  Using no AGPRs
//    leaves the kernel the whole 256-register budget of two waves per SIMD
//    as VGPRs (any AGPR use splits that budget in half).  This pass runs
//    first: each unit forms D_i = dO_i . O_i (fp32 sum of exact 16-bit
//    products) and -L_i log2 e for its rows and also writes them to the
//    workspace, where the dK/dV pass reads them.
// ---------------------------------------------------------------------------
template <int D>
struct QTile {
    static constexpr int BR = 128;                 // queries per unit
    static constexpr int BC = 64;                  // keys per streamed stage
    static constexpr int THREADS = 256;
    static constexpr int CPR = D / 8;
    static constexpr int T_ELEMS = BC * D;         // one K or V stage
    static constexpr int LPW = BC * CPR / 64 / 4;  // 1 KiB loads per wave per tile
    static constexpr int RPL = 64 / CPR;
    static constexpr int DS = D / 16;
    static constexpr int DB = D / 32;
};

template <typename E, int D, bool CAUSAL, bool DROP, bool VARLEN>
__global__ __launch_bounds__(256, 2) void dq_kernel(BwdParams p) {
    using T = QTile<D>;
    // one LDS object, so each stage buffer is the same base plus a constant
    // that fits a ds_read's immediate offset
    __shared__ __attribute__((aligned(16))) bf16 smem[4 * T::T_ELEMS];
    bf16* const k_lds0 = smem;
    bf16* const k_lds1 = smem + T::T_ELEMS;
    bf16* const v_lds0 = smem + 2 * T::T_ELEMS;
    bf16* const v_lds1 = smem + 3 * T::T_ELEMS;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5;
    const int g = lane >> 4, i16 = lane & 15;
    int head, uidx;
    unit_of(blockIdx.x, gridDim.x, p.per_head, head, uidx);
    int n;
    int64_t row0;
    slice_rows<VARLEN>(p, head, n, row0);
    const int nqt = (n + T::BR - 1) / T::BR;
    // query tiles of this unit: under causal masking a heavy one (late, many
    // keys) and the matching light one
    int t0, t1;
    if (!unit_tiles(CAUSAL, true, uidx, nqt, t0, t1)) return;

    const uint32_t bytes = (uint32_t)n * D * 2;
    const Buf qb = make_buf(p.q + row0 * D, bytes);
    const Buf kb = make_buf(p.k + row0 * D, bytes);
    const Buf vb = make_buf(p.v + row0 * D, bytes);
    const Buf dob = make_buf(p.dout + row0 * D, bytes);
    const Buf nlb = make_buf(p.nl2 + row0, (uint32_t)n * 4);
    const Buf ddb = make_buf(p.dd + row0, (uint32_t)n * 4);
    const Buf dqb = make_buf(p.dq + row0 * D, bytes);
    const Buf ob = make_buf(p.o + row0 * D, bytes);
    const Buf lb = make_buf(p.lse + row0, (uint32_t)n * 4);

    uint32_t koff[T::LPW];
#pragma unroll
    for (int x = 0; x < T::LPW; ++x) {
        const int L = wave * T::LPW + x;
        const int r = L * T::RPL + lane / T::CPR;
        const int pc = lane % T::CPR;
        koff[x] = (uint32_t)(r * D + ((pc ^ qd_swz<D>(r)) << 3)) * 2;
    }
    auto load_stage = [&](int k0, bf16* __restrict__ kd, bf16* __restrict__ vd)
                          __attribute__((always_inline)) {
#pragma unroll
        for (int x = 0; x < T::LPW; ++x) {
            const int L = wave * T::LPW + x;
            load16_lds(kb, koff[x] + (uint32_t)k0 * D * 2, kd + 512 * L);
            load16_lds(vb, koff[x] + (uint32_t)k0 * D * 2, vd + 512 * L);
        }
    };

    // Per-lane LDS element offsets, computed once: the swizzle depends on the
    // row mod 16 only, so a 32-key block b and a k-step t add (32b + 16t) D,
    // a constant the reads take as an immediate.
    int row_off[T::DS];     // K / V rows of key block 0, k-step ss
#pragma unroll
    for (int ss = 0; ss < T::DS; ++ss) row_off[ss] = qd_off<D>(l32, 2 * ss + hi);
    int tr_off[T::DB][2];   // K^T, d-block e, rows +0 / +8, key block 0, k-step 0
#pragma unroll
    for (int e = 0; e < T::DB; ++e) {
        const int rr = 4 * hi + (i16 >> 2);
        const int cc = 4 * e + 2 * (g & 1) + ((i16 & 3) >> 1);
        tr_off[e][0] = qd_off<D>(rr, cc) + 4 * (i16 & 1);
        tr_off[e][1] = qd_off<D>(rr + 8, cc) + 4 * (i16 & 1);
    }
    bf16x8 qreg[T::DS], doreg[T::DS];
    f32x16 acc[T::DB];
    int qi = 0;
    float nl2 = 0.f, dd = 0.f;

    // dS^T = P^T (dP^T - D), P^T = exp2(S^T c - L log2 e), in bf16 B-operand
    // order; MASK zeroes the weights of keys after the lane's query.
    auto weights = [&](int kb0, const f32x16& s, const f32x16& dp, bf16x8* sb,
                       auto mask_tag) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int lim = qi - kb0 - 4 * hi;  // masked where local key offset > lim
        float sf[16];
        // Dropout: a generator call covers 4 queries x 4 keys and this lane
        // needs word qi % 4 of the calls for its 4 key groups (keys kb0 + 8g
        // + 4hi ..).  The four lanes of a quad (queries q .. q+3) need the
        // same four calls: lane t makes the call of group t and the quad
        // trades words, wd[g] being word qi % 4 of group g.
        u32x4 wd{};
        if constexpr (DROP) {
            const int t = qi & 3;
            const u32x4 mine = dropout_block(p.drop, head, qi, kb0 + 8 * t + 4 * hi);
            wd = quad_share(t, xor_permute(mine, t));  // word t ^ d to quad lane t ^ d
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float pv = exp2_fast(__builtin_fmaf(s[r], p.c, nl2));
            if (MASK) pv = 8 * (r >> 2) + (r & 3) > lim ? 0.f : pv;
            if constexpr (DROP) {
                const float z = dropout_keep(wd[r >> 2], r & 3, p.drop.thresh) ? p.drop.inv_keep : 0.f;
                sf[r] = pv * (dp[r] * z - dd);
            } else {
                sf[r] = pv * (dp[r] - dd);
            }
        }
        sb[0] = pack8<E>(sf);
        sb[1] = pack8<E>(sf + 8);
    };
    // One 32-key block b of a stage as a stream of steps in a fixed order:
    // steps 0 .. DS-1 take S^T = K Q^T and dP^T = V dO^T one k-step at a time
    // (lane: query qi, local keys 32b + 8(r/4) + 4hi + r%4 in register r),
    // the weights follow the last of them, and steps DS .. take dQ^T +=
    // K^T dS^T with K^T from transpose reads (k-step outer).  Every operand
    // is requested PF steps ahead, and a scheduling barrier after each step
    // keeps that distance (left to itself the compiler requested most of
    // them one MFMA ahead).  A distance of 3 measured the same and spills.
    auto block = [&](const bf16* __restrict__ ks, const bf16* __restrict__ vs, int b, int kb0,
                     auto mask_tag) __attribute__((always_inline)) {
        constexpr int NS = T::DS, NT = NS + 2 * T::DB;
        constexpr int PF = 2;
        bf16x8 ka[NT], va[NS];
        auto fetch = [&](int st) __attribute__((always_inline)) {
            if (st < NS) {
                const int off = row_off[st] + 32 * b * D;
                ka[st] = lds_read16(ks + off);
                va[st] = lds_read16(vs + off);
            } else {
                const int j = st - NS, e = j % T::DB, t = j / T::DB;
                const int o = (32 * b + 16 * t) * D;
                ka[st] = cat(lds_read_tr(ks + tr_off[e][0] + o), lds_read_tr(ks + tr_off[e][1] + o));
            }
        };
        f32x16 s{}, dp{};
        bf16x8 sb[2];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int st = 0; st < PF; ++st) fetch(st);
#pragma clang loop unroll(full)
        for (int st = 0; st < NT; ++st) {
            if (st + PF < NT) fetch(st + PF);
            if (st < NS) {
                s = mfma32<E>(ka[st], qreg[st], s);
                dp = mfma32<E>(va[st], doreg[st], dp);
            } else {
                const int j = st - NS, e = j % T::DB, t = j / T::DB;
                acc[e] = mfma32<E>(ka[st], sb[t], acc[e]);
            }
            if (st == NS - 1) weights(kb0, s, dp, sb, mask_tag);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    using True = std::true_type;
    using False = std::false_type;

    // One 64-key stage.  MASKED: a stage on the causal diagonal (blocks
    // wholly after this wave's queries skipped, the rest masked).
    auto step = [&](int ks_i, bool more, const bf16* __restrict__ ks,
                    const bf16* __restrict__ vs, bf16* __restrict__ kn,
                    bf16* __restrict__ vn, int qw0, auto mask_tag)
                    __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(mask_tag)::value;
        if (more) load_stage((ks_i + 1) * T::BC, kn, vn);
        const int k0 = ks_i * T::BC;
        if constexpr (!MASKED) {
            // two workgroups per CU interleave one wave's matrix products
            // with the other's exponentials; keeping the blocks apart keeps
            // the registers within that occupancy
            block(ks, vs, 0, k0, False{});
            block(ks, vs, 1, k0 + 32, False{});
        } else {
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int kb0 = k0 + 32 * b;
                if (kb0 > qw0 + 31) continue;  // every key follows our queries
                block(ks, vs, b, kb0, True{});
            }
        }
        wait_vmem_lds();
        barrier_only();
    };
    auto run_stage = [&](int ks_i, int nks, int qw0, auto mask_tag)
                         __attribute__((always_inline)) {
        const bool more = ks_i + 1 < nks;
        const bool odd = ks_i & 1;
        step(ks_i, more, odd ? k_lds1 : k_lds0, odd ? v_lds1 : v_lds0, odd ? k_lds0 : k_lds1,
             odd ? v_lds0 : v_lds1, qw0, mask_tag);
    };

    for (int rep = 0; rep < 2; ++rep) {
        const int qt = rep == 0 ? t0 : t1;
        if (qt < 0) break;
        const int q0 = qt * T::BR;
        const int qw0 = q0 + 32 * wave;
        qi = qw0 + l32;
#pragma unroll
        for (int s = 0; s < T::DS; ++s) {
            const uint32_t off = ((uint32_t)qi * D + 16 * s + 8 * hi) * 2;
            qreg[s] = __builtin_bit_cast(bf16x8, load16(qb, off));
            doreg[s] = __builtin_bit_cast(bf16x8, load16(dob, off));
        }
        // D_i = dO_i . O_i from the saved O (the lane pair qi, qi + 32 holds
        // the two halves of the row) and -L_i log2 e; both also go to the
        // workspace for the dK/dV pass, which runs after this one
        {
            float part = 0.f;
#pragma unroll
            for (int s = 0; s < T::DS; ++s) {
                const uint32_t off = ((uint32_t)qi * D + 16 * s + 8 * hi) * 2;
                const bf16x8 ov = __builtin_bit_cast(bf16x8, load16(ob, off));
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    part = __builtin_fmaf(to_f32<E>(ov[j]), to_f32<E>(doreg[s][j]), part);
            }
            dd = pair_sum(part);
            nl2 = -loadf(lb, (uint32_t)qi * 4) * kLog2e;
            if (hi == 0) {
                store4(ddb, (uint32_t)qi * 4, __builtin_bit_cast(uint32_t, dd));
                store4(nlb, (uint32_t)qi * 4, __builtin_bit_cast(uint32_t, nl2));
            }
        }
#pragma unroll
        for (int e = 0; e < T::DB; ++e) acc[e] = f32x16{};

        // key stages: causal units stop at the tile's last query; the last
        // two stages (keys q0 .. q0+127) are the diagonal
        const int kend = CAUSAL ? min(n, q0 + T::BR) : n;
        const int nks = (kend + T::BC - 1) / T::BC;
        const int n_plain = CAUSAL ? max(0, min(nks, q0 / T::BC)) : nks;
        load_stage(0, k_lds0, v_lds0);
        wait_vmem_lds();
        barrier_only();
        int ks_i = 0;
        // two plain stages per trip, so each reads and fills statically
        // known buffers
        for (; ks_i + 1 < n_plain; ks_i += 2) {
            step(ks_i, true, k_lds0, v_lds0, k_lds1, v_lds1, qw0, False{});
            step(ks_i + 1, ks_i + 2 < nks, k_lds1, v_lds1, k_lds0, v_lds0, qw0, False{});
        }
        for (; ks_i < n_plain; ++ks_i) run_stage(ks_i, nks, qw0, False{});
        if (CAUSAL)
            for (; ks_i < nks; ++ks_i) run_stage(ks_i, nks, qw0, True{});

        // dQ[qi][d] = scale * acc, through a K/V stage buffer of this
        // wave's own (all waves are past the last stage's barrier)
        static_assert(32 * (D + 8) <= T::T_ELEMS, "a wave's rows fit in one stage buffer");
        bf16* const st = wave == 0 ? k_lds0 : wave == 1 ? k_lds1 : wave == 2 ? v_lds0 : v_lds1;
        store_rows<E, D>(st, acc, p.scale, dqb, qw0, lane);
        // the second query tile's first stage refills these buffers
        if (rep == 0 && t1 >= 0) barrier_only();
    }
}

template <typename E, int D, bool CAUSAL, bool DROP, bool VARLEN = false>
hipError_t run_bwd(const BwdArgs& a, hipStream_t stream) {
    BwdParams p;
    p.q = static_cast<const bf16*>(a.q);
    p.k = static_cast<const bf16*>(a.k);
    p.v = static_cast<const bf16*>(a.v);
    p.o = static_cast<const bf16*>(a.o);
    p.lse = a.lse;
    p.dout = static_cast<const bf16*>(a.dout);
    p.dq = static_cast<bf16*>(a.dq);
    p.dk = static_cast<bf16*>(a.dk);
    p.dv = static_cast<bf16*>(a.dv);
    // rows of [B, H, N] (dense) or of [H, total] (varlen: N = total)
    const int64_t rows = VARLEN ? (int64_t)a.H * a.N : (int64_t)a.B * a.H * a.N;
    p.dd = a.ws;
    p.nl2 = a.ws + ((rows + 63) & ~(int64_t)63);  // second region, 256-byte aligned
    p.cu = a.cu;
    p.H = a.H;
    p.N = a.N;
    p.c = (float)((double)a.scale * 1.4426950408889634);
    p.scale = a.scale;
    p.drop = a.drop;

    // units per (sequence, head) come from the longest sequence; units past
    // a shorter sequence's tiles return at once
    const int nmax = VARLEN ? a.max_seqlen : a.N;
    // the dQ pass: per_head query tiles (pairs under causal masking)
    const int nqt = (nmax + QTile<D>::BR - 1) / QTile<D>::BR;
    p.per_head = CAUSAL ? (nqt + 1) / 2 : nqt;
    const int64_t qunits = (int64_t)p.per_head * a.H * a.B;
    hipLaunchKernelGGL((dq_kernel<E, D, CAUSAL, DROP, VARLEN>), dim3((unsigned)qunits),
                       dim3(256), 0, stream, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;

    if constexpr (DROP) {  // the dropout replay keeps 32 keys per wave
        const int nkt = (nmax + KvTile<D>::BK - 1) / KvTile<D>::BK;
        p.per_head = CAUSAL ? (nkt + 1) / 2 : nkt;
        const int64_t units = (int64_t)p.per_head * a.H * a.B;
        hipLaunchKernelGGL((dkdv_kernel<E, D, CAUSAL, DROP, VARLEN>), dim3((unsigned)units),
                           dim3(256), 0, stream, p);
    } else {
        const int nkt = (nmax + Kv64Tile<D>::BK - 1) / Kv64Tile<D>::BK;
        p.per_head = CAUSAL ? (nkt + 1) / 2 : nkt;
        const int64_t units = (int64_t)p.per_head * a.H * a.B;
        hipLaunchKernelGGL((dkdv64_kernel<E, D, CAUSAL, VARLEN>), dim3((unsigned)units),
                           dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

template <typename E, bool DROP>
hipError_t run_bwd_d(const BwdArgs& a, hipStream_t stream) {
    if (a.cu) {  // packed sequences
        if (a.D == 64)
            return a.causal ? run_bwd<E, 64, true, DROP, true>(a, stream)
                            : run_bwd<E, 64, false, DROP, true>(a, stream);
        return a.causal ? run_bwd<E, 128, true, DROP, true>(a, stream)
                        : run_bwd<E, 128, false, DROP, true>(a, stream);
    }
    if (a.D == 64)
        return a.causal ? run_bwd<E, 64, true, DROP>(a, stream)
                        : run_bwd<E, 64, false, DROP>(a, stream);
    return a.causal ? run_bwd<E, 128, true, DROP>(a, stream)
                    : run_bwd<E, 128, false, DROP>(a, stream);
}
template <typename E>
hipError_t run_bwd_e(const BwdArgs& a, hipStream_t stream) {
    return a.drop.thresh > 0 ? run_bwd_d<E, true>(a, stream) : run_bwd_d<E, false>(a, stream);
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
    return a.f16 ? run_bwd_e<f16>(a, stream) : run_bwd_e<bf16>(a, stream);
}

// ---- static scratch for the backward entry point that allocates nothing ----
//
// The backward's only scratch memory is its workspace (D_i and -L_i log2 e
// per query row).  fa_bwd_noalloc takes it from this array instead of a
// caller buffer: every GPU the library runs on holds its own copy, at its own
// address, until the process ends.  Host code never passes the array's name
// to a kernel (on the host it is only a stand-in symbol): it looks up the
// device address once per device with hipGetSymbolAddress and uses that.
static __device__ __align__(256) unsigned char scratch[kBwdScratchBytes];

hipError_t bwd_scratch(float** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {  // first call on this device: it is the current one
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = static_cast<float*>(addr[dev]);
    return hipSuccess;
}

}  // namespace fa
