// fa_fwd.hip -- forward pass of exact tiled softmax attention for gfx950.
//
// Query-first schedule (tensortonic "FlashAttention" section 6): one work
// unit owns a tile of BR query rows, keeps it in registers, and streams the
// key/value tiles of its (batch, head) past it through LDS.  Per query row it
// keeps the running maximum m, denominator l and unnormalised accumulator u
// (section 5); when a tile raises the maximum the old sums are rescaled by
// exp(m_old - m_new) before the tile's contribution is added.  O = u / l and
// L = m + ln l are written once, at the end.  Nothing of size N x N is ever
// stored.
//
// Mapping to CDNA4:
//  - 256 threads = 4 wave64s, each owning 32 query rows (BR = 128).
//  - Scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16
//    with K read from LDS and Q held in registers.  In that orientation each
//    lane holds ONE query row (lane % 32) and 16 of the 32 keys of a block,
//    so the row maximum and sum are in-lane reductions plus one exchange with
//    lane ^ 32, and the rescale factor is a per-lane scalar.
//  - The same registers, rounded to bf16, are already the B operand of
//    O^T += V^T P^T (the key order inside an MFMA k-step is a free
//    permutation, matched on the V side).  V stays row-major in LDS and is
//    read with ds_read_b64_tr_b16, which delivers it column-major.
//  - Exponentials use exp2 with scale*log2(e) folded into one FMA per score;
//    the running maximum moves lazily (see kLazyRescale), so the accumulator
//    rescale is skipped on almost every tile.
//  - K and V tiles have separate LDS double buffers with K one tile ahead:
//    while the softmax of tile j runs on the VALU, S for tile j+1 is already
//    computable on the MFMA unit from K_{j+1} in LDS.  Global loads for
//    K_{j+2} and V_{j+1} are issued at the top of iteration j and written to
//    the buffers no wave reads during it, so one barrier per tile suffices.
//  - Causal: key tiles wholly after the unit's last row are never loaded; a
//    wave skips tiles wholly after its own rows; the element mask runs only on
//    tiles crossing the diagonal (or the ragged end of the sequence).
//  - A 1-D grid is remapped so that each XCD owns whole heads (their K/V
//    re-reads hit its private L2), heaviest query tile first.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

template <int D>
struct FwdTile {
    static constexpr int BR = 128;       // query rows per work unit
    static constexpr int BC = 64;        // keys per streamed tile
    static constexpr int THREADS = 256;
    static constexpr int CPR = D / 8;    // 16-byte chunks per row
    // K: row pitch padded by one chunk, so the 16 rows a quarter-wave reads
    // with ds_read_b128 land 4 banks apart (conflict-free)
    static constexpr int KSTR = D + 8;
    static constexpr int KCH = KSTR / 8;               // chunks per padded row
    static constexpr int K_LOADS = BC * KCH / 64;      // wave-wide 1 KiB loads
    // V: unpadded rows, chunk index XOR-swizzled (see v_swz) so the transpose
    // reads of four rows x 64 bytes per half-wave hit distinct banks
    static constexpr int V_LOADS = BC * CPR / 64;
    static constexpr int K_ELEMS = BC * KSTR;
    static constexpr int V_ELEMS = BC * D;
    static constexpr int LDS_ELEMS = 2 * K_ELEMS + 2 * V_ELEMS;  // K x2, V x2
    static constexpr int DS = D / 16;    // MFMA k-steps across the head width
    static constexpr int DB = D / 32;    // 32-wide blocks of the output
    static constexpr int RPL = 64 / CPR; // V rows per wave-wide load
};

// XOR applied to the 16-byte chunk index of V row r in LDS.
template <int D>
__device__ __forceinline__ int v_swz(int r) {
    return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

// The running maximum only moves when a tile exceeds it by more than this
// many base-2 units; until then new weights are taken against the stale
// maximum (so they are at most 2^8) and the accumulators need no rescale.
// Every weight and both sums still share one reference point, so O = u / l
// and L = m + ln l are unchanged up to rounding.
constexpr float kLazyRescale = 8.f;

struct FwdParams {
    const bf16* q;
    const bf16* k;
    const bf16* v;
    bf16* o;
    float* lse;
    const int32_t* cu;
    int H;
    int N;     // tokens per sequence (dense) or packed total (varlen)
    int n_qt;  // query tiles per (batch, head) in the grid
    float c;   // softmax_scale * log2(e)
};

// Unit schedule.  Workgroup i of a 1-D grid is dispatched to XCD i % 8; the
// remap below gives each XCD a contiguous range of units, head-major and
// heaviest query tile first, so the K/V re-reads of one head stay in that
// XCD's L2 and the light units of the causal triangle run last.
__device__ __forceinline__ void unit_of(int i, int total, int n_qt, bool causal,
                                        int& head, int& qt) {
    const int L = (total & 7) == 0 ? (i & 7) * (total >> 3) + (i >> 3) : i;
    head = L / n_qt;
    const int r = L - head * n_qt;
    qt = causal ? n_qt - 1 - r : r;
}

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdParams p) {
    using T = FwdTile<D>;
    __shared__ __attribute__((aligned(16))) bf16 lds[T::LDS_ELEMS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int l32 = lane & 31, hi = lane >> 5;
    const int g = lane >> 4, i16 = lane & 15;
    int head, qt;
    unit_of(blockIdx.x, gridDim.x, p.n_qt, CAUSAL, head, qt);
    const int b = head / p.H, h = head - b * p.H;

    int n;
    int64_t row0;
    if constexpr (VARLEN) {
        int s = p.cu[b], e = p.cu[b + 1];
        s = min(max(s, 0), p.N);
        e = min(max(e, s), p.N);
        n = e - s;
        row0 = (int64_t)h * p.N + s;
    } else {
        n = p.N;
        row0 = ((int64_t)b * p.H + h) * p.N;
    }
    const int q0 = qt * T::BR;
    if (q0 >= n) return;  // whole unit past the end of its sequence

    const uint32_t bytes = (uint32_t)n * D * 2;
    const Buf qb = make_buf(p.q + row0 * D, bytes);
    const Buf kb = make_buf(p.k + row0 * D, bytes);
    const Buf vb = make_buf(p.v + row0 * D, bytes);
    const Buf ob = make_buf(p.o + row0 * D, bytes);
    const Buf lb = p.lse ? make_buf(p.lse + row0, (uint32_t)n * 4)
                         : make_buf(nullptr, 0);

    const int qw0 = q0 + 32 * wave;  // first query row of this wave
    const int qi = qw0 + l32;        // query row held by this lane

    // Q as the B operand of S^T = K Q^T: lane holds Q[qi][16s + 8hi + 0..7].
    bf16x8 qreg[T::DS];
#pragma unroll
    for (int s = 0; s < T::DS; ++s)
        qreg[s] = __builtin_bit_cast(
            bf16x8, load16(qb, ((uint32_t)qi * D + 16 * s + 8 * hi) * 2));

    const int kend = CAUSAL ? min(n, q0 + T::BR) : n;
    const int nkt = (kend + T::BC - 1) / T::BC;

    f32x16 acc[T::DB];
#pragma unroll
    for (int e = 0; e < T::DB; ++e) acc[e] = f32x16{};
    float m_run = kNegInf, l_run = 0.f;  // l_run: this lane's half of the keys

    // ---- tile movement: global -> LDS directly (no staging registers).
    //      Wave w issues the wave-wide 1 KiB loads w, w+4, ...; each lane's
    //      byte offset inside a tile is fixed, only the tile origin moves. ----
    constexpr int KL = (T::K_LOADS + 3) / 4, VL = (T::V_LOADS + 3) / 4;
    uint32_t koff[KL];
#pragma unroll
    for (int x = 0; x < KL; ++x) {
        const int t = wave + 4 * x;
        const int P = 64 * t + lane;  // padded chunk slot written by this lane
        const int r = P / T::KCH, c = P % T::KCH;
        koff[x] = (t < T::K_LOADS && c < T::CPR) ? (uint32_t)(r * D + c * 8) * 2
                                                  : kOutOfRange;  // pad: no fetch
    }
    // V: lane writes row RPL*t + lane/CPR, physical chunk lane%CPR, which holds
    // logical chunk (lane%CPR) ^ v_swz(row); v_swz depends on lane only here.
    const uint32_t voff = (uint32_t)((lane / T::CPR) * D +
                                     (((lane % T::CPR) ^ v_swz<D>(lane / T::CPR)) * 8)) * 2;
    auto load_k = [&](int k0, bf16* dst) {
#pragma unroll
        for (int x = 0; x < KL; ++x) {
            const int t = wave + 4 * x;
            if (t < T::K_LOADS)
                load16_lds(kb, koff[x] + (uint32_t)k0 * D * 2, dst + 512 * t);
        }
    };
    auto load_v = [&](int k0, bf16* dst) {
#pragma unroll
        for (int x = 0; x < VL; ++x) {
            const int t = wave + 4 * x;
            if (t < T::V_LOADS)
                load16_lds(vb, voff + (uint32_t)(k0 + T::RPL * t) * D * 2, dst + 512 * t);
        }
    };
    auto kbuf = [&](int i) { return lds + (i & 1) * T::K_ELEMS; };
    auto vbuf = [&](int i) { return lds + 2 * T::K_ELEMS + (i & 1) * T::V_ELEMS; };

    // ---- S^T = K Q^T for one tile: lane holds query qi and keys
    //      k0 + 32*bb + 8*(r/4) + 4*hi + r%4 ---------------------------------
    auto scores = [&](const bf16* ks, f32x16* s) {
        s[0] = f32x16{};
        s[1] = f32x16{};
#pragma unroll
        for (int ss = 0; ss < T::DS; ++ss)
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
                s[bb] = mfma32(
                    lds_read16(ks + (32 * bb + l32) * T::KSTR + 16 * ss + 8 * hi),
                    qreg[ss], s[bb]);
    };

    // ---- element mask: only on tiles crossing the diagonal or the sequence
    //      end.  Element (bb, r) is key k0 + 32bb + 8(r/4) + 4hi + r%4; it is
    //      allowed while that offset stays below this lane's limit. ----------
    auto needs_mask = [&](int k0) {
        return (CAUSAL && k0 + T::BC - 1 > qw0) || k0 + T::BC > n;
    };
    auto apply_mask = [&](f32x16* s, int k0) {
        int lim = n - k0;                             // keys before the end
        if (CAUSAL) lim = min(lim, qi - k0 + 1);      // keys j <= qi
        lim -= 4 * hi;
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (32 * bb + 8 * (r / 4) + (r & 3) >= lim) s[bb][r] = kNegInf;
    };

    // ---- online softmax statistics of one score tile: new running maximum
    //      (lazy), rescale factor, exponentials as bf16 B operands, row sum --
    auto softmax = [&](f32x16* s, bf16x8 (&pb)[2][2], float& alpha, bool& upd) {
        float mx = kNegInf;
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[bb][r]);
        mx = fmaxf(mx, xor32(mx)) * p.c;  // tile row maximum, base-2 units
        upd = mx > m_run + kLazyRescale;  // the first live tile always moves it
        const float m_new = upd ? mx : m_run;
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;  // no key yet: no NaN
        alpha = upd ? exp2_fast(m_run - m_use) : 1.f;
        m_run = m_new;
        float rs = 0.f;
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = exp2_fast(__builtin_fmaf(s[bb][r], p.c, -m_use));
                rs += e;
                pb[bb][r >> 3][r & 7] = to_bf16(e);
            }
        l_run = __builtin_fmaf(l_run, alpha, rs);
    };

    // ---- O^T += V^T P^T; V^T delivered by transpose reads of row-major V.
    //      Rows kr, kr+8 (kr = 32bb + 16t + 4hi + i16/4) share v_swz(kr), so
    //      the swizzled column depends on the lane and e only. ---------------
    auto pv = [&](const bf16x8 (&pb)[2][2], const bf16* vs) {
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int kr = 32 * bb + 16 * t + 4 * hi + (i16 >> 2);
#pragma unroll
                for (int e = 0; e < T::DB; ++e) {
                    const int dcol = 32 * e + 16 * (g & 1) + 4 * (i16 & 3);
                    const int col = (((dcol >> 3) ^ v_swz<D>(kr)) << 3) + (dcol & 7);
                    const bf16x4 va = lds_read_tr(vs + kr * D + col);
                    const bf16x4 vc = lds_read_tr(vs + (kr + 8) * D + col);
                    acc[e] = mfma32(cat(va, vc), pb[bb][t], acc[e]);
                }
            }
    };
    auto rescale = [&](float alpha, bool upd) {
        if (__any(upd)) {
#pragma unroll
            for (int e = 0; e < T::DB; ++e) acc[e] *= alpha;
        }
    };

    // ---- software pipeline: during tile j, K_{j+1} is already in LDS, so
    //      S_{j+1} = K_{j+1} Q^T (MFMA) and the softmax of S_j (VALU) form one
    //      branch-free block the scheduler can interleave.  K_{j+2} and V_{j+1}
    //      load into the buffers no wave reads this iteration, so one barrier
    //      per tile suffices.  The last tile is peeled off the loop. ---------
    load_k(0, kbuf(0));
    load_v(0, vbuf(0));
    if (nkt > 1) load_k(T::BC, kbuf(1));
    __builtin_amdgcn_s_waitcnt(0);  // Q registers and the first tiles landed
    __syncthreads();

    f32x16 s_cur[2], s_nxt[2];
    scores(kbuf(0), s_cur);  // tile 0 is never in any wave's future
    for (int j = 0; j + 1 < nkt; ++j) {
        const int k0 = j * T::BC;
        if (j + 2 < nkt) load_k(k0 + 2 * T::BC, kbuf(j));  // K_j consumed last iteration
        load_v(k0 + T::BC, vbuf(j + 1));                    // V_{j-1} likewise
        // a wave whose rows all precede tile j is done (its later tiles too)
        if (!(CAUSAL && k0 > qw0 + 31)) {
            if (needs_mask(k0)) apply_mask(s_cur, k0);
            bf16x8 pb[2][2];
            float alpha;
            bool upd;
            scores(kbuf(j + 1), s_nxt);
            softmax(s_cur, pb, alpha, upd);
            rescale(alpha, upd);
            pv(pb, vbuf(j));
            s_cur[0] = s_nxt[0];
            s_cur[1] = s_nxt[1];
        }
        wait_vmem();  // this iteration's tile loads have landed in LDS
        __syncthreads();
    }
    {
        const int j = nkt - 1, k0 = j * T::BC;
        if (!(CAUSAL && k0 > qw0 + 31)) {
            if (needs_mask(k0)) apply_mask(s_cur, k0);
            bf16x8 pb[2][2];
            float alpha;
            bool upd;
            softmax(s_cur, pb, alpha, upd);
            rescale(alpha, upd);
            pv(pb, vbuf(j));
        }
    }

    // epilogue: O = u / l (bf16), L = m + ln l (natural log, scaled units)
    const float l_tot = l_run + xor32(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int e = 0; e < T::DB; ++e)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int d = 32 * e + 8 * r4 + 4 * hi;
            store8(ob, ((uint32_t)qi * D + d) * 2,
                   pack4(acc[e][4 * r4] * inv, acc[e][4 * r4 + 1] * inv,
                         acc[e][4 * r4 + 2] * inv, acc[e][4 * r4 + 3] * inv));
        }
    if (hi == 0) {
        const float L = l_tot > 0.f ? (m_run + log2_fast(l_tot)) * kLn2 : kNegInf;
        store4(lb, (uint32_t)qi * 4, __builtin_bit_cast(uint32_t, L));
    }
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t run_fwd(const FwdArgs& a, hipStream_t stream) {
    using T = FwdTile<D>;
    FwdParams p;
    p.q = static_cast<const bf16*>(a.q);
    p.k = static_cast<const bf16*>(a.k);
    p.v = static_cast<const bf16*>(a.v);
    p.o = static_cast<bf16*>(a.o);
    p.lse = a.lse;
    p.cu = a.cu;
    p.H = a.H;
    p.N = a.N;
    p.n_qt = (a.max_seqlen + T::BR - 1) / T::BR;
    p.c = (float)((double)a.scale * 1.4426950408889634);
    const int64_t units = (int64_t)p.n_qt * a.H * a.B;
    hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, VARLEN>), dim3((unsigned)units),
                       dim3(T::THREADS), 0, stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t run_fwd_d(const FwdArgs& a, hipStream_t stream) {
    const bool varlen = a.cu != nullptr;
    if (a.causal)
        return varlen ? run_fwd<D, true, true>(a, stream)
                      : run_fwd<D, true, false>(a, stream);
    return varlen ? run_fwd<D, false, true>(a, stream)
                  : run_fwd<D, false, false>(a, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
    return a.D == 64 ? run_fwd_d<64>(a, stream) : run_fwd_d<128>(a, stream);
}

}  // namespace fa
