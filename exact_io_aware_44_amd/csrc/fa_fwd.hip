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
//  - Exponentials use exp2 with scale*log2(e) folded into one FMA per score.
//  - K/V tiles are double-buffered in LDS: the global loads of tile j+1 are
//    issued before the MFMAs of tile j and written to the other buffer after,
//    so one barrier per tile suffices.
//  - Causal: key tiles wholly after the unit's last row are never loaded; a
//    wave skips tiles wholly after its own rows; the element mask runs only on
//    tiles crossing the diagonal (or the ragged end of the sequence).
//  - Units are launched heaviest first under causal masking.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

template <int D>
struct FwdTile {
    static constexpr int BR = 128;       // query rows per work unit
    static constexpr int BC = 64;        // keys per streamed tile
    static constexpr int THREADS = 256;
    static constexpr int KSTR = D + 8;   // K row pitch (elements): rows 4 banks apart
    static constexpr int VSTR = D + 32;  // V row pitch: rows 16 banks apart
    static constexpr int K_ELEMS = BC * KSTR;
    static constexpr int STAGE = BC * (KSTR + VSTR);
    static constexpr int CPT = BC * D / 8 / THREADS;  // 16 B chunks / thread / tensor
    static constexpr int DS = D / 16;    // MFMA k-steps across the head width
    static constexpr int DB = D / 32;    // 32-wide blocks of the output
};

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

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdParams p) {
    using T = FwdTile<D>;
    __shared__ __attribute__((aligned(16))) bf16 lds[2 * T::STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int qt = CAUSAL ? (p.n_qt - 1 - (int)blockIdx.x) : (int)blockIdx.x;
    const int h = blockIdx.y, b = blockIdx.z;

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

    u32x4 kreg[T::CPT], vreg[T::CPT];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < T::CPT; ++i) {
            const int c = tid + T::THREADS * i;
            const int r = c / (D / 8), cc = c % (D / 8);
            const uint32_t off = ((uint32_t)(k0 + r) * D + cc * 8) * 2;
            kreg[i] = load16(kb, off);
            vreg[i] = load16(vb, off);
        }
    };
    auto lstore = [&](int stage) {
        bf16* ks = lds + stage * T::STAGE;
        bf16* vs = ks + T::K_ELEMS;
#pragma unroll
        for (int i = 0; i < T::CPT; ++i) {
            const int c = tid + T::THREADS * i;
            const int r = c / (D / 8), cc = c % (D / 8);
            lds_write16(ks + r * T::KSTR + cc * 8, kreg[i]);
            lds_write16(vs + r * T::VSTR + cc * 8, vreg[i]);
        }
    };

    const int g = lane >> 4, i16 = lane & 15;
    auto compute = [&](int stage, int k0) {
        if (CAUSAL && k0 > qw0 + 31) return;  // tile wholly in this wave's future
        const bf16* ks = lds + stage * T::STAGE;
        const bf16* vs = ks + T::K_ELEMS;

        // S^T for two 32-key blocks: lane holds query qi, keys
        // k0 + 32*bb + 8*(r/4) + 4*hi + r%4.
        f32x16 s[2];
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
            s[bb] = f32x16{};
#pragma unroll
            for (int ss = 0; ss < T::DS; ++ss)
                s[bb] = mfma32(
                    lds_read16(ks + (32 * bb + l32) * T::KSTR + 16 * ss + 8 * hi),
                    qreg[ss], s[bb]);
        }
        // element mask only on tiles crossing the diagonal or the sequence end
        const bool need_mask =
            (CAUSAL && k0 + T::BC - 1 > qw0) || (k0 + T::BC > n);
        if (need_mask) {
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 32 * bb + 8 * (r / 4) + 4 * hi + (r & 3);
                    if ((CAUSAL && key > qi) || key >= n) s[bb][r] = kNegInf;
                }
        }
        // running maximum (scaled, base-2 units)
        float mx = kNegInf;
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[bb][r]);
        mx = fmaxf(mx, xor32(mx));
        const float m_new = fmaxf(m_run, mx * p.c);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;  // no key yet: no NaN
        const float alpha = exp2_fast(m_run - m_use);
        float rs = 0.f;
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = exp2_fast(__builtin_fmaf(s[bb][r], p.c, -m_use));
                s[bb][r] = e;
                rs += e;
            }
        l_run = __builtin_fmaf(l_run, alpha, rs);
#pragma unroll
        for (int e = 0; e < T::DB; ++e) acc[e] *= alpha;
        m_run = m_new;

        // P^T as bf16 B operands: k-step t of block bb = registers 8t..8t+7
        bf16x8 pb[2][2];
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int j = 0; j < 8; ++j) pb[bb][t][j] = to_bf16(s[bb][8 * t + j]);

        // O^T += V^T P^T, V^T delivered by transpose reads of row-major V
#pragma unroll
        for (int e = 0; e < T::DB; ++e) {
            const int dcol = 32 * e + 16 * (g & 1) + 4 * (i16 & 3);
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int kr = 32 * bb + 16 * t + 4 * hi + (i16 >> 2);
                    const bf16x4 va = lds_read_tr(vs + kr * T::VSTR + dcol);
                    const bf16x4 vc = lds_read_tr(vs + (kr + 8) * T::VSTR + dcol);
                    acc[e] = mfma32(cat(va, vc), pb[bb][t], acc[e]);
                }
        }
    };

    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nkt; ++kt) {
        const bool more = kt + 1 < nkt;
        if (more) gload((kt + 1) * T::BC);
        compute(kt & 1, kt * T::BC);
        if (more) lstore((kt + 1) & 1);
        __syncthreads();
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
    const dim3 grid(p.n_qt, a.H, a.B);
    hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, VARLEN>), grid, dim3(T::THREADS), 0,
                       stream, p);
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
