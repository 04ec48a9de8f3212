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
// Three launches, no atomics, deterministic:
//   1. dsum:  D_i = dO_i . O_i from the saved bf16 O (HBM-bound, tiny).
//   2. dkdv:  one unit per 128-key tile keeps K and V in registers and streams
//             query tiles (Q, dO, L, D) through LDS: S, P, dV += P^T dO,
//             dP = dO V^T, dS, dK += dS^T Q.
//   3. dq:    one unit per 128-query tile keeps Q and dO in registers and
//             streams key tiles (K, V) through LDS: S^T, P^T, dP^T, dS^T,
//             dQ += dS K.
// Recomputing S and dP in the dq pass costs two extra products out of seven
// but avoids a cross-unit reduction of dQ.
//
// Register layouts follow fa_device.hpp: with the score tile in the
// [query][key] orientation each lane holds one key and 16 queries of a 32x32
// block, which is exactly the B operand of the products contracted over
// queries (dV^T = dO^T P, dK^T = Q^T dS); their A operands (dO^T, Q^T) are
// transpose reads of the row-major LDS tiles.  The dq pass mirrors the
// forward kernel (lane = query).
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
    float* dsum;
    int H, N;
    float c;      // scale * log2(e)
    float scale;
};

// ---------------------------------------------------------------------------
// 1. D_i = dO_i . O_i  (fp32 sum of exact bf16 products)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void dsum_kernel(const bf16* o, const bf16* dout,
                                                   float* dsum, int64_t rows) {
    constexpr int LPR = D / 8;  // lanes per row, 16 bytes each
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gid / LPR;
    const int part = (int)(gid % LPR);
    float acc = 0.f;
    if (row < rows) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(o + row * D + part * 8);
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(dout + row * D + part * 8);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc = __builtin_fmaf((float)a[j], (float)b[j], acc);
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (row < rows && part == 0) dsum[row] = acc;
}

// ---------------------------------------------------------------------------
// 2. dK, dV: unit = (batch, head, 128-key tile); 4 waves x 32 keys.
// ---------------------------------------------------------------------------
template <int D>
struct KvTile {
    static constexpr int BK = 128;       // keys per unit
    static constexpr int BQ = 64;        // queries per streamed tile
    static constexpr int THREADS = 256;
    static constexpr int QSTR = D + 8;   // Q / dO row pitch in LDS (elements)
    static constexpr int T_ELEMS = BQ * QSTR;
    // stage layout: Q tile, dO tile (bf16), then L2 and D (fp32, BQ each)
    static constexpr int STAGE_BYTES = 2 * T_ELEMS * 2 + 2 * BQ * 4;
    static constexpr int CPT = BQ * D / 8 / THREADS;
    static constexpr int DS = D / 16;
    static constexpr int DB = D / 32;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void dkdv_kernel(BwdParams p) {
    using T = KvTile<D>;
    __shared__ __attribute__((aligned(16))) char lds_raw[2 * T::STAGE_BYTES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int g = lane >> 4, i16 = lane & 15;
    const int kt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int n = p.N;
    const int64_t row0 = ((int64_t)b * p.H + h) * n;
    const uint32_t bytes = (uint32_t)n * D * 2;
    const Buf qb = make_buf(p.q + row0 * D, bytes);
    const Buf kb = make_buf(p.k + row0 * D, bytes);
    const Buf vb = make_buf(p.v + row0 * D, bytes);
    const Buf dob = make_buf(p.dout + row0 * D, bytes);
    const Buf lb = make_buf(p.lse + row0, (uint32_t)n * 4);
    const Buf db = make_buf(p.dsum + row0, (uint32_t)n * 4);
    const Buf dkb = make_buf(p.dk + row0 * D, bytes);
    const Buf dvb = make_buf(p.dv + row0 * D, bytes);

    const int k0u = kt * T::BK;           // first key of the unit
    const int kw0 = k0u + 32 * wave;      // first key of this wave
    const int kj = kw0 + l32;             // key held by this lane

    // K and V as B operands (lane: row kj, columns 16s + 8hi + 0..7)
    bf16x8 kreg[T::DS], vreg[T::DS];
#pragma unroll
    for (int s = 0; s < T::DS; ++s) {
        const uint32_t off = ((uint32_t)kj * D + 16 * s + 8 * hi) * 2;
        kreg[s] = __builtin_bit_cast(bf16x8, load16(kb, off));
        vreg[s] = __builtin_bit_cast(bf16x8, load16(vb, off));
    }

    f32x16 dv[T::DB], dk[T::DB];
#pragma unroll
    for (int e = 0; e < T::DB; ++e) {
        dv[e] = f32x16{};
        dk[e] = f32x16{};
    }

    const int qt0 = CAUSAL ? k0u / T::BQ : 0;  // earlier queries see none of these keys
    const int nqt = (n + T::BQ - 1) / T::BQ;

    u32x4 qreg_g[T::CPT], doreg_g[T::CPT];
    float lval = 0.f;
    auto gload = [&](int q0) {
#pragma unroll
        for (int i = 0; i < T::CPT; ++i) {
            const int c = tid + T::THREADS * i;
            const int r = c / (D / 8), cc = c % (D / 8);
            const uint32_t off = ((uint32_t)(q0 + r) * D + cc * 8) * 2;
            qreg_g[i] = load16(qb, off);
            doreg_g[i] = load16(dob, off);
        }
        if (tid < T::BQ) lval = loadf(lb, (uint32_t)(q0 + tid) * 4) * kLog2e;
        else if (tid < 2 * T::BQ) lval = loadf(db, (uint32_t)(q0 + tid - T::BQ) * 4);
    };
    auto lstore = [&](int stage) {
        char* base = lds_raw + stage * T::STAGE_BYTES;
        bf16* qs = reinterpret_cast<bf16*>(base);
        bf16* dos = qs + T::T_ELEMS;
        float* fs = reinterpret_cast<float*>(dos + T::T_ELEMS);
#pragma unroll
        for (int i = 0; i < T::CPT; ++i) {
            const int c = tid + T::THREADS * i;
            const int r = c / (D / 8), cc = c % (D / 8);
            lds_write16(qs + r * T::QSTR + cc * 8, qreg_g[i]);
            lds_write16(dos + r * T::QSTR + cc * 8, doreg_g[i]);
        }
        if (tid < 2 * T::BQ) fs[tid] = lval;  // L2 at [0, BQ), D at [BQ, 2BQ)
    };

    auto compute = [&](int stage, int q0) {
        if (CAUSAL && q0 + T::BQ - 1 < kw0) return;  // every query precedes our keys
        const char* base = lds_raw + stage * T::STAGE_BYTES;
        const bf16* qs = reinterpret_cast<const bf16*>(base);
        const bf16* dos = qs + T::T_ELEMS;
        const float* l2s = reinterpret_cast<const float*>(dos + T::T_ELEMS);
        const float* dss = l2s + T::BQ;

        // S[query][key] for two 32-query blocks; lane holds key kj and local
        // queries 32*qb + 8*(r/4) + 4*hi + r%4.
        f32x16 s[2], dp[2];
#pragma unroll
        for (int qb2 = 0; qb2 < 2; ++qb2) {
            s[qb2] = f32x16{};
            dp[qb2] = f32x16{};
#pragma unroll
            for (int ss = 0; ss < T::DS; ++ss) {
                const int off = (32 * qb2 + l32) * T::QSTR + 16 * ss + 8 * hi;
                s[qb2] = mfma32(lds_read16(qs + off), kreg[ss], s[qb2]);
                dp[qb2] = mfma32(lds_read16(dos + off), vreg[ss], dp[qb2]);
            }
        }
        const bool need_mask = (CAUSAL && q0 < kw0 + 31) || (q0 + T::BQ > n);
        // P = exp2(S c - L2), dS = P (dP - D)
        bf16x8 pb[2][2], sb[2][2];
#pragma unroll
        for (int qb2 = 0; qb2 < 2; ++qb2)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int lq = 32 * qb2 + 8 * r4 + 4 * hi;  // first of 4 local queries
                const f32x4 l2 = *reinterpret_cast<const f32x4*>(l2s + lq);
                const f32x4 dd = *reinterpret_cast<const f32x4*>(dss + lq);
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int r = 4 * r4 + x;
                    float pv = exp2_fast(__builtin_fmaf(s[qb2][r], p.c, -l2[x]));
                    if (need_mask) {
                        const int qi = q0 + lq + x;
                        if ((CAUSAL && kj > qi) || qi >= n) pv = 0.f;
                    }
                    const float dsv = pv * (dp[qb2][r] - dd[x]);
                    pb[qb2][r / 8][r % 8] = to_bf16(pv);
                    sb[qb2][r / 8][r % 8] = to_bf16(dsv);
                }
            }
        // dV^T += dO^T P and dK^T += Q^T dS (A operands by transpose reads)
#pragma unroll
        for (int e = 0; e < T::DB; ++e) {
            const int dcol = 32 * e + 16 * (g & 1) + 4 * (i16 & 3);
#pragma unroll
            for (int qb2 = 0; qb2 < 2; ++qb2)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int qr = 32 * qb2 + 16 * t + 4 * hi + (i16 >> 2);
                    const bf16x8 doT = cat(lds_read_tr(dos + qr * T::QSTR + dcol),
                                           lds_read_tr(dos + (qr + 8) * T::QSTR + dcol));
                    dv[e] = mfma32(doT, pb[qb2][t], dv[e]);
                    const bf16x8 qT = cat(lds_read_tr(qs + qr * T::QSTR + dcol),
                                          lds_read_tr(qs + (qr + 8) * T::QSTR + dcol));
                    dk[e] = mfma32(qT, sb[qb2][t], dk[e]);
                }
        }
    };

    if (qt0 < nqt) {
        gload(qt0 * T::BQ);
        lstore(0);
        __syncthreads();
        for (int it = 0, qt = qt0; qt < nqt; ++qt, ++it) {
            const bool more = qt + 1 < nqt;
            if (more) gload((qt + 1) * T::BQ);
            compute(it & 1, qt * T::BQ);
            if (more) lstore((it + 1) & 1);
            __syncthreads();
        }
    }

    // dV[kj][d], dK[kj][d] = scale * acc (lane: key kj, d = 32e + 8(r/4) + 4hi + r%4)
#pragma unroll
    for (int e = 0; e < T::DB; ++e)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int d = 32 * e + 8 * r4 + 4 * hi;
            const uint32_t off = ((uint32_t)kj * D + d) * 2;
            store8(dvb, off, pack4(dv[e][4 * r4], dv[e][4 * r4 + 1],
                                   dv[e][4 * r4 + 2], dv[e][4 * r4 + 3]));
            store8(dkb, off,
                   pack4(dk[e][4 * r4] * p.scale, dk[e][4 * r4 + 1] * p.scale,
                         dk[e][4 * r4 + 2] * p.scale, dk[e][4 * r4 + 3] * p.scale));
        }
}

// ---------------------------------------------------------------------------
// 3. dQ: unit = (batch, head, 128-query tile); 4 waves x 32 queries.
// ---------------------------------------------------------------------------
template <int D>
struct QTile {
    static constexpr int BR = 128;
    static constexpr int BC = 64;
    static constexpr int THREADS = 256;
    static constexpr int KSTR = D + 8;
    static constexpr int K_ELEMS = BC * KSTR;
    static constexpr int STAGE = 2 * K_ELEMS;  // K then V
    static constexpr int CPT = BC * D / 8 / THREADS;
    static constexpr int DS = D / 16;
    static constexpr int DB = D / 32;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void dq_kernel(BwdParams p, int n_qt) {
    using T = QTile<D>;
    __shared__ __attribute__((aligned(16))) bf16 lds[2 * T::STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int g = lane >> 4, i16 = lane & 15;
    const int qt = CAUSAL ? (n_qt - 1 - (int)blockIdx.x) : (int)blockIdx.x;
    const int h = blockIdx.y, b = blockIdx.z;
    const int n = p.N;
    const int q0 = qt * T::BR;
    const int64_t row0 = ((int64_t)b * p.H + h) * n;
    const uint32_t bytes = (uint32_t)n * D * 2;
    const Buf qb = make_buf(p.q + row0 * D, bytes);
    const Buf kb = make_buf(p.k + row0 * D, bytes);
    const Buf vb = make_buf(p.v + row0 * D, bytes);
    const Buf dob = make_buf(p.dout + row0 * D, bytes);
    const Buf lb = make_buf(p.lse + row0, (uint32_t)n * 4);
    const Buf db = make_buf(p.dsum + row0, (uint32_t)n * 4);
    const Buf dqb = make_buf(p.dq + row0 * D, bytes);

    const int qw0 = q0 + 32 * wave;
    const int qi = qw0 + l32;

    bf16x8 qreg[T::DS], doreg[T::DS];
#pragma unroll
    for (int s = 0; s < T::DS; ++s) {
        const uint32_t off = ((uint32_t)qi * D + 16 * s + 8 * hi) * 2;
        qreg[s] = __builtin_bit_cast(bf16x8, load16(qb, off));
        doreg[s] = __builtin_bit_cast(bf16x8, load16(dob, off));
    }
    const float l2 = loadf(lb, (uint32_t)qi * 4) * kLog2e;
    const float dd = loadf(db, (uint32_t)qi * 4);

    const int kend = CAUSAL ? min(n, q0 + T::BR) : n;
    const int nkt = (kend + T::BC - 1) / T::BC;

    f32x16 acc[T::DB];
#pragma unroll
    for (int e = 0; e < T::DB; ++e) acc[e] = f32x16{};

    u32x4 kreg_g[T::CPT], vreg_g[T::CPT];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < T::CPT; ++i) {
            const int c = tid + T::THREADS * i;
            const int r = c / (D / 8), cc = c % (D / 8);
            const uint32_t off = ((uint32_t)(k0 + r) * D + cc * 8) * 2;
            kreg_g[i] = load16(kb, off);
            vreg_g[i] = load16(vb, off);
        }
    };
    auto lstore = [&](int stage) {
        bf16* ks = lds + stage * T::STAGE;
        bf16* vs = ks + T::K_ELEMS;
#pragma unroll
        for (int i = 0; i < T::CPT; ++i) {
            const int c = tid + T::THREADS * i;
            const int r = c / (D / 8), cc = c % (D / 8);
            lds_write16(ks + r * T::KSTR + cc * 8, kreg_g[i]);
            lds_write16(vs + r * T::KSTR + cc * 8, vreg_g[i]);
        }
    };
    auto compute = [&](int stage, int k0) {
        if (CAUSAL && k0 > qw0 + 31) return;
        const bf16* ks = lds + stage * T::STAGE;
        const bf16* vs = ks + T::K_ELEMS;
        // S^T and dP^T: lane holds query qi, keys k0 + 32bb + 8(r/4) + 4hi + r%4
        f32x16 s[2], dp[2];
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
            s[bb] = f32x16{};
            dp[bb] = f32x16{};
#pragma unroll
            for (int ss = 0; ss < T::DS; ++ss) {
                const int off = (32 * bb + l32) * T::KSTR + 16 * ss + 8 * hi;
                s[bb] = mfma32(lds_read16(ks + off), qreg[ss], s[bb]);
                dp[bb] = mfma32(lds_read16(vs + off), doreg[ss], dp[bb]);
            }
        }
        const bool need_mask = (CAUSAL && k0 + T::BC - 1 > qw0) || (k0 + T::BC > n);
        bf16x8 sb[2][2];
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float pv = exp2_fast(__builtin_fmaf(s[bb][r], p.c, -l2));
                if (need_mask) {
                    const int key = k0 + 32 * bb + 8 * (r / 4) + 4 * hi + (r & 3);
                    if ((CAUSAL && key > qi) || key >= n) pv = 0.f;
                }
                sb[bb][r / 8][r % 8] = to_bf16(pv * (dp[bb][r] - dd));
            }
        // dQ^T += K^T dS^T (K^T by transpose reads of row-major K)
#pragma unroll
        for (int e = 0; e < T::DB; ++e) {
            const int dcol = 32 * e + 16 * (g & 1) + 4 * (i16 & 3);
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int kr = 32 * bb + 16 * t + 4 * hi + (i16 >> 2);
                    const bf16x8 kT = cat(lds_read_tr(ks + kr * T::KSTR + dcol),
                                          lds_read_tr(ks + (kr + 8) * T::KSTR + dcol));
                    acc[e] = mfma32(kT, sb[bb][t], acc[e]);
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

#pragma unroll
    for (int e = 0; e < T::DB; ++e)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int d = 32 * e + 8 * r4 + 4 * hi;
            store8(dqb, ((uint32_t)qi * D + d) * 2,
                   pack4(acc[e][4 * r4] * p.scale, acc[e][4 * r4 + 1] * p.scale,
                         acc[e][4 * r4 + 2] * p.scale, acc[e][4 * r4 + 3] * p.scale));
        }
}

template <int D, bool CAUSAL>
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
    p.dsum = a.dsum;
    p.H = a.H;
    p.N = a.N;
    p.c = (float)((double)a.scale * 1.4426950408889634);
    p.scale = a.scale;

    const int64_t rows = (int64_t)a.B * a.H * a.N;
    const int64_t threads = rows * (D / 8);
    hipLaunchKernelGGL((dsum_kernel<D>), dim3((unsigned)((threads + 255) / 256)),
                       dim3(256), 0, stream, p.o, p.dout, p.dsum, rows);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;

    const int nkt = (a.N + KvTile<D>::BK - 1) / KvTile<D>::BK;
    hipLaunchKernelGGL((dkdv_kernel<D, CAUSAL>), dim3(nkt, a.H, a.B), dim3(256), 0,
                       stream, p);
    err = hipGetLastError();
    if (err != hipSuccess) return err;

    const int nqt = (a.N + QTile<D>::BR - 1) / QTile<D>::BR;
    hipLaunchKernelGGL((dq_kernel<D, CAUSAL>), dim3(nqt, a.H, a.B), dim3(256), 0,
                       stream, p, nqt);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
    if (a.D == 64)
        return a.causal ? run_bwd<64, true>(a, stream) : run_bwd<64, false>(a, stream);
    return a.causal ? run_bwd<128, true>(a, stream) : run_bwd<128, false>(a, stream);
}

}  // namespace fa
