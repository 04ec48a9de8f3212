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
    float* dd;     // [B, H, N]  D_i = dO_i . O_i
    float* nl2;    // [B, H, N]  -L_i * log2(e)
    int H, N;
    int per_head;  // dK/dV units per (batch, head): key tiles, or pairs if causal
    float c;       // scale * log2(e)
    float scale;
};

// Direct global -> LDS load of one dword per lane (lane i writes M0 + 4*i).
__device__ __forceinline__ void load4_lds(Buf b, uint32_t off, void* lds_wave_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(b.r, (FA_LDS void*)lds_wave_base, 4, off, 0,
                                             0, 0);
}
// s_waitcnt vmcnt(0) lgkmcnt(0): this wave's loads (global and LDS) are done.
__device__ __forceinline__ void wait_vmem_lds() { __builtin_amdgcn_s_waitcnt(0x0070); }

// Workgroup i of a 1-D grid runs on XCD i % 8; this remap gives each XCD a
// contiguous, head-major range of units so one head's tiles stay in one L2.
__device__ __forceinline__ void unit_of(int i, int total, int per_head, int& head,
                                        int& idx) {
    const int L = (total & 7) == 0 ? (i & 7) * (total >> 3) + (i >> 3) : i;
    head = L / per_head;
    idx = L - head * per_head;
}

// ---------------------------------------------------------------------------
// 1. Per-row constants: D_i = dO_i . O_i (fp32 sum of exact bf16 products)
//    and -L_i log2(e), the exponent offset that turns a score into its weight.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void dsum_kernel(const bf16* o, const bf16* dout,
                                                   const float* lse, float* dd, float* nl2,
                                                   int64_t rows) {
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
    if (row < rows && part == 0) {
        dd[row] = acc;
        nl2[row] = -lse[row] * kLog2e;
    }
}

// ---------------------------------------------------------------------------
// 2. dK, dV: unit = (batch, head, 128-key tile); wave w owns keys 32w..32w+31
//    of the tile and keeps their dK^T, dV^T accumulators in registers; K and V
//    sit in LDS for the whole unit while 64-query stages of Q, dO,
//    -L log2 e and D stream through double-buffered LDS.
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
    // K / V of the unit: row pitch padded by one chunk so the 16 rows a
    // quarter-wave reads with ds_read_b128 land 4 banks apart
    static constexpr int KSTR = D + 8;
    static constexpr int KV_ELEMS = BK * KSTR;
    static constexpr int KV_LOADS = BK * CPR / 64;  // 1 KiB loads per K or V tile
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

template <int D, bool CAUSAL>
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
    __shared__ __attribute__((aligned(16))) bf16 k_lds[T::KV_ELEMS];
    __shared__ __attribute__((aligned(16))) bf16 v_lds[T::KV_ELEMS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5;
    const int g = lane >> 4, i16 = lane & 15;
    int head, uidx;
    unit_of(blockIdx.x, gridDim.x, p.per_head, head, uidx);
    const int n = p.N;
    const int nkt = (n + T::BK - 1) / T::BK;
    // key tiles of this unit: under causal masking a heavy one (many queries
    // follow it) and the matching light one, so all units carry equal work
    int kt0 = uidx, kt1 = -1;
    if (CAUSAL) {
        kt1 = nkt - 1 - uidx;
        if (kt1 < kt0) return;
        if (kt1 == kt0) kt1 = -1;
    } else if (kt0 >= nkt) {
        return;
    }

    const int64_t row0 = (int64_t)head * n;
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

    f32x16 dk[T::DB], dv[T::DB];
    int kw0 = 0, kj = 0;

    // One 32-query block of a stage: S = Q K^T and dP = dO V^T (lane: key kj,
    // local queries 8(r/4) + 4hi + r%4), P = exp2(S c - L log2 e),
    // dS = P (dP - D), then dV^T += dO^T P and dK^T += Q^T dS with dO^T, Q^T
    // delivered by transpose reads.
    auto block = [&](const bf16* __restrict__ qs, const bf16* __restrict__ dos,
                     const float* __restrict__ fs, int q0, int b)
                     __attribute__((always_inline)) {
        const int qb0 = q0 + 32 * b;
        if (CAUSAL && qb0 + 31 < kw0) return;  // every query precedes our keys
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int ss = 0; ss < T::DS; ++ss) {
            const int off = qd_off<D>(32 * b + l32, 2 * ss + hi);
            const int koff = (32 * wave + l32) * T::KSTR + 16 * ss + 8 * hi;
            s = mfma32(lds_read16(qs + off), lds_read16(k_lds + koff), s);
            dp = mfma32(lds_read16(dos + off), lds_read16(v_lds + koff), dp);
        }
        const bool need_mask = CAUSAL && qb0 < kw0 + 31;
        const int tm = kj - qb0 - 4 * hi;  // masked where tm > local query offset
        bf16x8 pb[2], sb[2];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const f32x4 nl = *reinterpret_cast<const f32x4*>(fs + 32 * b + 8 * a + 4 * hi);
            const f32x4 dd = *reinterpret_cast<const f32x4*>(fs + T::BQ + 32 * b + 8 * a + 4 * hi);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int r = 4 * a + x;
                float pv = exp2_fast(__builtin_fmaf(s[r], p.c, nl[x]));
                if (need_mask) pv = tm > 8 * a + x ? 0.f : pv;
                const float dsv = pv * (dp[r] - dd[x]);
                pb[r / 8][r % 8] = to_bf16(pv);
                sb[r / 8][r % 8] = to_bf16(dsv);
            }
        }
#pragma unroll
        for (int e = 0; e < T::DB; ++e)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int rr = 32 * b + 16 * t + 4 * hi + (i16 >> 2);
                const int cc = 4 * e + 2 * (g & 1) + ((i16 & 3) >> 1);
                const int o0 = qd_off<D>(rr, cc) + 4 * (i16 & 1);
                const int o1 = qd_off<D>(rr + 8, cc) + 4 * (i16 & 1);
                const bf16x8 doT = cat(lds_read_tr(dos + o0), lds_read_tr(dos + o1));
                dv[e] = mfma32(doT, pb[t], dv[e]);
                const bf16x8 qT = cat(lds_read_tr(qs + o0), lds_read_tr(qs + o1));
                dk[e] = mfma32(qT, sb[t], dk[e]);
            }
    };
    auto step = [&](int qt, bool more, const bf16* __restrict__ qs,
                    const bf16* __restrict__ dos, const float* __restrict__ fs,
                    bf16* __restrict__ qn, bf16* __restrict__ don, float* __restrict__ fn)
                    __attribute__((always_inline)) {
        if (more) load_stage((qt + 1) * T::BQ, qn, don, fn);
        block(qs, dos, fs, qt * T::BQ, 0);
        // keep the two blocks apart: interleaving them would need more
        // registers than a wave has
        __builtin_amdgcn_sched_barrier(0);
        block(qs, dos, fs, qt * T::BQ, 1);
        wait_vmem_lds();  // next stage landed; this stage's reads are done
        barrier_only();
    };

    for (int rep = 0; rep < 2; ++rep) {
        const int kt = rep == 0 ? kt0 : kt1;
        if (kt < 0) break;
        const int k0u = kt * T::BK;
        kw0 = k0u + 32 * wave;
        kj = kw0 + l32;
        // K and V of the tile into LDS (rows padded to KSTR): the padded
        // layout is not contiguous, so these go through registers
#pragma unroll
        for (int x = 0; x < T::KV_LOADS / 4; ++x) {
            const int c = 64 * (wave + 4 * x) + lane;  // chunk index in the tile
            const int r = c / T::CPR, cc = c % T::CPR;
            const uint32_t off = ((uint32_t)(k0u + r) * D + cc * 8) * 2;
            lds_write16(k_lds + r * T::KSTR + cc * 8, load16(kb, off));
            lds_write16(v_lds + r * T::KSTR + cc * 8, load16(vb, off));
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
        for (int qt = qt_begin; qt < nqt; ++qt) {
            const bool more = qt + 1 < nqt;
            const bool odd = (qt - qt_begin) & 1;
            step(qt, more, odd ? q_lds1 : q_lds0, odd ? do_lds1 : do_lds0,
                 odd ? f_lds1 : f_lds0, odd ? q_lds0 : q_lds1, odd ? do_lds0 : do_lds1,
                 odd ? f_lds0 : f_lds1);
        }
        // dV[kj][d], dK[kj][d] = scale * acc (d = 32e + 8(r/4) + 4hi + r%4)
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
    const Buf nlb = make_buf(p.nl2 + row0, (uint32_t)n * 4);
    const Buf ddb = make_buf(p.dd + row0, (uint32_t)n * 4);
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
    const float nl2 = loadf(nlb, (uint32_t)qi * 4);
    const float dd = loadf(ddb, (uint32_t)qi * 4);

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
                float pv = exp2_fast(__builtin_fmaf(s[bb][r], p.c, nl2));
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
    const int64_t rows = (int64_t)a.B * a.H * a.N;
    p.dd = a.ws;
    p.nl2 = a.ws + ((rows + 63) & ~(int64_t)63);  // second region, 256-byte aligned
    p.H = a.H;
    p.N = a.N;
    p.c = (float)((double)a.scale * 1.4426950408889634);
    p.scale = a.scale;

    const int64_t threads = rows * (D / 8);
    hipLaunchKernelGGL((dsum_kernel<D>), dim3((unsigned)((threads + 255) / 256)),
                       dim3(256), 0, stream, p.o, p.dout, p.lse, p.dd, p.nl2, rows);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;

    const int nkt = (a.N + KvTile<D>::BK - 1) / KvTile<D>::BK;
    p.per_head = CAUSAL ? (nkt + 1) / 2 : nkt;
    const int64_t units = (int64_t)p.per_head * a.H * a.B;
    hipLaunchKernelGGL((dkdv_kernel<D, CAUSAL>), dim3((unsigned)units), dim3(256), 0,
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
