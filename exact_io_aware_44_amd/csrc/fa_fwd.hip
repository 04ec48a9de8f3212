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
//  - 256 threads = 4 wave64s; wave w owns the 32 query rows q0 + 4i + w of the
//    128-row tile.  Spreading the rows makes every wave's causal range of key
//    tiles identical, so the loop has no per-wave branches.
//  - Scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16
//    with K read from LDS and Q held in registers.  In that orientation each
//    lane holds ONE query row (lane % 32) and 16 of the 32 keys of a block, so
//    the row maximum and sum are in-lane reductions plus one exchange with
//    lane ^ 32 (v_permlane32_swap), and the rescale factor is a per-lane
//    scalar.
//  - The same registers, rounded to bf16, are already the B operand of
//    O^T += V^T P^T (the key order inside an MFMA k-step is a free
//    permutation, matched on the V side).  V stays row-major in LDS and is
//    read with ds_read_b64_tr_b16, which delivers it column-major.
//  - Software pipeline on 32-key half tiles: half-step h issues, in one
//    branch-free block, the MFMAs of S_{h+1} = K_{h+1} Q^T and of
//    O^T += V_{h-1}^T P_{h-1}^T together with the VALU softmax of S_h.  The
//    three are independent, so the wave keeps the matrix pipe busy while its
//    own exponentials run; every MFMA operand is requested from LDS six
//    MFMAs ahead.  Two workgroups per CU give each SIMD a second such wave.
//  - Exponentials use exp2 with scale*log2(e) folded into one FMA per score;
//    the running maximum moves lazily (see kLazyRescale), so the accumulator
//    rescale is skipped on almost every tile.
//  - Tiles (64 keys) move global -> LDS directly (buffer_load ... lds),
//    double-buffered; the two half-steps of tile-step j read only K tile j+1
//    and V tile j, so K_{j+2} and V_{j+1} load into the other buffers meanwhile
//    and one barrier per tile suffices.
//  - Causal: key tiles wholly after the unit's last row are never loaded; the
//    element mask runs only on tiles crossing the diagonal (or the ragged end
//    of the sequence); a unit processes a light and a heavy query tile of the
//    same head so all units carry equal work.
//  - A 1-D grid is remapped so that each XCD owns whole heads (their K/V
//    re-reads hit its private L2).
#include <algorithm>
#include <type_traits>

#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

template <int D>
struct FwdTile {
    static constexpr int WAVES = 4;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int BR = 32 * WAVES;  // query rows per tile
    static constexpr int BC = 64;          // keys per streamed tile
    static constexpr int CPR = D / 8;      // 16-byte chunks per row
    // K: row pitch padded by one chunk, so the 16 rows a quarter-wave reads
    // with ds_read_b128 land 4 banks apart (conflict-free)
    static constexpr int KSTR = D + 8;
    static constexpr int KCH = KSTR / 8;           // chunks per padded row
    // wave-wide 1 KiB loads per K tile, rounded up to a multiple of the four
    // waves so every wave issues the same count with no guard; the extra
    // loads are out of range (no fetch) and only zero-fill the buffer's tail
    static constexpr int K_LOADS = (BC * KCH / 64 + 3) / 4 * 4;
    // V: unpadded rows, chunk index XOR-swizzled (see v_swz) so the transpose
    // reads of four rows x 64 bytes per half-wave hit distinct banks
    static constexpr int V_LOADS = BC * CPR / 64;
    static constexpr int K_ELEMS = K_LOADS * 512;  // >= BC * KSTR
    static constexpr int V_ELEMS = BC * D;
    static constexpr int DS = D / 16;      // MFMA k-steps across the head width
    static constexpr int DB = D / 32;      // 32-wide blocks of the output
    static constexpr int RPL = 64 / CPR;   // V rows per wave-wide load
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
constexpr float kLazyLimit = 256.f;  // 2^kLazyRescale

struct FwdParams {
    const bf16* q;
    const bf16* k;
    const bf16* v;
    bf16* o;
    float* lse;
    const int32_t* cu;
    int H;
    int N;         // queries per sequence (dense) or packed total (varlen)
    int Nk;        // keys per sequence (dense; varlen sequences use their own)
    int per_head;  // units per (batch, head): query tiles, or pairs if causal
    float c;       // softmax_scale * log2(e)
    // split key ranges (decoding): unit (query tile, split s) reads keys
    // [s * chunk, (s + 1) * chunk) and writes its normalised partial O (fp32)
    // and L to part_o / part_l, row (s * B * H + head) * N + i
    int splits;
    int chunk;
    int heads;     // B * H
    float* part_o;
    float* part_l;
    Dropout drop;  // attention dropout (dense forward only)
    // dense causal: the last `tail` heads of each XCD are issued as single
    // query tiles, heaviest first (0: every unit is a pair of tiles)
    int tail;
};


using True = std::true_type;
using False = std::false_type;

template <typename E, int D, bool CAUSAL, bool VARLEN, bool SPLIT, bool DROP>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdParams p) {
    using T = FwdTile<D>;
    // Separate LDS objects per buffer, always selected statically, so the
    // compiler can tell a tile being read from the tile a DMA is filling and
    // does not hold the reads back until every load has landed.
    __shared__ __attribute__((aligned(16))) bf16 k_lds0[T::K_ELEMS];
    __shared__ __attribute__((aligned(16))) bf16 k_lds1[T::K_ELEMS];
    __shared__ __attribute__((aligned(16))) bf16 v_lds0[T::V_ELEMS];
    __shared__ __attribute__((aligned(16))) bf16 v_lds1[T::V_ELEMS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int l32 = lane & 31, hi = lane >> 5;
    const int g = lane >> 4, i16 = lane & 15;
    int head, uidx, rank = -1;
    if (CAUSAL && !SPLIT && !VARLEN && p.tail > 0)
        tail_unit(blockIdx.x, p.heads, p.per_head, p.tail, head, uidx, rank);
    else
        unit_of(blockIdx.x, gridDim.x, p.per_head, head, uidx);
    const int b = head / p.H, h = head - b * p.H;
    int split = 0;
    if constexpr (SPLIT) {
        split = uidx % p.splits;
        uidx /= p.splits;
    }

    // n queries attend to nk keys; under the causal mask query i reads keys
    // j <= i + shift (shift = nk - n: the queries are the last n positions)
    int n, nk;
    int64_t row0, krow0;
    if constexpr (VARLEN) {
        int s = p.cu[b], e = p.cu[b + 1];
        s = min(max(s, 0), p.N);
        e = min(max(e, s), p.N);
        n = nk = e - s;
        row0 = krow0 = (int64_t)h * p.N + s;
    } else {
        n = p.N;
        nk = p.Nk;
        row0 = ((int64_t)b * p.H + h) * p.N;
        krow0 = ((int64_t)b * p.H + h) * p.Nk;
    }
    int shift = nk - n;
    // split mode: this unit reads keys [kbeg, kbeg + nk) of the sequence;
    // rebasing K/V there keeps every key index below relative to the range
    int kbeg = 0;
    if constexpr (SPLIT) {
        kbeg = min(nk, split * p.chunk);
        nk = min(nk - kbeg, p.chunk);
        shift -= kbeg;
    }
    // the query tiles of this unit, heavy first; ntiles is workgroup-uniform
    const int n_tiles = (n + T::BR - 1) / T::BR;
    int tile0, tile1;
    if (!fwd_tiles(CAUSAL && !SPLIT, rank, uidx, n_tiles, tile0, tile1)) return;
    const int ntiles = tile1 >= 0 ? 2 : 1;

    const uint32_t bytes = (uint32_t)n * D * 2;
    const uint32_t kbytes = (uint32_t)nk * D * 2;
    const Buf qb = make_buf(p.q + row0 * D, bytes);
    const Buf ob = make_buf(p.o + row0 * D, bytes);
    const Buf lb = p.lse ? make_buf(p.lse + row0, (uint32_t)n * 4)
                         : make_buf(nullptr, 0);
    // split mode: partial outputs of this key range (fp32)
    const int64_t prow0 = ((int64_t)split * p.heads + head) * n;
    const Buf pob = SPLIT ? make_buf(p.part_o + prow0 * D, (uint32_t)n * D * 4)
                          : make_buf(nullptr, 0);
    const Buf plb = SPLIT ? make_buf(p.part_l + prow0, (uint32_t)n * 4)
                          : make_buf(nullptr, 0);

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
        koff[x] = (r < T::BC && c < T::CPR) ? (uint32_t)(r * D + c * 8) * 2
                                             : kOutOfRange;  // pad: no fetch
    }
    // V: lane writes row RPL*t + lane/CPR, physical chunk lane%CPR, which holds
    // logical chunk (lane%CPR) ^ v_swz(row); v_swz depends on lane only here.
    const uint32_t voff = (uint32_t)((lane / T::CPR) * D +
                                     (((lane % T::CPR) ^ v_swz<D>(lane / T::CPR)) * 8)) * 2;
    static_assert(T::K_LOADS % 4 == 0 && T::V_LOADS % 4 == 0, "loads split evenly");
    // A tile's origin moves the (scalar) buffer descriptor, not the per-lane
    // offsets: its base advances and its range shrinks by k0 rows, so the
    // range check still ends at the last key and the loop does no per-lane
    // address arithmetic for the DMAs.
    const bf16* kbase = p.k + (krow0 + kbeg) * D;
    const bf16* vbase = p.v + (krow0 + kbeg) * D;
    uint32_t voffx[VL];
#pragma unroll
    for (int x = 0; x < VL; ++x) voffx[x] = voff + (uint32_t)(T::RPL * (wave + 4 * x)) * D * 2;
    auto tile_buf = [&](const bf16* base, int k0) {
        // callers load only tiles that start before the last key: k0 < nk
        const uint32_t rest = __builtin_amdgcn_readfirstlane(kbytes - (uint32_t)k0 * D * 2);
        return make_buf(base + (size_t)k0 * D, rest);
    };
    auto load_k = [&](int k0, bf16* dst) {
        const Buf b = tile_buf(kbase, k0);
#pragma unroll
        for (int x = 0; x < KL; ++x)
            load16_lds(b, koff[x], dst + 512 * (wave + 4 * x));
    };
    auto load_v = [&](int k0, bf16* dst) {
        const Buf b = tile_buf(vbase, k0);
#pragma unroll
        for (int x = 0; x < VL; ++x)
            load16_lds(b, voffx[x], dst + 512 * (wave + 4 * x));
    };

    for (int rep = 0; rep < ntiles; ++rep) {
    const int q0 = (rep == 0 ? tile0 : tile1) * T::BR;
    // Query row held by this lane: the waves interleave (every fourth row),
    // so each wave meets the causal diagonal's mask in the same measure.
    // Under dropout a wave holds 32 consecutive rows instead, which puts the
    // 4 queries of one generator call in one quad of lanes.
    auto row_of = [&](int l) { return DROP ? q0 + 32 * wave + l : q0 + 4 * l + wave; };
    const int qi = row_of(l32);

    // Q as the B operand of S^T = K Q^T: lane holds Q[qi][16s + 8hi + 0..7].
    bf16x8 qreg[T::DS];
#pragma unroll
    for (int s = 0; s < T::DS; ++s)
        qreg[s] = __builtin_bit_cast(
            bf16x8, load16(qb, ((uint32_t)qi * D + 16 * s + 8 * hi) * 2));

    // keys the tile reads: up to its last row's limit (none at all when
    // every row precedes the first key)
    const int kend = CAUSAL ? max(0, min(nk, q0 + T::BR + shift)) : nk;
    const int nkt = (kend + T::BC - 1) / T::BC;
    // Order of the key tiles.  The units of a head that run together on one
    // XCD start their heavy tiles together and walk them up from key 0 in
    // step, so they share each K/V tile in L2.  Their light tiles start at
    // staggered times (unit u after n_tiles - u heavy steps); walked up from
    // key 0 they would each want a different tile, but walked down from the
    // last one, every light tile of the round reads the same key position at
    // the same time (u's light tile has u + 1 tiles, so at time t it is at
    // tile n_tiles - t).  Step tile t of the walk is key tile kt0(t) / BC;
    // logical half h (the order the pipeline runs) is physical half ph(h).
    // Any order of the key tiles gives the same softmax up to rounding.
    const bool rev = CAUSAL && !SPLIT && tile1 >= 0 && rep == 1;
    auto kt0 = [&](int t) { return (rev ? nkt - 1 - t : t) * T::BC; };
    auto ph = [&](int h) { return rev ? 2 * (nkt - 1 - (h >> 1)) + (h & 1) : h; };

    f32x16 acc[T::DB];
#pragma unroll
    for (int e = 0; e < T::DB; ++e) acc[e] = f32x16{};
    float m_run = kNegInf, l_run = 0.f;  // l_run: this lane's half of the keys
    float m_thr = kNegInf;                 // m_run + kLazyRescale
    float l_new = 0.f;                     // sum of the latest half's weights

    // ---- the pipeline works on 32-key half tiles: half h holds keys
    //      32h' .. 32h'+31 with h' = ph(h) (LDS tile h/2, rows 32*(h%2) ..).
    //      Its scores live in one f32x16 (lane: query qi, keys 32h' + 8(r/4)
    //      + 4hi + r%4) and its weights in two bf16x8 B operands (k-steps of
    //      16 keys). -----------------------------------------------------------
    //
    // element mask: only on halves crossing the diagonal or the sequence end;
    // element r is allowed while its key offset stays below this lane's limit
    auto needs_mask = [&](int hl) {
        const int h = ph(hl);
        return (CAUSAL && 32 * h + 31 > q0 + shift) || 32 * h + 32 > nk;
    };
    auto apply_mask = [&](f32x16& s, int hl) {
        const int h = ph(hl);
        int lim = nk - 32 * h;                                  // keys before the end
        if (CAUSAL) lim = min(lim, qi + shift - 32 * h + 1);    // keys j <= qi + shift
        lim -= 4 * hi;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (8 * (r / 4) + (r & 3) >= lim) s[r] = kNegInf;
    };

    // online softmax of one half: new running maximum (lazy), exponentials as
    // bf16 B operands, row sum.  m_use is the reference maximum the half's
    // weights are taken against; the running state (m_run, m_thr) moves only
    // in rescale(), whose branch runs on the rare half-steps where some
    // lane's maximum grew.  CHK: the half may hold a row with no live key so
    // far (only masked halves can), whose maximum is -inf.
    auto softmax = [&](f32x16& s, bf16x8 (&pb)[2], float& m_use, bool& upd, int hsm,
                       auto chk) {
        constexpr bool CHK = decltype(chk)::value;
        float t4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            t4[i] = fmaxf(fmaxf(s[4 * i], s[4 * i + 1]), fmaxf(s[4 * i + 2], s[4 * i + 3]));
        float mx = fmaxf(fmaxf(t4[0], t4[1]), fmaxf(t4[2], t4[3]));
        mx = pair_max(mx) * p.c;  // row maximum of the half, base-2 units
        upd = mx > m_thr;  // the first live half always moves it
        const float m_new = upd ? mx : m_run;
        m_use = (CHK && m_new == kNegInf) ? 0.f : m_new;  // no key yet: no NaN
        // exponentials in place, summed in fp32 in four independent chains
        // (summing the bf16-rounded weights instead would put up to 2^-9
        // relative error into l when one weight dominates and the reference
        // maximum is stale), then rounded to 16-bit B operands
        float rs[4];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s[r] = exp2_fast(__builtin_fmaf(s[r], p.c, -m_use));
            rs[r & 3] = r < 4 ? s[r] : rs[r & 3] + s[r];
        }
        if constexpr (DROP) {
            // dropped weights leave the P.V operand, not the sum l (L is the
            // log-sum-exp of all allowed scores).  Each group a of 4 keys is
            // one generator call and this lane reads the word of its query;
            // the quad's lanes (queries q .. q+3) need the same 4 calls, so
            // lane t makes the call of group t and the quad trades words.
            const int t = qi & 3;
            const u32x4 mine = dropout_block(p.drop, head, qi, 32 * ph(hsm) + 8 * t + 4 * hi);
            // word t ^ d of this lane's call goes to quad lane t ^ d
            const u32x4 wd = quad_share(t, xor_permute(mine, t));
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    if (!dropout_keep(wd[a], x, p.drop.thresh)) s[4 * a + x] = 0.f;
        }
        pb[0] = pack8<E>(s, 0);
        pb[1] = pack8<E>(s, 8);
        l_new = (rs[0] + rs[1]) + (rs[2] + rs[3]);  // taken against m_new
    };
    // Interior halves (every row already has a finite running maximum, no
    // mask, no dropout): the weights are taken against the running maximum
    // as it stands, without first finding the half's maximum; s is left
    // intact.  The lazy bound still holds when every weight is at most 2^8,
    // which a row sum l_new <= 2^8 guarantees (an overflow shows there as
    // inf); settle() checks it after the half-step and otherwise redoes the
    // half exactly as softmax() and rescale() would, so the result is the
    // same either way.
    auto softmax_fast = [&](const f32x16& s, bf16x8 (&pb)[2]) {
        float w[16], rs[4];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            w[r] = exp2_fast(__builtin_fmaf(s[r], p.c, -m_run));
            rs[r & 3] = r < 4 ? w[r] : rs[r & 3] + w[r];
        }
        pb[0] = pack8<E>(w);
        pb[1] = pack8<E>(w + 8);
        l_new = (rs[0] + rs[1]) + (rs[2] + rs[3]);
    };
    // Bring the old sums (u, and l before this half) to the new maximum, then
    // add this half's sum.  The log2 factor m_old - m_new is 0 on lanes whose
    // maximum did not move, and the exponential and the multiplies run only
    // when some lane moved.
    auto rescale = [&](float m_use, bool upd) {
        if (__any(upd)) {
            const float f = exp2_fast(m_run - m_use);
            m_run = upd ? m_use : m_run;
            m_thr = m_run + kLazyRescale;
#pragma unroll
            for (int e = 0; e < T::DB; ++e) acc[e] *= f;
            l_run *= f;
        }
        l_run += l_new;
    };
    auto settle = [&](f32x16& s, bf16x8 (&pb)[2], int hsm) {
        if (__any(l_new > kLazyLimit)) {  // a weight may exceed 2^8: the exact path
            float m_use;
            bool upd;
            softmax(s, pb, m_use, upd, hsm, False{});
            rescale(m_use, upd);
        } else {
            l_run += l_new;
        }
    };

    uint32_t voffb[T::DB];
#pragma unroll
    for (int e = 0; e < T::DB; ++e) {
        const int kr = 4 * hi + (i16 >> 2);
        const int dcol = 32 * e + 16 * (g & 1) + 4 * (i16 & 3);
        voffb[e] = (uint32_t)(kr * D + (((dcol >> 3) ^ v_swz<D>(kr)) << 3) + (dcol & 7)) * 2;
    }
    // MFMA operands.  S: A = K rows (ds_read_b128), B = Q registers.  P.V:
    // A = V^T by transpose reads, B = P^T; rows kr, kr+8 (kr = 16bt + 4hi +
    // i16/4) share v_swz(kr), so the swizzled column depends on lane and e.
    auto k_op = [&](const bf16* ks, int half, int ss) {
        return lds_read16(ks + (32 * half + l32) * T::KSTR + 16 * ss + 8 * hi);
    };
    auto v_op = [&](const bf16* vs, int bt, int e) {
        // byte offset of this lane's read: row 4hi + i16/4 (+16 bt, +8),
        // swizzled column of block e (the swizzle depends on the row mod 4
        // only, so bt does not change it)
        const char* p = reinterpret_cast<const char*>(vs) + voffb[e] + 16 * bt * D * 2;
        return cat(lds_read_tr(reinterpret_cast<const bf16*>(p)),
                   lds_read_tr(reinterpret_cast<const bf16*>(p + 8 * D * 2)));
    };

    // ---- one half-step: S of the next half (DS MFMAs, rows 32*kh of ks) if
    //      DO_S, P.V of the previous half (2*DB MFMAs, rows 32*vh of vs, with
    //      pb_prev) if DO_PV, and the softmax of s_cur into pb_new if DO_SM.
    //      MFMAs alternate S / P.V (independent neighbours) and every operand
    //      is requested from LDS six MFMAs ahead; the compiler interleaves
    //      the softmax VALU work (pinning a fixed pattern measured slower). --
    auto half_step = [&](auto do_s, auto do_pv, auto do_sm, auto chk, int hsm, const bf16* ks,
                         int kh, const bf16* vs, int vh, f32x16& s_cur, f32x16& s_nxt,
                         const bf16x8 (&pb_prev)[2], bf16x8 (&pb_new)[2], float& m_use,
                         bool& upd) {
        constexpr bool DO_S = decltype(do_s)::value, DO_PV = decltype(do_pv)::value;
        constexpr bool DO_SM = decltype(do_sm)::value;
        constexpr int NS = DO_S ? T::DS : 0, NP = DO_PV ? 2 * T::DB : 0;
        constexpr int NM = NS + NP;
        constexpr bool MIX = DO_S && DO_PV;  // NS == NP: alternate
        auto kind_s = [](int i) { return MIX ? (i & 1) == 0 : DO_S; };
        auto fetch = [&](int i) -> bf16x8 {
            if (kind_s(i)) return k_op(ks, kh, MIX ? i >> 1 : i);
            const int k = MIX ? i >> 1 : i;  // P.V k-step t = k / DB, block e = k % DB
            return v_op(vs, 2 * vh + k / T::DB, k % T::DB);
        };
        auto apply = [&](int i, bf16x8 a) {
            if (kind_s(i)) {
                s_nxt = mfma32<E>(a, qreg[MIX ? i >> 1 : i], s_nxt);
            } else {
                const int k = MIX ? i >> 1 : i;
                acc[k % T::DB] = mfma32<E>(a, pb_prev[k / T::DB], acc[k % T::DB]);
            }
        };
        if constexpr (DO_S) s_nxt = f32x16{};
        constexpr int PF = 6;  // operand read distance, in MFMAs
        bf16x8 op[NM > 0 ? NM : 1];
#pragma unroll
        for (int i = 0; i < PF && i < NM; ++i) op[i] = fetch(i);
        if constexpr (DO_SM) {
            if constexpr (!decltype(chk)::value && !DROP) softmax_fast(s_cur, pb_new);
            else softmax(s_cur, pb_new, m_use, upd, hsm, chk);
        }
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            if (i + PF < NM) op[i + PF] = fetch(i + PF);
            apply(i, op[i]);
        }
        // the new weights and their sum are due here, inside this block of
        // MFMAs, not after the rescale branch that follows the half-step:
        // otherwise the compiler sinks the exponentials past that branch,
        // into a block with no matrix work to overlap
        if constexpr (DO_SM) {
            const bf16x8 w0 = pb_new[0], w1 = pb_new[1];
            const float ls = l_new;
            asm volatile("" ::"v"(w0), "v"(w1), "v"(ls));
        }
    };

    // a tile whose queries all precede the first key reads nothing: O = 0,
    // L = -inf (the epilogue below with zero sums)
    if (nkt > 0) {
        // ---- prologue: K_0, K_1, V_0 -> LDS; S of half 0; half-step 0 (S of
        //      half 1 with the softmax of half 0) -------------------------------
        load_k(kt0(0), k_lds0);
        if (nkt > 1) load_k(kt0(1), k_lds1);
        load_v(kt0(0), v_lds0);
        wait_vmem();  // Q registers and the first tiles landed
        barrier_only();
        f32x16 sA, sB;  // scores of even / odd halves
        bf16x8 pA[2], pB[2];  // weights of even / odd halves
        float m_use;  // reference maximum of the latest half's weights
        bool upd;
        sA = f32x16{};
    #pragma unroll
        for (int ss = 0; ss < T::DS; ++ss) sA = mfma32<E>(k_op(k_lds0, 0, ss), qreg[ss], sA);
        if (needs_mask(0)) apply_mask(sA, 0);
        half_step(True{}, False{}, True{}, True{}, 0, k_lds0, 1, nullptr, 0, sA, sB, pB, pA,
                  m_use, upd);
        m_run = upd ? m_use : m_run;  // first half: nothing to rescale
        m_thr = m_run + kLazyRescale;
        l_run = l_new;
        __syncthreads();  // K_0 is consumed before tile-step 0 reloads its buffer

        // ---- tile-steps.  Tile-step j runs half-steps 2j+1 (odd: softmax sB ->
        //      pB, S of half 2j+2 -> sA, P.V of half 2j with pA) and 2j+2 (even:
        //      softmax sA -> pA, S of half 2j+3 -> sB, P.V of half 2j+1 with pB).
        //      It reads only K tile j+1 (buffer (j+1)%2) and V tile j (buffer
        //      j%2), so K_{j+2} and V_{j+1} load into the other buffers during
        //      it; one barrier ends it. ---------------------------------------
        // The buffer pointers are __restrict__: the tile a DMA is filling never
        // overlaps a tile being read, which lets the compiler leave the loads in
        // flight while the reads proceed.
        // MASKED: the tile-step may hold halves on the causal diagonal or past
        // the end; interior tile-steps skip the checks, so their body holds
        // no branch besides the (rare) rescale.  Walking up, interior
        // tile-steps only run when every row of the tile reads keys 0..95
        // (see j_int below), so half 0 already gave each row a finite
        // maximum: their softmax needs no -inf guard (mask_tag doubles as
        // CHK).  Walking down, they follow every masked step; a row whose
        // allowed keys all lie in interior tiles (a bottom-right mask can
        // do that) enters them with maximum -inf, its first interior half
        // then sums to +inf in softmax_fast(), and settle() redoes that half
        // exactly against the half's own (finite) maximum
        auto tile_step = [&](int j, const bf16* __restrict__ k_rd, const bf16* __restrict__ v_rd,
                             bf16* __restrict__ k_wr, bf16* __restrict__ v_wr, auto mask_tag) {
            constexpr bool MASKED = decltype(mask_tag)::value;
            if (j + 2 < nkt) load_k(kt0(j + 2), k_wr);
            load_v(kt0(j + 1), v_wr);
            if (MASKED && needs_mask(2 * j + 1)) apply_mask(sB, 2 * j + 1);
            half_step(True{}, True{}, True{}, mask_tag, 2 * j + 1, k_rd, 0, v_rd, 0, sB, sA, pA,
                      pB, m_use, upd);
            if (MASKED || DROP) rescale(m_use, upd);
            else settle(sB, pB, 2 * j + 1);
            if (MASKED && needs_mask(2 * j + 2)) apply_mask(sA, 2 * j + 2);
            half_step(True{}, True{}, True{}, mask_tag, 2 * j + 2, k_rd, 1, v_rd, 1, sA, sB, pB,
                      pA, m_use, upd);
            if (MASKED || DROP) rescale(m_use, upd);
            else settle(sA, pA, 2 * j + 2);
            wait_vmem();  // K_{j+2} and V_{j+1} landed
            barrier_only();
        };
        // tile-steps whose halves 2j+1, 2j+2 all lie before the diagonal and
        // the end need no mask: j < j_int
        // (half 2j+2 ends at key 64j + 95: it must not pass the first row's
        // limit q0 + shift, nor the last key nk - 1)
        int j_int = (nk - 32) / T::BC;
        if (CAUSAL) j_int = min(j_int, (q0 + shift - 31) / T::BC);
        j_int = max(0, min(j_int, nkt - 1));
        int j = 0;
        if (rev) {
            // reverse walk: masked steps first.  Physical halves from hm on
            // need the mask; step j reads physical halves 2(nkt-1-j)+1 and
            // 2(nkt-2-j), so it is interior once nkt-1-j <= (hm-2)/2.  The
            // masked prefix is rounded up to an even count so the interior
            // pairs below keep their static buffers.
            int hm = nk / 32;
            if (CAUSAL) hm = min(hm, q0 + shift < 31 ? 0 : (q0 + shift - 31) / 32 + 1);
            const int tmax = hm >= 2 ? (hm - 2) / 2 : -1;
            const int j_lo = max(0, nkt - 1 - tmax);
            const int j_pre = min(nkt - 1, (j_lo + 1) & ~1);
            for (; j < j_pre; ++j) {
                const bool odd = j & 1;
                tile_step(j, odd ? k_lds0 : k_lds1, odd ? v_lds1 : v_lds0, odd ? k_lds1 : k_lds0,
                          odd ? v_lds0 : v_lds1, True{});
            }
            j_int = nkt - 1;
        }
        // two tile-steps per trip: the buffers of each are then static
        for (; j + 1 < j_int; j += 2) {
            tile_step(j, k_lds1, v_lds0, k_lds0, v_lds1, False{});
            tile_step(j + 1, k_lds0, v_lds1, k_lds1, v_lds0, False{});
        }
        for (; j < j_int; ++j) {
            const bool odd = j & 1;
            tile_step(j, odd ? k_lds0 : k_lds1, odd ? v_lds1 : v_lds0, odd ? k_lds1 : k_lds0,
                      odd ? v_lds0 : v_lds1, False{});
        }
        for (; j + 1 < nkt; ++j) {
            const bool odd = j & 1;
            tile_step(j, odd ? k_lds0 : k_lds1, odd ? v_lds1 : v_lds0, odd ? k_lds1 : k_lds0,
                      odd ? v_lds0 : v_lds1, True{});
        }
        // last tile-step j = nkt - 1: softmax of half 2nkt-1 with P.V of half
        // 2nkt-2, then P.V of half 2nkt-1
        {
            const int j = nkt - 1;
            const bf16* v_rd = (j & 1) ? v_lds1 : v_lds0;
            if (needs_mask(2 * j + 1)) apply_mask(sB, 2 * j + 1);
            half_step(False{}, True{}, True{}, True{}, 2 * j + 1, nullptr, 0, v_rd, 0, sB, sA, pA,
                      pB, m_use, upd);
            rescale(m_use, upd);
            half_step(False{}, True{}, False{}, True{}, 0, nullptr, 0, v_rd, 1, sA, sB, pB, pA,
                      m_use, upd);
        }
        // no barrier here: the last tile-step reads only V, the epilogue
        // below stages each wave's O rows in the K buffers (last read before
        // the previous tile-step's barrier), and the barrier that follows the
        // staging orders every wave's reads before the next tile's loads
    }

    // epilogue: O = u / l (bf16), L = m + ln l (natural log, scaled units);
    // in split mode the same quantities of the key range, in fp32
    const float l_tot = pair_sum(l_run);
    // kept weights carry 1 / (1 - p'), folded into the normalisation
    const float inv = l_tot > 0.f ? (DROP ? p.drop.inv_keep : 1.f) / l_tot : 0.f;
    const float L = l_tot > 0.f ? (m_run + log2_fast(l_tot)) * kLn2 : kNegInf;
    if constexpr (SPLIT) {
#pragma unroll
        for (int e = 0; e < T::DB; ++e)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d = 32 * e + 8 * r4 + 4 * hi;
                const f32x4 ov{acc[e][4 * r4] * inv, acc[e][4 * r4 + 1] * inv,
                               acc[e][4 * r4 + 2] * inv, acc[e][4 * r4 + 3] * inv};
                store16(pob, ((uint32_t)qi * D + d) * 4, __builtin_bit_cast(u32x4, ov));
            }
    } else {
        // O leaves through LDS: a lane holds 8-byte pieces of one row, and
        // stored directly each store instruction would write 32 rows in
        // 16-byte pieces.  The wave stages its 32 rows in a K buffer (free
        // after the last tile-step) and writes them back as whole rows, 16
        // bytes per lane, with the non-temporal hint (written once, not read
        // again here).  Staged rows are padded by 16 bytes so the 8-byte
        // writes of 32 rows spread over the banks.
        constexpr int OSTR = D + 8;
        constexpr int RPI = 64 / T::CPR;  // rows per read-back instruction
        static_assert(2 * 32 * OSTR <= T::K_ELEMS, "two waves' rows fit in one K buffer");
        bf16* const ost = ((wave & 2) ? k_lds1 : k_lds0) + (wave & 1) * 32 * OSTR;
#pragma unroll
        for (int e = 0; e < T::DB; ++e)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d = 32 * e + 8 * r4 + 4 * hi;
                *reinterpret_cast<u32x2*>(ost + l32 * OSTR + d) =
                    pack4<E>(acc[e][4 * r4] * inv, acc[e][4 * r4 + 1] * inv,
                             acc[e][4 * r4 + 2] * inv, acc[e][4 * r4 + 3] * inv);
            }
        // the wave reads rows other lanes wrote: its writes land first
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int t = 0; t < 32 / RPI; ++t) {
            const int i = RPI * t + lane / T::CPR, c = lane % T::CPR;
            const u32x4 w = *reinterpret_cast<const u32x4*>(ost + i * OSTR + 8 * c);
            store16_nt(ob, ((uint32_t)row_of(i) * D + 8 * c) * 2, w);
        }
        // the next tile's loads refill the K buffers: every wave's reads first
        if (rep + 1 < ntiles) {
            __builtin_amdgcn_s_waitcnt(0xC07F);
            barrier_only();
        }
    }
    if (hi == 0) store4(SPLIT ? plb : lb, (uint32_t)qi * 4, __builtin_bit_cast(uint32_t, L));
    }  // query tiles of the unit
}

// Split key ranges, second step: per query row, L = ln sum_s exp(L_s) and
// O = sum_s exp(L_s - L) O_s (the running-softmax rule of tensortonic
// section 5 applied to whole key ranges).  One thread per 4 output columns.
template <typename E, int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* part_o, const float* part_l,
                                                    bf16* o, float* lse, int64_t rows,
                                                    int splits) {
    constexpr int TPR = D / 4;  // threads per row
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gid / TPR;
    const int c = (int)(gid % TPR);
    if (row >= rows) return;
    float m = kNegInf;
    for (int s = 0; s < splits; ++s) m = fmaxf(m, part_l[s * rows + row]);
    f32x4 acc{0.f, 0.f, 0.f, 0.f};
    float L = kNegInf;
    if (m != kNegInf) {  // some range had a readable key
        float sum = 0.f;
        for (int s = 0; s < splits; ++s) sum += exp2_fast((part_l[s * rows + row] - m) * kLog2e);
        const float inv = 1.f / sum;
        for (int s = 0; s < splits; ++s) {
            const float w = exp2_fast((part_l[s * rows + row] - m) * kLog2e) * inv;
            const f32x4 po = *reinterpret_cast<const f32x4*>(part_o + (s * rows + row) * D + 4 * c);
            acc += w * po;
        }
        L = m + log2_fast(sum) * kLn2;
    }
    *reinterpret_cast<u32x2*>(o + row * D + 4 * c) = pack4<E>(acc[0], acc[1], acc[2], acc[3]);
    if (lse && c == 0) lse[row] = L;
}

// ---- decoding: a handful of queries against a long key range ---------------
//
// With N_q <= 32 every (batch, head) has one query tile, so the forward tile
// of 128 rows would spend its matrix work on empty rows while the HBM stream
// of K and V is what bounds the call.  This kernel is shaped for that stream:
//  - the four waves of a workgroup take interleaved 32-key blocks of the
//    unit's key range (wave w: blocks w, w + 4, ...) and run independently,
//    with no barrier until the end;
//  - K and V blocks are read with wave-wide loads of 1 KiB of consecutive
//    rows into registers, two blocks ahead, so each CU keeps 128 KiB in
//    flight.  (Loading the MFMA operands themselves touches 32 rows per
//    load, 32 bytes each; alone, that pattern streams at about 3.8 TB/s.)
//    A block is then written into the wave's own LDS region, K rows padded
//    and V rows swizzled as in fwd_kernel, and read back as MFMA operands.
//    Every K/V byte is read exactly once, so the loads carry the
//    non-temporal hint: with it the stream reaches about 6.8 TB/s on this
//    workload, without it about 6.05 (filling the LDS by global->LDS DMA
//    measured the same as plain loads).
//  - at the end the waves' (m, l, u) are merged through LDS by the same
//    running-softmax rule, then O and L (or the range's partials) are stored.
template <int D>
struct DecTile {
    static constexpr int BK = 32;                 // keys per block
    static constexpr int CPR = D / 8;             // 16-byte chunks per row
    static constexpr int RPL = 64 / CPR;          // V rows per wave-wide load
    static constexpr int V_ELEMS = BK * D;        // one V block in LDS
    static constexpr int KSTR = D + 8;            // padded K row (see FwdTile)
    static constexpr int K_ELEMS = BK * KSTR;
    static constexpr int LOADS = BK * CPR / 64;   // wave-wide 1 KiB loads per K or V block
    static constexpr int DS = D / 16, DB = D / 32;
};

template <typename E, int D, bool CAUSAL, bool PART>
__global__ __launch_bounds__(256, 1) void decode_kernel(FwdParams p) {
    using T = DecTile<D>;
    // each wave's current K and V block
    __shared__ __attribute__((aligned(16))) bf16 k_st[4 * T::K_ELEMS];
    __shared__ __attribute__((aligned(16))) bf16 v_st[4 * T::V_ELEMS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5;
    const int g = lane >> 4, i16 = lane & 15;
    int head, split;
    unit_of(blockIdx.x, gridDim.x, p.splits, head, split);
    const int b = head / p.H, h = head - b * p.H;

    const int n = p.N;
    int nk = p.Nk;
    const int64_t row0 = ((int64_t)b * p.H + h) * n;
    const int64_t krow0 = ((int64_t)b * p.H + h) * p.Nk;
    int shift = nk - n;  // query i reads keys j <= i + shift (causal)
    const int kbeg = min(nk, split * p.chunk);
    nk = min(nk - kbeg, p.chunk);
    shift -= kbeg;
    // keys any query of the unit reads
    const int kend = CAUSAL ? max(0, min(nk, n + shift)) : nk;
    const int nblk = (kend + T::BK - 1) / T::BK;
    // this wave's blocks: wave, wave + 4, ...
    const int nb = nblk > wave ? (nblk - wave + 3) / 4 : 0;

    const uint32_t kbytes = (uint32_t)nk * D * 2;
    const Buf qb = make_buf(p.q + row0 * D, (uint32_t)n * D * 2);
    const Buf kb = make_buf(p.k + (krow0 + kbeg) * D, kbytes);
    const Buf vb = make_buf(p.v + (krow0 + kbeg) * D, kbytes);

    const int qi = l32;  // query held by this lane (rows >= n read zeros)
    bf16x8 qreg[T::DS];
#pragma unroll
    for (int s = 0; s < T::DS; ++s)
        qreg[s] = __builtin_bit_cast(bf16x8,
                                     load16(qb, ((uint32_t)qi * D + 16 * s + 8 * hi) * 2));

    // load t of a block brings rows RPL t + lane / CPR, chunk lane % CPR; the
    // lane stores its chunk at these LDS element offsets (row swizzle
    // depends on lane only, as RPL is a multiple of 4)
    const int lrow = lane / T::CPR, lch = lane % T::CPR;
    const uint32_t gofs = (uint32_t)(lrow * D + lch * 8) * 2;
    const int kls = lrow * T::KSTR + lch * 8;
    const int vls = lrow * D + ((lch ^ v_swz<D>(lrow)) * 8);
    static_assert(T::RPL % 4 == 0, "swizzle of row RPL t + r equals that of r");
    uint32_t voffb[T::DB];
#pragma unroll
    for (int e = 0; e < T::DB; ++e) {
        const int kr = 4 * hi + (i16 >> 2);
        const int dcol = 32 * e + 16 * (g & 1) + 4 * (i16 & 3);
        voffb[e] = (uint32_t)(kr * D + (((dcol >> 3) ^ v_swz<D>(kr)) << 3) + (dcol & 7)) * 2;
    }
    bf16* const kw = k_st + wave * T::K_ELEMS;
    bf16* const vw = v_st + wave * T::V_ELEMS;

    // block i of this wave: keys 32 * (wave + 4 i) .. of the range (rows
    // past the range read zeros).  Requests for blocks past the wave's last
    // are still issued, out of range (no memory access), so every step has
    // the same number of loads in flight and the compiler's waits stay exact.
    struct Blk {
        u32x4 k[T::LOADS], v[T::LOADS];
    };
    // Step i reads the wave's block (i + rot) mod nb.  With one range per
    // head every unit's stream would start at a head boundary and all of
    // them would move through the memory channels in lockstep; rotating the
    // start per unit measured 2-3 % faster.  Split ranges already start at
    // different offsets, and there the rotation measured slower, so it is
    // not applied.  (The order of the blocks changes the result only by
    // rounding.)
    const int rot = (p.splits == 1 && nb > 0)
                        ? (int)(((uint32_t)blockIdx.x * 5u) % (uint32_t)nb) : 0;
    auto phys = [&](int i) {
        const int r = i + rot;
        return wave + 4 * (r >= nb ? r - nb : r);
    };
    auto issue = [&](int i, Blk& r) {
        const uint32_t o = i < nb ? (uint32_t)phys(i) * T::BK * D * 2 + gofs : kOutOfRange;
#pragma unroll
        for (int t = 0; t < T::LOADS; ++t) r.k[t] = load16_nt(kb, o + t * 1024);
#pragma unroll
        for (int t = 0; t < T::LOADS; ++t) r.v[t] = load16_nt(vb, o + t * 1024);
    };
    // LDS reads of the previous block come first in the wave's LDS queue,
    // so the writes can follow them directly
    auto stage = [&](const Blk& r) {
#pragma unroll
        for (int t = 0; t < T::LOADS; ++t) {
            lds_write16(kw + kls + T::RPL * t * T::KSTR, r.k[t]);
            lds_write16(vw + vls + T::RPL * t * D, r.v[t]);
        }
    };

    f32x16 acc[T::DB];
#pragma unroll
    for (int e = 0; e < T::DB; ++e) acc[e] = f32x16{};
    float m_run = kNegInf, l_run = 0.f;

    auto block = [&](int i, const bf16* ks, const bf16* vs) {
        const int blk = phys(i);
        f32x16 s = f32x16{};
#pragma unroll
        for (int ss = 0; ss < T::DS; ++ss)
            s = mfma32<E>(lds_read16(ks + l32 * T::KSTR + 16 * ss + 8 * hi), qreg[ss], s);
        // mask keys past the range end or after the query's causal limit
        int lim = nk - T::BK * blk;
        if (CAUSAL) lim = min(lim, qi + shift - T::BK * blk + 1);
        if (lim < T::BK) {
            lim -= 4 * hi;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (8 * (r / 4) + (r & 3) >= lim) s[r] = kNegInf;
        }
        float mx = s[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = pair_max(mx) * p.c;
        const bool upd = mx > m_run + kLazyRescale;
        const float m_new = upd ? mx : m_run;
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = m_run - m_use;
        m_run = m_new;
        float rs[4];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s[r] = exp2_fast(__builtin_fmaf(s[r], p.c, -m_use));
            rs[r & 3] = r < 4 ? s[r] : rs[r & 3] + s[r];
        }
        const bf16x8 pb0 = pack8<E>(s, 0), pb1 = pack8<E>(s, 8);
        if (__any(upd)) {
            const float f = exp2_fast(alpha);
#pragma unroll
            for (int e = 0; e < T::DB; ++e) acc[e] *= f;
            l_run *= f;
        }
        l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);
#pragma unroll
        for (int bt = 0; bt < 2; ++bt)
#pragma unroll
            for (int e = 0; e < T::DB; ++e) {
                const char* vp = reinterpret_cast<const char*>(vs) + voffb[e] + 16 * bt * D * 2;
                const bf16x8 a = cat(lds_read_tr(reinterpret_cast<const bf16*>(vp)),
                                     lds_read_tr(reinterpret_cast<const bf16*>(vp + 8 * D * 2)));
                acc[e] = mfma32<E>(a, bt ? pb1 : pb0, acc[e]);
            }
    };

    // each step: block i's registers (loaded two steps before) go to LDS,
    // block i + 2 is requested into the same registers, block i is computed;
    // two steps per trip keep the register sets static
    Blk r0, r1;
    issue(0, r0);
    issue(1, r1);
    auto step = [&](int i, Blk& r) {
        stage(r);  // waits for block i's loads only
        issue(i + 2, r);
        block(i, kw, vw);
    };
    int i = 0;
    for (; i + 1 < nb; i += 2) {
        step(i, r0);
        step(i + 1, r1);
    }
    if (i < nb) step(i, r0);

    // ---- merge the four waves: stage (m, l, u) in LDS and let each thread
    //      combine some (query, 4 columns) items; u goes in two passes of half
    //      the columns, each filling one stage object --------------------------
    __syncthreads();  // every wave is done with its blocks
    constexpr int HD = D / 2;                             // columns per pass
    float* const cu_o = reinterpret_cast<float*>(v_st);   // [4][32][HD]
    float* const cm = reinterpret_cast<float*>(k_st);     // [4][32]
    float* const cl = cm + 4 * 32;                        // [4][32]
    static_assert(4 * 32 * HD * 4 <= 4 * T::V_ELEMS * 2, "half of u fits the V blocks");
    const float l_tot = pair_sum(l_run);
    if (hi == 0) {
        cm[wave * 32 + qi] = m_run;
        cl[wave * 32 + qi] = l_tot;
    }
    constexpr int TPR = HD / 4;  // items per query row and pass
    const int64_t prow0 = ((int64_t)split * p.heads + head) * n;
    const int nq = min(n, 32);
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int e = pass * T::DB / 2; e < (pass + 1) * T::DB / 2; ++e)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d = 32 * e + 8 * r4 + 4 * hi - pass * HD;
                *reinterpret_cast<f32x4*>(cu_o + (wave * 32 + qi) * HD + d) =
                    f32x4{acc[e][4 * r4], acc[e][4 * r4 + 1], acc[e][4 * r4 + 2],
                          acc[e][4 * r4 + 3]};
            }
        __syncthreads();
        for (int it = tid; it < nq * TPR; it += 256) {
            const int q = it / TPR, c = it - q * TPR;
            float M = kNegInf;
#pragma unroll
            for (int w = 0; w < 4; ++w) M = fmaxf(M, cm[w * 32 + q]);
            f32x4 o{0.f, 0.f, 0.f, 0.f};
            float lsum = 0.f;
            if (M != kNegInf) {
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float f = exp2_fast(cm[w * 32 + q] - M);  // 0 for an empty wave
                    lsum += f * cl[w * 32 + q];
                    o += f * *reinterpret_cast<const f32x4*>(cu_o + (w * 32 + q) * HD + 4 * c);
                }
            }
            const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
            o *= inv;
            const int col = pass * HD + 4 * c;
            if constexpr (PART) {
                *reinterpret_cast<f32x4*>(p.part_o + (prow0 + q) * D + col) = o;
            } else {
                *reinterpret_cast<u32x2*>(p.o + (row0 + q) * D + col) =
                    pack4<E>(o[0], o[1], o[2], o[3]);
            }
            if (pass == 0 && c == 0) {
                const float L = lsum > 0.f ? (M + log2_fast(lsum)) * kLn2 : kNegInf;
                if constexpr (PART) p.part_l[prow0 + q] = L;
                else if (p.lse) p.lse[row0 + q] = L;
            }
        }
        __syncthreads();  // the next pass overwrites the staged columns
    }
}

template <typename E, int D, bool CAUSAL>
hipError_t run_decode(const FwdArgs& a, hipStream_t stream) {
    FwdParams p{};
    p.q = static_cast<const bf16*>(a.q);
    p.k = static_cast<const bf16*>(a.k);
    p.v = static_cast<const bf16*>(a.v);
    p.o = static_cast<bf16*>(a.o);
    p.lse = a.lse;
    p.H = a.H;
    p.N = a.N;
    p.Nk = a.Nk;
    p.c = (float)((double)a.scale * 1.4426950408889634);
    p.splits = a.splits;
    p.chunk = a.splits > 1 ? a.chunk : a.Nk;
    p.heads = a.B * a.H;
    const int64_t rows = (int64_t)a.B * a.H * a.N;
    p.part_o = a.part;
    p.part_l = a.part ? a.part + ((rows * a.splits * D + 63) & ~(int64_t)63) : nullptr;
    const unsigned units = (unsigned)((int64_t)a.B * a.H * a.splits);
    if (a.splits > 1) {
        hipLaunchKernelGGL((decode_kernel<E, D, CAUSAL, true>), dim3(units), dim3(256), 0,
                           stream, p);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        const int64_t threads = rows * (D / 4);
        hipLaunchKernelGGL((merge_kernel<E, D>), dim3((unsigned)((threads + 255) / 256)),
                           dim3(256), 0, stream, p.part_o, p.part_l, p.o, p.lse, rows,
                           a.splits);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((decode_kernel<E, D, CAUSAL, false>), dim3(units), dim3(256), 0, stream,
                       p);
    return hipGetLastError();
}

template <typename E, int D, bool CAUSAL, bool VARLEN, bool SPLIT, bool DROP = false>
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
    p.Nk = a.Nk;
    const int n_qt = (a.max_seqlen + T::BR - 1) / T::BR;
    p.per_head = SPLIT ? n_qt * a.splits : CAUSAL ? (n_qt + 1) / 2 : n_qt;
    p.c = (float)((double)a.scale * 1.4426950408889634);
    p.splits = a.splits;
    p.chunk = a.chunk;
    p.heads = a.B * a.H;
    const int64_t rows = (int64_t)a.B * a.H * a.N;
    p.part_o = a.part;
    p.part_l = a.part + ((rows * a.splits * D + 63) & ~(int64_t)63);
    int64_t units = (int64_t)p.per_head * a.H * a.B;
    p.drop = a.drop;
    p.tail = 0;
    if (CAUSAL && !SPLIT && !VARLEN) {
        const FwdGrid grid = fwd_causal_grid(p.heads, n_qt);
        p.tail = grid.tail;
        units = grid.units;
    }
    hipLaunchKernelGGL((fwd_kernel<E, D, CAUSAL, VARLEN, SPLIT, DROP>), dim3((unsigned)units),
                       dim3(T::THREADS), 0, stream, p);
    if (!SPLIT) return hipGetLastError();
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t threads = rows * (D / 4);
    hipLaunchKernelGGL((merge_kernel<E, D>), dim3((unsigned)((threads + 255) / 256)), dim3(256),
                       0, stream, p.part_o, p.part_l, p.o, p.lse, rows, a.splits);
    return hipGetLastError();
}

template <typename E, int D>
hipError_t run_fwd_d(const FwdArgs& a, hipStream_t stream) {
    if (a.decode)
        return a.causal ? run_decode<E, D, true>(a, stream) : run_decode<E, D, false>(a, stream);
    const bool varlen = a.cu != nullptr;
    if (a.drop.thresh > 0) {  // dropout: dense batch or packed sequences
        if (varlen)
            return a.causal ? run_fwd<E, D, true, true, false, true>(a, stream)
                            : run_fwd<E, D, false, true, false, true>(a, stream);
        return a.causal ? run_fwd<E, D, true, false, false, true>(a, stream)
                        : run_fwd<E, D, false, false, false, true>(a, stream);
    }
    if (a.splits > 1)
        return a.causal ? run_fwd<E, D, true, false, true>(a, stream)
                        : run_fwd<E, D, false, false, true>(a, stream);
    if (a.causal)
        return varlen ? run_fwd<E, D, true, true, false>(a, stream)
                      : run_fwd<E, D, true, false, false>(a, stream);
    return varlen ? run_fwd<E, D, false, true, false>(a, stream)
                  : run_fwd<E, D, false, false, false>(a, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
    if (a.f16) return a.D == 64 ? run_fwd_d<f16, 64>(a, stream) : run_fwd_d<f16, 128>(a, stream);
    return a.D == 64 ? run_fwd_d<bf16, 64>(a, stream) : run_fwd_d<bf16, 128>(a, stream);
}

}  // namespace fa
