// sanitize_check.cpp -- host-only driver for an AddressSanitizer and
// UndefinedBehaviorSanitizer build of the two pieces of host code that
// handle untrusted sizes and pointers: the oracle (oracle/oracle.c) and the
// C ABI's argument validation (exact_io_aware_44_amd/csrc/fa_api.cpp).
//
// The kernel launchers are replaced by counters: the ABI part checks that
// every entry point rejects each invalid argument with its documented status
// and reaches exactly one launch for valid arguments (stand-in device
// addresses, never dereferenced), including at extreme int sizes where
// unchecked arithmetic would overflow.  The oracle part runs every oracle
// function on small inputs and checks results fixed by the mathematics
// (constant values return themselves, causal row 0 returns v_0, gradients of
// keys sum to zero, sampled rows equal full rows, the published Philox
// vectors).  Any sanitizer report aborts the run with a non-zero status.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "fa.h"
#include "fa_launch.hpp"

namespace fa {
static int g_fwd_calls = 0, g_bwd_calls = 0;
hipError_t launch_fwd(const FwdArgs& a, hipStream_t) {
    // read every field the launchers read, so uninitialised or out-of-range
    // values surface under the sanitizers
    volatile int64_t sink = (int64_t)a.B + a.H + a.N + a.max_seqlen + a.D + a.Nk + a.splits +
                            a.chunk + a.causal + a.f16 + a.decode + a.drop.thresh;
    (void)sink;
    if (a.B < 1 || a.H < 1 || a.N < 1 || a.Nk < 1 || a.max_seqlen < 1 || a.max_seqlen > a.N)
        std::abort();
    ++g_fwd_calls;
    return hipSuccess;
}
hipError_t bwd_scratch(float** ptr) {  // stand-in address, never dereferenced
    *ptr = reinterpret_cast<float*>(0x40000);
    return hipSuccess;
}
hipError_t launch_bwd(const BwdArgs& a, hipStream_t) {
    volatile int64_t sink = (int64_t)a.B + a.H + a.N + a.D + a.causal + a.f16 + a.drop.thresh +
                            a.max_seqlen;
    (void)sink;
    if (a.B < 1 || a.H < 1 || a.N < 1) std::abort();
    ++g_bwd_calls;
    return hipSuccess;
}
}  // namespace fa

extern "C" {
int oracle_attn_fwd(const double*, const double*, const double*, double*, double*, int64_t,
                    int64_t, int64_t, int64_t, double, int);
int oracle_attn_fwd_rows(const double*, const double*, const double*, const int64_t*,
                         const int64_t*, int64_t, double*, double*, int64_t, int64_t, int64_t,
                         int64_t, double, int);
int oracle_attn_fwd_qk(const double*, const double*, const double*, double*, double*, int64_t,
                       int64_t, int64_t, int64_t, int64_t, double, int);
int oracle_attn_fwd_qk_rows(const double*, const double*, const double*, const int64_t*,
                            const int64_t*, int64_t, double*, double*, int64_t, int64_t,
                            int64_t, int64_t, int64_t, double, int);
int oracle_attn_fwd_varlen(const double*, const double*, const double*, double*, double*,
                           const int32_t*, int64_t, int64_t, int64_t, int64_t, double, int);
int oracle_attn_fwd_varlen_rows(const double*, const double*, const double*, const int32_t*,
                                int64_t, int64_t, int64_t, int64_t, double, int,
                                const int64_t*, const int64_t*, int64_t, double*, double*);
int oracle_attn_bwd(const double*, const double*, const double*, const double*, double*,
                    double*, double*, int64_t, int64_t, int64_t, int64_t, double, int);
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
int oracle_dropout_threshold(double p);
int oracle_dropout_mask(uint8_t*, int64_t, int64_t, int64_t, double, uint64_t, uint64_t);
int oracle_attn_fwd_dropout(const double*, const double*, const double*, double*, double*,
                            int64_t, int64_t, int64_t, int64_t, double, int, double, uint64_t,
                            uint64_t);
int oracle_attn_bwd_dropout(const double*, const double*, const double*, const double*,
                            double*, double*, double*, int64_t, int64_t, int64_t, int64_t,
                            double, int, double, uint64_t, uint64_t);
}

static int g_fail = 0;
#define CHECK(cond)                                                           \
    do {                                                                      \
        if (!(cond)) {                                                        \
            std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__,       \
                         __LINE__, #cond);                                    \
            ++g_fail;                                                         \
        }                                                                     \
    } while (0)

// ---------------------------------------------------------------- ABI part --
static void* const P = reinterpret_cast<void*>(0x10000);   // aligned stand-in
static void* const PM = reinterpret_cast<void*>(0x10008);  // misaligned by 8
static float* const F = reinterpret_cast<float*>(0x20000);
static const int32_t* const CU = reinterpret_cast<const int32_t*>(0x30000);
static hipStream_t const S = nullptr;

static void abi_forward() {
    const int calls0 = fa::g_fwd_calls;
    CHECK(fa_fwd(P, P, P, P, F, 2, 3, 200, 128, 0.1f, 1, S) == FA_OK);
    CHECK(fa_fwd(P, P, P, P, nullptr, 1, 1, 1, 64, 0.1f, 0, S) == FA_OK);
    CHECK(fa_fwd_f16(P, P, P, P, F, 1, 1, 77, 64, 0.1f, 0, S) == FA_OK);
    CHECK(fa::g_fwd_calls == calls0 + 3);
    CHECK(fa_fwd(nullptr, P, P, P, F, 1, 1, 8, 64, 0.1f, 0, S) == FA_ERR_NULL);
    CHECK(fa_fwd(P, P, P, nullptr, F, 1, 1, 8, 64, 0.1f, 0, S) == FA_ERR_NULL);
    CHECK(fa_fwd(P, P, P, P, F, 0, 1, 8, 64, 0.1f, 0, S) == FA_ERR_SHAPE);
    CHECK(fa_fwd(P, P, P, P, F, 1, 0, 8, 64, 0.1f, 0, S) == FA_ERR_SHAPE);
    CHECK(fa_fwd(P, P, P, P, F, 1, 1, 0, 64, 0.1f, 0, S) == FA_ERR_SHAPE);
    CHECK(fa_fwd(P, P, P, P, F, INT_MIN, INT_MIN, INT_MIN, 64, 0.1f, 0, S) == FA_ERR_SHAPE);
    CHECK(fa_fwd(P, P, P, P, F, 1, 1, 8, 96, 0.1f, 0, S) == FA_ERR_UNSUPPORTED);
    CHECK(fa_fwd(P, P, P, P, F, 1, 1, 8, 64, 0.1f, 2, S) == FA_ERR_UNSUPPORTED);
    CHECK(fa_fwd(P, P, P, P, F, 1, 1, 8, 64, NAN, 0, S) == FA_ERR_ARG);
    CHECK(fa_fwd(P, P, P, P, F, 1, 1, 8, 64, INFINITY, 0, S) == FA_ERR_ARG);
    CHECK(fa_fwd(P, P, P, P, F, 1, 1, 8, 64, -1.f, 0, S) == FA_ERR_ARG);
    CHECK(fa_fwd(PM, P, P, P, F, 1, 1, 8, 64, 0.1f, 0, S) == FA_ERR_ALIGN);
    CHECK(fa_fwd(P, P, P, P, reinterpret_cast<float*>(PM), 1, 1, 8, 64, 0.1f, 0, S) ==
          FA_ERR_ALIGN);
    CHECK(fa_fwd(P, P, P, P, F, 1, 1, INT_MAX, 128, 0.1f, 0, S) == FA_ERR_TOO_LARGE);
    CHECK(fa_fwd(P, P, P, P, F, INT_MAX, INT_MAX, 8, 64, 0.1f, 0, S) == FA_ERR_SHAPE);
    CHECK(fa_fwd_dropout(P, P, P, P, F, 1, 2, 64, 64, 0.1f, 1, 0.25f, 7, 9, S) == FA_OK);
    CHECK(fa_fwd_dropout(P, P, P, P, F, 1, 2, 64, 64, 0.1f, 1, 1.0f, 7, 9, S) == FA_ERR_ARG);
    CHECK(fa_fwd_dropout(P, P, P, P, F, 1, 2, 64, 64, 0.1f, 1, -0.1f, 7, 9, S) == FA_ERR_ARG);
    CHECK(fa_fwd_dropout(P, P, P, P, F, 1, 2, 64, 64, 0.1f, 1, NAN, 7, 9, S) == FA_ERR_ARG);
    CHECK(fa_fwd_dropout_f16(P, P, P, P, F, 1, 2, 64, 64, 0.1f, 1, 0.5f, UINT64_MAX,
                             UINT64_MAX, S) == FA_OK);

    CHECK(fa_fwd_qk(P, P, P, P, F, 1, 2, 100, 333, 64, 0.1f, 1, S) == FA_OK);
    CHECK(fa_fwd_qk_f16(P, P, P, P, F, 1, 2, 333, 100, 128, 0.1f, 1, S) == FA_OK);
    CHECK(fa_fwd_qk(P, P, P, P, F, 1, 2, 100, 0, 64, 0.1f, 1, S) == FA_ERR_SHAPE);
    CHECK(fa_fwd_qk(P, P, P, P, F, 1, 2, 100, INT_MAX, 64, 0.1f, 1, S) == FA_ERR_TOO_LARGE);
    CHECK(fa_fwd_qk(P, P, P, P, F, 1, 2, INT_MAX, 100, 64, 0.1f, 1, S) == FA_ERR_TOO_LARGE);

    CHECK(fa_fwd_varlen(P, P, P, P, F, CU, 3, 500, 300, 2, 128, 0.1f, 1, S) == FA_OK);
    CHECK(fa_fwd_varlen(P, P, P, P, F, CU, 3, 500, INT_MAX, 2, 128, 0.1f, 1, S) == FA_OK);
    CHECK(fa_fwd_varlen_f16(P, P, P, P, nullptr, CU, 1, 1, 1, 1, 64, 0.1f, 0, S) == FA_OK);
    CHECK(fa_fwd_varlen_dropout(P, P, P, P, F, CU, 3, 500, 300, 2, 128, 0.1f, 1, 0.1f, 1, 2,
                                S) == FA_OK);
    CHECK(fa_fwd_varlen_dropout_f16(P, P, P, P, F, CU, 3, 500, 300, 2, 128, 0.1f, 1, 0.1f, 1,
                                    2, S) == FA_OK);
    CHECK(fa_fwd_varlen(P, P, P, P, F, nullptr, 3, 500, 300, 2, 128, 0.1f, 1, S) ==
          FA_ERR_NULL);
    CHECK(fa_fwd_varlen(P, P, P, P, F, CU, 0, 500, 300, 2, 128, 0.1f, 1, S) == FA_ERR_SHAPE);
    CHECK(fa_fwd_varlen(P, P, P, P, F, CU, 65536, 500, 300, 2, 128, 0.1f, 1, S) ==
          FA_ERR_SHAPE);
    CHECK(fa_fwd_varlen(P, P, P, P, F, CU, 3, INT_MAX, 300, 2, 128, 0.1f, 1, S) ==
          FA_ERR_TOO_LARGE);
    CHECK(fa_fwd_varlen(P, P, P, P, F, CU + 1, 3, 500, 300, 2, 128, 0.1f, 1, S) == FA_OK);
    CHECK(fa_fwd_varlen(P, P, P, P, F, reinterpret_cast<const int32_t*>(0x30002), 3, 500, 300,
                        2, 128, 0.1f, 1, S) == FA_ERR_ALIGN);
}

static void abi_splitkv() {
    // workspace sizes over a grid that includes the extreme ints
    const int vals[] = {INT_MIN, -1, 0, 1, 31, 32, 33, 64, 700, 16384, 1 << 24, INT_MAX};
    for (int b : vals)
        for (int nq : vals)
            for (int nk : vals)
                for (int s : {-1, 0, 1, 3, 1000, INT_MAX}) {
                    const size_t w = fa_fwd_splitkv_workspace_size(b, 2, nq, nk, 128, s);
                    if (b < 1 || nq < 1 || nk < 1 || s < 0) CHECK(w == 0);
                }
    for (int n : vals) {
        const size_t w = fa_bwd_workspace_size(2, 3, n, 64);
        if (n < 1 || ((int64_t)n + 256) * 64 * 2 >= ((int64_t)1 << 31)) CHECK(w == 0);
        else CHECK(w >= (size_t)2 * 2 * 3 * (size_t)n * sizeof(float));
        (void)fa_bwd_workspace_size(n, n, n, 128);  // must not overflow
    }
    CHECK(fa_bwd_workspace_size(1, 1, 8, 96) == 0);

    const int calls0 = fa::g_fwd_calls;
    const size_t need = fa_fwd_splitkv_workspace_size(1, 2, 3, 700, 128, 3);
    CHECK(need > 0);
    CHECK(fa_fwd_splitkv(P, P, P, P, F, P, need, 1, 2, 3, 700, 128, 0.1f, 1, 3, S) == FA_OK);
    CHECK(fa_fwd_splitkv(P, P, P, P, F, P, need - 1, 1, 2, 3, 700, 128, 0.1f, 1, 3, S) ==
          FA_ERR_WORKSPACE);
    CHECK(fa_fwd_splitkv(P, P, P, P, F, nullptr, need, 1, 2, 3, 700, 128, 0.1f, 1, 3, S) ==
          FA_ERR_WORKSPACE);
    CHECK(fa_fwd_splitkv(P, P, P, P, F, PM, need, 1, 2, 3, 700, 128, 0.1f, 1, 3, S) ==
          FA_ERR_ALIGN);
    CHECK(fa_fwd_splitkv(P, P, P, P, F, P, need, 1, 2, 3, 700, 128, 0.1f, 1, -1, S) ==
          FA_ERR_ARG);
    CHECK(fa_fwd_splitkv(P, P, P, P, F, nullptr, 0, 1, 2, 3, 700, 128, 0.1f, 1, 1, S) == FA_OK);
    const size_t need2 = fa_fwd_splitkv_workspace_size(1, 2, 40, 700, 64, 0);
    CHECK(fa_fwd_splitkv_f16(P, P, P, P, F, P, need2, 1, 2, 40, 700, 64, 0.1f, 0, 0, S) ==
          FA_OK);
    CHECK(fa_fwd_splitkv(P, P, P, P, F, P, SIZE_MAX, 1, 1, 1, INT_MAX, 128, 0.1f, 1, 0, S) ==
          FA_ERR_TOO_LARGE);
    CHECK(fa::g_fwd_calls == calls0 + 3);
}

static void abi_backward() {
    const int calls0 = fa::g_bwd_calls;
    const size_t ws = fa_bwd_workspace_size(2, 3, 200, 128);
    CHECK(fa_bwd(P, P, P, P, F, P, P, P, P, P, ws, 2, 3, 200, 128, 0.1f, 1, S) == FA_OK);
    CHECK(fa_bwd_f16(P, P, P, P, F, P, P, P, P, P, ws, 2, 3, 200, 128, 0.1f, 0, S) == FA_OK);
    CHECK(fa_bwd_dropout(P, P, P, P, F, P, P, P, P, P, ws, 2, 3, 200, 128, 0.1f, 1, 0.3f, 5, 6,
                         S) == FA_OK);
    CHECK(fa_bwd_dropout_f16(P, P, P, P, F, P, P, P, P, P, ws, 2, 3, 200, 128, 0.1f, 1, 0.3f, 5,
                             6, S) == FA_OK);
    CHECK(fa::g_bwd_calls == calls0 + 4);
    CHECK(fa_bwd(P, P, P, P, F, P, P, P, P, P, ws - 1, 2, 3, 200, 128, 0.1f, 1, S) ==
          FA_ERR_WORKSPACE);
    CHECK(fa_bwd(P, P, P, P, F, P, P, P, P, nullptr, ws, 2, 3, 200, 128, 0.1f, 1, S) ==
          FA_ERR_WORKSPACE);
    CHECK(fa_bwd(P, P, P, P, F, P, P, P, P, PM, ws, 2, 3, 200, 128, 0.1f, 1, S) == FA_ERR_ALIGN);
    CHECK(fa_bwd(P, P, P, P, nullptr, P, P, P, P, P, ws, 2, 3, 200, 128, 0.1f, 1, S) ==
          FA_ERR_NULL);
    CHECK(fa_bwd(P, P, P, P, F, P, P, P, PM, P, ws, 2, 3, 200, 128, 0.1f, 1, S) == FA_ERR_ALIGN);
    CHECK(fa_bwd(P, P, P, P, F, P, P, P, P, P, SIZE_MAX, 1, 1, INT_MAX, 128, 0.1f, 1, S) ==
          FA_ERR_TOO_LARGE);
    CHECK(fa_bwd(P, P, P, P, F, P, P, P, P, P, SIZE_MAX, INT_MAX, INT_MAX, 8, 128, 0.1f, 1, S) ==
          FA_ERR_SHAPE);
    CHECK(fa_bwd_dropout(P, P, P, P, F, P, P, P, P, P, ws, 2, 3, 200, 128, 0.1f, 1, 2.f, 5, 6,
                         S) == FA_ERR_ARG);

    const size_t wsv = fa_bwd_workspace_size(1, 2, 500, 64);
    CHECK(fa_bwd_varlen(P, P, P, P, F, P, P, P, P, CU, 3, 500, 300, P, wsv, 2, 64, 0.1f, 1, S) ==
          FA_OK);
    CHECK(fa_bwd_varlen_f16(P, P, P, P, F, P, P, P, P, CU, 3, 500, INT_MAX, P, wsv, 2, 64, 0.1f,
                            1, S) == FA_OK);
    CHECK(fa_bwd_varlen_dropout(P, P, P, P, F, P, P, P, P, CU, 3, 500, 300, P, wsv, 2, 64, 0.1f,
                                1, 0.2f, 1, 1, S) == FA_OK);
    CHECK(fa_bwd_varlen_dropout_f16(P, P, P, P, F, P, P, P, P, CU, 3, 500, 300, P, wsv, 2, 64,
                                    0.1f, 1, 0.2f, 1, 1, S) == FA_OK);
    CHECK(fa_bwd_varlen(P, P, P, P, F, P, P, P, P, CU, 3, 500, 300, P, wsv - 1, 2, 64, 0.1f, 1,
                        S) == FA_ERR_WORKSPACE);
    CHECK(fa_bwd_varlen(P, P, P, P, F, P, P, P, P, nullptr, 3, 500, 300, P, wsv, 2, 64, 0.1f, 1,
                        S) == FA_ERR_NULL);
    CHECK(fa_bwd_varlen(P, P, P, P, F, P, P, P, P, CU, 3, INT_MAX, 300, P, SIZE_MAX, 2, 64, 0.1f,
                        1, S) == FA_ERR_TOO_LARGE);
    CHECK(fa::g_bwd_calls == calls0 + 8);
    const int calls1 = fa::g_bwd_calls;
    CHECK(fa_bwd_noalloc(P, P, P, P, F, P, P, P, P, 2, 32, 32768, 128, 0.1f, 1, S) == FA_OK);
    CHECK(fa_bwd_noalloc(P, P, P, P, F, P, P, P, P, 2, 32, 32769, 128, 0.1f, 1, S) ==
          FA_ERR_SCRATCH);
    CHECK(fa_bwd_noalloc(P, P, P, P, F, P, P, P, P, 65535, 65535, 8, 64, 0.1f, 1, S) ==
          FA_ERR_SCRATCH);
    CHECK(fa_bwd_noalloc(P, P, P, P, F, P, P, P, P, INT_MAX, 1, 8, 64, 0.1f, 1, S) ==
          FA_ERR_SHAPE);
    CHECK(fa_bwd_noalloc(P, P, P, P, F, P, P, P, P, 1, 1, INT_MAX, 64, 0.1f, 1, S) ==
          FA_ERR_TOO_LARGE);
    CHECK(fa_bwd_noalloc(P, P, P, nullptr, F, P, P, P, P, 1, 1, 8, 64, 0.1f, 1, S) ==
          FA_ERR_NULL);
    CHECK(fa::g_bwd_calls == calls1 + 1);
    for (int st = -3; st < 12; ++st) CHECK(fa_status_string(st) != nullptr);
}

// ------------------------------------------------------------- oracle part --
static uint64_t g_rng = 0x9E3779B97F4A7C15ull;
static double urand() {  // uniform in [-1, 1): a 64-bit LCG, top 53 bits
    g_rng = g_rng * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(g_rng >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}
static std::vector<double> randv(size_t n) {
    std::vector<double> x(n);
    for (auto& e : x) e = urand();
    return x;
}

static void oracle_forward() {
    const int64_t B = 2, H = 2, N = 37, D = 8;
    const size_t n = (size_t)(B * H * N * D);
    std::vector<double> q = randv(n), k = randv(n), v = randv(n), o(n), l(B * H * N);
    for (int causal = 0; causal < 2; ++causal) {
        // constant values return themselves
        std::vector<double> vc(n, 0.75), oc(n);
        CHECK(oracle_attn_fwd(q.data(), k.data(), vc.data(), oc.data(), l.data(), B, H, N, D,
                              0.5, causal) == 0);
        for (double x : oc) CHECK(std::fabs(x - 0.75) < 1e-14);
        CHECK(oracle_attn_fwd(q.data(), k.data(), v.data(), o.data(), l.data(), B, H, N, D, 0.5,
                              causal) == 0);
        if (causal) {  // row 0 reads key 0 alone
            for (int64_t bh = 0; bh < B * H; ++bh)
                for (int64_t d = 0; d < D; ++d)
                    CHECK(o[bh * N * D + d] == v[bh * N * D + d]);
        }
        // sampled rows equal the full rows
        const int64_t bh[] = {0, 3, 1, 2}, row[] = {0, 36, 17, 5};
        std::vector<double> orow(4 * D), lrow(4);
        CHECK(oracle_attn_fwd_rows(q.data(), k.data(), v.data(), bh, row, 4, orow.data(),
                                   lrow.data(), B, H, N, D, 0.5, causal) == 0);
        for (int t = 0; t < 4; ++t) {
            CHECK(std::fabs(lrow[t] - l[bh[t] * N + row[t]]) < 1e-13);
            for (int64_t d = 0; d < D; ++d)
                CHECK(std::fabs(orow[t * D + d] - o[(bh[t] * N + row[t]) * D + d]) < 1e-13);
        }
        // equal lengths through the unequal-length entry
        std::vector<double> o2(n), l2(B * H * N);
        CHECK(oracle_attn_fwd_qk(q.data(), k.data(), v.data(), o2.data(), l2.data(), B, H, N, N,
                                 D, 0.5, causal) == 0);
        for (size_t i = 0; i < n; ++i) CHECK(std::fabs(o2[i] - o[i]) < 1e-13);
        // more queries than keys (rows with no key under the causal mask)
        const int64_t Nq = 40, Nk = 9;
        std::vector<double> qq = randv((size_t)(B * H * Nq * D)), kk = randv((size_t)(B * H * Nk * D)),
                            vv = randv((size_t)(B * H * Nk * D)), oq((size_t)(B * H * Nq * D)),
                            lq((size_t)(B * H * Nq));
        CHECK(oracle_attn_fwd_qk(qq.data(), kk.data(), vv.data(), oq.data(), lq.data(), B, H, Nq,
                                 Nk, D, 0.5, causal) == 0);
        const int64_t qb[] = {0, 3}, qr[] = {39, 0};
        std::vector<double> oqr(2 * D), lqr(2);
        CHECK(oracle_attn_fwd_qk_rows(qq.data(), kk.data(), vv.data(), qb, qr, 2, oqr.data(),
                                      lqr.data(), B, H, Nq, Nk, D, 0.5, causal) == 0);
        CHECK(std::fabs(lqr[0] - lq[qb[0] * Nq + qr[0]]) < 1e-13);
    }
}

static void oracle_packed() {
    const int64_t H = 2, D = 8;
    const int32_t cu[] = {0, 13, 13, 40, 41};  // lengths 13, 0, 27, 1
    const int64_t nseq = 4, total = 41;
    const size_t n = (size_t)(H * total * D);
    std::vector<double> q = randv(n), k = randv(n), v = randv(n), o(n), l(H * total);
    for (int causal = 0; causal < 2; ++causal) {
        CHECK(oracle_attn_fwd_varlen(q.data(), k.data(), v.data(), o.data(), l.data(), cu, nseq,
                                     H, total, D, 0.25, causal) == 0);
        // the one-token sequence reads only itself
        for (int64_t h = 0; h < H; ++h)
            for (int64_t d = 0; d < D; ++d)
                CHECK(o[(h * total + 40) * D + d] == v[(h * total + 40) * D + d]);
        const int64_t hh[] = {0, 1, 1}, tok[] = {0, 40, 20};
        std::vector<double> orow(3 * D), lrow(3);
        CHECK(oracle_attn_fwd_varlen_rows(q.data(), k.data(), v.data(), cu, nseq, H, total, D,
                                          0.25, causal, hh, tok, 3, orow.data(),
                                          lrow.data()) == 0);
        for (int t = 0; t < 3; ++t) CHECK(std::fabs(lrow[t] - l[hh[t] * total + tok[t]]) < 1e-13);
    }
    const int32_t bad[] = {0, 20, 10, 41};  // decreasing offsets are rejected
    CHECK(oracle_attn_fwd_varlen(q.data(), k.data(), v.data(), o.data(), l.data(), bad, 3, H,
                                 total, D, 0.25, 1) != 0);
}

static void oracle_backward() {
    const int64_t B = 1, H = 2, N = 19, D = 4;
    const size_t n = (size_t)(B * H * N * D);
    std::vector<double> q = randv(n), k = randv(n), v = randv(n), dout = randv(n);
    std::vector<double> dq(n), dk(n), dv(n), dq2(n), dk2(n), dv2(n), o(n), l(B * H * N);
    for (int causal = 0; causal < 2; ++causal) {
        CHECK(oracle_attn_bwd(q.data(), k.data(), v.data(), dout.data(), dq.data(), dk.data(),
                              dv.data(), B, H, N, D, 0.7, causal) == 0);
        for (int64_t bh = 0; bh < B * H; ++bh)
            for (int64_t d = 0; d < D; ++d) {
                double sk = 0, sv = 0, so = 0;
                for (int64_t j = 0; j < N; ++j) {
                    sk += dk[(bh * N + j) * D + d];
                    sv += dv[(bh * N + j) * D + d];
                    so += dout[(bh * N + j) * D + d];
                }
                CHECK(std::fabs(sk) < 1e-12);       // softmax is shift invariant in k
                CHECK(std::fabs(sv - so) < 1e-12);  // rows of P sum to one
            }
        // dropout with p = 0 is the plain attention, bit for bit
        CHECK(oracle_attn_fwd_dropout(q.data(), k.data(), v.data(), o.data(), l.data(), B, H, N,
                                      D, 0.7, causal, 0.0, 1, 2) == 0);
        CHECK(oracle_attn_bwd_dropout(q.data(), k.data(), v.data(), dout.data(), dq2.data(),
                                      dk2.data(), dv2.data(), B, H, N, D, 0.7, causal, 0.0, 1,
                                      2) == 0);
        for (size_t i = 0; i < n; ++i) CHECK(dq2[i] == dq[i] && dk2[i] == dk[i] && dv2[i] == dv[i]);
        CHECK(oracle_attn_bwd_dropout(q.data(), k.data(), v.data(), dout.data(), dq2.data(),
                                      dk2.data(), dv2.data(), B, H, N, D, 0.7, causal, 0.3, 1,
                                      2) == 0);
        CHECK(oracle_attn_fwd_dropout(q.data(), k.data(), v.data(), o.data(), l.data(), B, H, N,
                                      D, 0.7, causal, 0.3, 1, 2) == 0);
    }
}

static void oracle_generator() {
    const uint32_t kat[3][10] = {
        {0, 0, 0, 0, 0, 0, 0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8},
        {0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff, 0x408f276d,
         0x41c83b0e, 0xa20bc7c6, 0x6d5451fd},
        {0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344, 0xa4093822, 0x299f31d0, 0xd16cfe09,
         0x94fdcceb, 0x5001e420, 0x24126ea1}};
    for (const auto& t : kat) {
        uint32_t out[4];
        oracle_philox4x32_10(t, t + 4, out);
        for (int i = 0; i < 4; ++i) CHECK(out[i] == t[6 + i]);
    }
    CHECK(oracle_dropout_threshold(0.0) == 0 && oracle_dropout_threshold(0.999) == 255);
    std::vector<uint8_t> m(33 * 70);
    CHECK(oracle_dropout_mask(m.data(), 5, 33, 70, 0.4, UINT64_MAX, 12) == 0);
    long kept = 0;
    for (uint8_t x : m) kept += x;
    CHECK(kept > 0 && kept < (long)m.size());
}

int main() {
    abi_forward();
    abi_splitkv();
    abi_backward();
    oracle_forward();
    oracle_packed();
    oracle_backward();
    oracle_generator();
    if (g_fail) {
        std::fprintf(stderr, "%d checks failed\n", g_fail);
        return 1;
    }
    std::printf("sanitize ok: %d forward and %d backward launches reached\n", fa::g_fwd_calls,
                fa::g_bwd_calls);
    return 0;
}
