// fa_launch.hpp -- internal interface between the C ABI (fa_api.cpp) and the
// kernel launchers.  Arguments are already validated; every launcher returns
// the hipError_t of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Attention dropout parameters: generator seed and offset, drop threshold T
// (a decision byte below T drops the weight) and the scale of kept weights.
struct Dropout {
    uint32_t seed_lo, seed_hi, offset;
    uint32_t thresh;   // T in [0, 255]; 0 = no dropout
    float inv_keep;    // 256 / (256 - T)
};

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;             // may be null
    const int32_t* cu;      // packed offsets (varlen) or null (dense)
    int B;                  // batch (dense) or number of sequences (varlen)
    int H;
    int N;                  // queries per sequence (dense) or packed total
    int max_seqlen;         // longest sequence (== N when dense)
    int D;
    float scale;
    bool causal;
    int Nk;                 // keys per sequence (dense; == N when square)
    int splits = 1;         // > 1: key ranges split across units (dense only)
    int chunk = 0;          // keys per split, a multiple of 64
    float* part = nullptr;  // split workspace: partial O, then partial L (fp32)
    bool f16 = false;       // element type: bf16, or fp16 when set
    Dropout drop{};         // thresh 0: no dropout
    bool decode = false;    // N <= 32 queries per (batch, head): decoding kernel
};

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const float* lse;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    float* ws;              // workspace: two fp32 [B, H, N] regions, each
                            // padded to 256 bytes (D_i, then -L_i log2 e)
    int B, H, N, D;         // varlen: B = number of sequences, N = packed total
    float scale;
    bool causal;
    bool f16 = false;       // element type: bf16, or fp16 when set
    Dropout drop{};         // thresh 0: no dropout
    const int32_t* cu = nullptr;  // packed offsets [B + 1] (varlen) or null (dense)
    int max_seqlen = 0;     // longest sequence (varlen)
};

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);

// Size of the static device scratch behind fa_bwd_noalloc: the backward
// workspace of up to 2^21 query rows (B * H * N), two padded fp32 regions.
constexpr size_t kBwdScratchBytes = (size_t)16 << 20;
// Device address of that scratch on the current device (looked up once per
// device, then cached).
hipError_t bwd_scratch(float** ptr);

}  // namespace fa
