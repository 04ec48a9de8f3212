// fa_device.hpp -- device-side building blocks for the gfx950 attention
// kernels: vector types, range-checked buffer loads/stores, the bf16 MFMA and
// the LDS transpose read.
//
// Register layouts used throughout (verified on gfx950 with an in-bounds
// probe of the builtins):
//
//   v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//     A: lane l holds A[l % 32][8*(l/32) + j],          j = 0..7
//     B: lane l holds B[8*(l/32) + j][l % 32],          j = 0..7
//     D: lane l, register r holds D[8*(r/4) + 4*(l/32) + r%4][l % 32]
//
//   ds_read_b64_tr_b16 (per 16-lane group; lane i of the group supplies an
//   address of four 16-bit values c_i[0..3]):
//     lane l receives { c_{4j + (l%16)/4}[l % 4] : j = 0..3 }
//   So if lane i addresses row R + i/4, column C + 4*(i%4) of a row-major
//   bf16 matrix, lane l receives the column C + l%16 of rows R..R+3: a
//   row-major tile becomes a column-major MFMA operand without a transposed
//   copy in LDS.
//
//   buffer_load_dwordx4 ... lds: lane i writes its 16 bytes at M0 + 16*i.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_launch.hpp"  // Dropout
#include "fa_schedule.hpp"

namespace fa {

// 16-bit elements travel (global, LDS, registers) as bf16-typed vectors; the
// element type E (bf16 or f16) only matters where they are computed with:
// the MFMA and the rounding of fp32 values to 16 bits.
typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// ---- range-checked buffer access ------------------------------------------
// A buffer resource covers [base, base + bytes); loads outside return zero and
// stores outside are dropped, which handles ragged tiles without branches.
struct Buf {
    __amdgpu_buffer_rsrc_t r;
};

__device__ __forceinline__ Buf make_buf(const void* base, uint32_t bytes) {
    // word 3 = 0x00020000: raw 32-bit dword format for the gfx9 family
    return Buf{__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base),
                                                 (short)0, (int)bytes,
                                                 0x00020000)};
}

__device__ __forceinline__ u32x4 load16(Buf b, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(b.r, off, 0, 0);
}
// Cache-policy bit of a buffer access: nt (non-temporal), for data read or
// written once, so it does not displace lines that other units re-read.
constexpr int kNonTemporal = 2;
__device__ __forceinline__ u32x4 load16_nt(Buf b, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(b.r, off, 0, kNonTemporal);
}
__device__ __forceinline__ void store16(Buf b, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, b.r, off, 0, 0);
}
__device__ __forceinline__ void store16_nt(Buf b, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, b.r, off, 0, kNonTemporal);
}
__device__ __forceinline__ void store8(Buf b, uint32_t off, u32x2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, b.r, off, 0, 0);
}
__device__ __forceinline__ void store4(Buf b, uint32_t off, uint32_t v) {
    __builtin_amdgcn_raw_buffer_store_b32(v, b.r, off, 0, 0);
}
// Direct global -> LDS load (buffer_load_dwordx4 ... lds): lane i of the wave
// writes its 16 bytes to lds_wave_base + 16*i (the base must be wave-uniform;
// it goes to M0).  Out-of-range lanes write zeros and fetch nothing.
__device__ __forceinline__ void load16_lds(Buf b, uint32_t off, void* lds_wave_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(b.r, (FA_LDS void*)lds_wave_base, 16, off,
                                             0, 0, 0);
}
// Offset that is out of range for every buffer (all buffers are < 2 GiB).
constexpr uint32_t kOutOfRange = 0x80000000u;
// s_waitcnt vmcnt(0) only (gfx9 encoding: expcnt and lgkmcnt left at max).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier without the release/acquire fences of __syncthreads: the
// caller has already waited (s_waitcnt) for whatever other waves must see,
// e.g. tiles DMA-loaded into LDS.  The memory clobber keeps the compiler from
// moving memory accesses across it.  (The fences would force vmcnt(0), also
// for loads deliberately left in flight across the barrier.)
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ float loadf(Buf b, uint32_t off) {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_raw_buffer_load_b32(b.r, off, 0, 0));
}

// ---- MFMA ------------------------------------------------------------------
// D += A B on v_mfma_f32_32x32x16_{bf16,f16}: same shape and register layout.
template <typename E>
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    if constexpr (__is_same(E, f16))
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0,
                                                      0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---- LDS -------------------------------------------------------------------
__device__ __forceinline__ bf16x8 lds_read16(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void lds_write16(bf16* p, u32x4 v) {
    *reinterpret_cast<u32x4*>(p) = v;
}
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
    i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(p));
    return __builtin_bit_cast(bf16x4, v);
}
__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// ---- conversions / math ----------------------------------------------------
// Two fp32 values rounded to nearest-even 16-bit elements of type E, packed
// (low half = a) into one dword.
template <typename E>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    if constexpr (__is_same(E, f16))
        return __builtin_bit_cast(uint32_t, f16x2{(f16)a, (f16)b});
    else
        return __builtin_bit_cast(uint32_t, bf16x2{(bf16)a, (bf16)b});
}
// Eight fp32 values as one MFMA operand of element type E.
template <typename E>
__device__ __forceinline__ bf16x8 pack8(const float* x) {
    const u32x4 w{pack2<E>(x[0], x[1]), pack2<E>(x[2], x[3]), pack2<E>(x[4], x[5]),
                  pack2<E>(x[6], x[7])};
    return __builtin_bit_cast(bf16x8, w);
}
// Elements o .. o+7 of a score block as one MFMA operand of element type E.
template <typename E>
__device__ __forceinline__ bf16x8 pack8(const f32x16& x, int o) {
    const u32x4 w{pack2<E>(x[o], x[o + 1]), pack2<E>(x[o + 2], x[o + 3]),
                  pack2<E>(x[o + 4], x[o + 5]), pack2<E>(x[o + 6], x[o + 7])};
    return __builtin_bit_cast(bf16x8, w);
}
// The value of a 16-bit element of type E.
template <typename E>
__device__ __forceinline__ float to_f32(bf16 raw) {
    if constexpr (__is_same(E, f16))
        return (float)__builtin_bit_cast(f16, raw);
    else
        return (float)raw;
}
__device__ __forceinline__ float exp2_fast(float x) {
    return __builtin_amdgcn_exp2f(x);  // v_exp_f32; exp2(-inf) = 0
}
__device__ __forceinline__ float log2_fast(float x) {
    return __builtin_amdgcn_logf(x);  // v_log_f32 (base 2)
}
__device__ __forceinline__ float xor32(float x) {  // value of lane l ^ 32
    return __shfl_xor(x, 32, 64);
}
// v_permlane32_swap with both operands x: each lane ends up holding its own
// value and that of lane l ^ 32 (in some order), so max/sum of the pair is a
// pair reduction across the two halves of the wave without an LDS round trip.
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                    __builtin_bit_cast(unsigned, x),
                                                    false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]),
                 __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                    __builtin_bit_cast(unsigned, x),
                                                    false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

template <typename E>
__device__ __forceinline__ u32x2 pack4(float a, float b, float c, float d) {
    return u32x2{pack2<E>(a, b), pack2<E>(c, d)};
}

// ---- attention dropout -------------------------------------------------------
// Drop decisions come from the counter-based generator Philox4x32-10 (Salmon,
// Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC
// 2011): ten rounds, each forming the 64-bit products 0xD2511F53 * c0 and
// 0xCD9E8D57 * c2 and mixing their halves with c1, c3 and the key, the key
// advancing by (0x9E3779B9, 0xBB67AE85) between rounds.  For query i and key
// j of head bh the counter is (j / 4, i / 4, bh, offset) and the key the
// 64-bit seed; byte j % 4 of output word i % 4 is compared with the threshold
// T (kept iff >= T), so one call decides a 4 x 4 block of (query, key) pairs.
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                               uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        // three-input XORs as one v_bitop3_b32 each (truth table 0x96: odd
        // number of ones); the compiler emits two v_xor_b32 otherwise
        const uint32_t n0 = (uint32_t)__builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
        const uint32_t n2 = (uint32_t)__builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
    }
    return u32x4{c0, c1, c2, c3};
}

// The decision bytes of the 4 x 4 block holding (query i, key j): word w of
// the result holds queries i0 + w (i0 = i & ~3), byte t keys j0 + t.
__device__ __forceinline__ u32x4 dropout_block(const Dropout& d, uint32_t bh, int i, int j) {
    return philox4x32_10((uint32_t)j >> 2, (uint32_t)i >> 2, bh, d.offset, d.seed_lo,
                         d.seed_hi);
}
__device__ __forceinline__ bool dropout_keep(uint32_t word, int byte, uint32_t thresh) {
    return ((word >> (8 * byte)) & 0xFFu) >= thresh;
}

// The 4 words of v in the order of an XOR with t (0..3): element g is
// v[g ^ t].  Two rounds of selects, no branches.
__device__ __forceinline__ u32x4 xor_permute(const u32x4& v, int t) {
    const bool s1 = (t & 1) != 0, s2 = (t & 2) != 0;
    const u32x4 a{s1 ? v[1] : v[0], s1 ? v[0] : v[1], s1 ? v[3] : v[2], s1 ? v[2] : v[3]};
    return u32x4{s2 ? a[2] : a[0], s2 ? a[3] : a[1], s2 ? a[0] : a[2], s2 ? a[1] : a[3]};
}

// Sharing generator calls inside a quad of lanes (lanes 4m .. 4m+3, t = lane
// % 4).  Where the quad's lanes hold the 4 queries (or the 4 keys) of one
// block and each needs the same 4 blocks, lane t computes block t and the
// quad trades the pieces: p[d] is the 32-bit piece of this lane's block that
// quad lane t ^ d needs; the result's element g is the piece of block g meant
// for this lane.  DPP quad permutations xor 1, 2 and 3 (quad_perm selectors
// 0xB1, 0x4E, 0x1B) read the partners' registers; every lane of the quad
// must be active.
__device__ __forceinline__ u32x4 quad_share(int t, const u32x4& p) {
    // element d: what quad lane t ^ d computed for this lane, a piece of
    // block t ^ d
    const u32x4 got{p[0], (uint32_t)__builtin_amdgcn_mov_dpp((int)p[1], 0xB1, 0xF, 0xF, false),
                    (uint32_t)__builtin_amdgcn_mov_dpp((int)p[2], 0x4E, 0xF, 0xF, false),
                    (uint32_t)__builtin_amdgcn_mov_dpp((int)p[3], 0x1B, 0xF, 0xF, false)};
    return xor_permute(got, t);
}
// byte c of each of a block's 4 words, packed (byte x from word x)
__device__ __forceinline__ uint32_t block_column(const u32x4& b, int c) {
    // v_perm_b32: selector bytes 0-3 take the second source, 4-7 the first
    const uint32_t sel = (uint32_t)c | ((uint32_t)(4 + c) << 8) | 0x0C0C0000u;
    const uint32_t lo = __builtin_amdgcn_perm(b[1], b[0], sel);
    const uint32_t up = __builtin_amdgcn_perm(b[3], b[2], sel);
    return __builtin_amdgcn_perm(up, lo, 0x05040100u);
}

}  // namespace fa
