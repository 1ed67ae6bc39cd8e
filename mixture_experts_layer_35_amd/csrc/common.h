// common.h -- device helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Two fp32 -> packed bf16 pair (lo in bits 0-15), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950 (same result as f32_to_bf16 for finite inputs).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){lo, hi}, b2));
}

// Stores two adjacent 16-feature blocks of one token's bf16 results (block i
// from a[], block i+1 from b[]; lane group g = lane/16 holds features 4g..4g+3
// of each) with one 16-byte store per lane: lanes of even groups keep block i
// and take their partner's (lane ^ 16) four block-i values, odd groups do the
// same for block i+1.  A token's 32 features then leave as two 32-byte runs
// instead of four 16-byte ones.  Both partners hold the same token, so they are
// active together.
// pair_bf16_value / pair_bf16_col: the lane's 16 bytes and their first feature, for
// callers that store them later.
__device__ __forceinline__ u32x4 pair_bf16_value(const float a[4], const float b[4], int lane) {
    const bool odd = (lane >> 4) & 1;
    const uint32_t a01 = pack_bf16x2(a[0], a[1]), a23 = pack_bf16x2(a[2], a[3]);
    const uint32_t b01 = pack_bf16x2(b[0], b[1]), b23 = pack_bf16x2(b[2], b[3]);
    const uint32_t r0 = __shfl_xor(odd ? a01 : b01, 16, 64), r1 = __shfl_xor(odd ? a23 : b23, 16, 64);
    return odd ? u32x4{r0, r1, b01, b23} : u32x4{a01, a23, r0, r1};
}
__device__ __forceinline__ int pair_bf16_col(int f_block, int lane) {
    return f_block + (((lane >> 4) & 1) ? 16 : 0) + 4 * ((lane >> 4) & ~1);
}
__device__ __forceinline__ void store_pair_bf16(uint16_t *row, int f_block, const float a[4], const float b[4],
                                                int lane, int F) {
    const u32x4 v = pair_bf16_value(a, b, lane);
    const int f = pair_bf16_col(f_block, lane);
    if (f < F) *(u32x4 *)(row + f) = v;
}

// Four fp32 values (already in [-448, 448]) -> four E4M3FN codes, nearest even.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
    uint32_t v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
    return v;
}

// SwiGLU gradient at one feature: h = SiLU(a) * b, SiLU(a) = a * s, s = sigmoid(a);
// da = dh * b * SiLU'(a) with SiLU'(a) = s (1 + a (1 - s)), db = dh * SiLU(a).  One
// definition for the expert kernel's recomputing epilogue and the kernel that reads
// saved (a, b), so both give the same bits.
__device__ __forceinline__ void swiglu_grad(float dh, float a, float b, float &da, float &db) {
    const float sg = 1.0f / (1.0f + __expf(-a));
    da = dh * b * sg * (1.0f + a * (1.0f - sg));
    db = dh * a * sg;
}

__device__ __forceinline__ float clamp448(float x) { return fminf(fmaxf(x, -448.0f), 448.0f); }

// Activation / weight quantisation scale for a group with absolute max amax.
__device__ __forceinline__ float quant_scale(float amax) { return amax == 0.0f ? 1.0f : amax / 448.0f; }

// Total order key for (value, index): larger value first, then lower index.
__device__ __forceinline__ uint64_t order_key(float v, int idx) {
    uint32_t b = __float_as_uint(v == 0.0f ? 0.0f : v);
    uint32_t k = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)k << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)idx);
}
__device__ __forceinline__ int key_index(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
    uint32_t lo = __shfl_xor((int)(uint32_t)v, m, kWave);
    uint32_t hi = __shfl_xor((int)(uint32_t)(v >> 32), m, kWave);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        uint64_t o = shfl_xor_u64(v, m);
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
    return v;
}

}  // namespace moe
