// lds_ring.h -- building blocks of the MFMA kernels that stream operands
// through an LDS ring filled by direct global->LDS loads (gfx950).
//
// Operand rows are staged 128 bytes of the reduction dimension at a time, as
// eight 16-byte chunks in XOR-permuted slots, so that the 16 rows a fragment
// read touches land in distinct LDS banks.  Loads complete in order per wave;
// a wave waits for its own loads with an explicit vmcnt and the workgroup then
// meets at a barrier that carries no memory fence (a fence would wait for every
// outstanding load and drain the ring).
#pragma once

#include "common.h"

namespace moe {
namespace {

template <int DT>
struct FTraits;
template <>
struct FTraits<DT_F32> {
    static constexpr int esz = 4;
    __device__ static f32x4 mma(float a, float b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0); }
};
template <>
struct FTraits<DT_BF16> {
    static constexpr int esz = 2;
    __device__ static f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct FTraits<DT_E4M3> {
    // one 16x16x128 MFMA covers exactly one 128-long quantisation block
    static constexpr int esz = 1;
    __device__ static f32x4 mma(i32x8 a, i32x8 b, f32x4 c) {
        // zero scale operands give the unscaled instruction (bit-identical to unit E8M0
        // scales, and faster to issue)
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
    }
};

// Staged rows hold CB bytes of the reduction dimension (128: one e4m3 MFMA
// step, two bf16 steps, eight fp32 steps), as CB/16 chunks of 16 bytes in
// XOR-permuted slots.  Lanes 0-15 of a fragment read take one chunk column
// (bf16: chunk g = lane/16; e4m3: chunks 2g and 2g+1) of 16 consecutive rows.
// gfx950 serves a 16-byte LDS read in four passes of 16 lanes over 64 banks
// (256 bytes); a pass takes four lane quads of one wave half, those whose
// quad index (lane/4 mod 8) has the same bit parity (0,3,5,6 or 1,2,4,7),
// as bank-conflict counters on the box show.  Rows are 128 bytes apart, so
// the row's bit 0 picks the bank half; for CB = 128 the slot permutation
// below puts every pass of the bf16 and e4m3 fragment reads in 16 distinct
// 16-byte bank groups (the previous (row & 7) ^ (row >> 3 & 1) left every
// bf16 pass two-way conflicted).
template <int CB>
__device__ __forceinline__ int swz(int row) {
    if (CB == 128) return (row & 1) ^ ((row & 2) << 1) ^ (((row >> 2) & 1) * 3);
    return ((row >> 1) ^ (row >> 3)) & 3;
}

template <int DT>
struct Frag;
template <>
struct Frag<DT_F32> {
    static constexpr int CB = 128, kSub = 8;  // 16x16x4 steps per 128-byte row
    typedef float t;
    __device__ static t load(const char *stage, int row, int s, int lane) {
        return *(const float *)(stage + row * CB + ((s ^ swz<CB>(row)) << 4) + (lane >> 4) * 4);
    }
};
template <>
struct Frag<DT_BF16> {
    static constexpr int CB = 128, kSub = 2;  // 16x16x32 steps per 128-byte row
    typedef bf16x8 t;
    __device__ static t load(const char *stage, int row, int s, int lane) {
        return *(const bf16x8 *)(stage + row * CB + (((s * 4 + (lane >> 4)) ^ swz<CB>(row)) << 4));
    }
};
template <>
struct Frag<DT_E4M3> {
    static constexpr int CB = 128, kSub = 1;  // one 16x16x128 step per 128-byte row
    typedef i32x8 t;
    __device__ static t load(const char *stage, int row, int s, int lane) {
        const int c = 2 * (lane >> 4);
        const i32x4 lo = *(const i32x4 *)(stage + row * CB + ((c ^ swz<CB>(row)) << 4));
        const i32x4 hi = *(const i32x4 *)(stage + row * CB + (((c + 1) ^ swz<CB>(row)) << 4));
        return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
};

// Fence-free workgroup barrier: the ring is filled by direct global->LDS loads
// whose completion each wave establishes with an explicit vmcnt wait.
__device__ __forceinline__ void cta_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt with only the LDS/scalar counter constrained (lgkmcnt(0)).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// s_waitcnt vmcnt(n) for a wave-uniform n (the immediate is encoded per case;
// counts above 47 wait for everything, which is only more conservative).
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
    switch (n) {
#define MOE_VMCNT_CASE(k) case k: wait_vmcnt<k>(); break;
        MOE_VMCNT_CASE(1) MOE_VMCNT_CASE(2) MOE_VMCNT_CASE(3) MOE_VMCNT_CASE(4) MOE_VMCNT_CASE(5)
        MOE_VMCNT_CASE(6) MOE_VMCNT_CASE(7) MOE_VMCNT_CASE(8) MOE_VMCNT_CASE(9) MOE_VMCNT_CASE(10)
        MOE_VMCNT_CASE(11) MOE_VMCNT_CASE(12) MOE_VMCNT_CASE(13) MOE_VMCNT_CASE(14) MOE_VMCNT_CASE(15)
        MOE_VMCNT_CASE(16) MOE_VMCNT_CASE(17) MOE_VMCNT_CASE(18) MOE_VMCNT_CASE(19) MOE_VMCNT_CASE(20)
        MOE_VMCNT_CASE(21) MOE_VMCNT_CASE(22) MOE_VMCNT_CASE(23) MOE_VMCNT_CASE(24) MOE_VMCNT_CASE(25)
        MOE_VMCNT_CASE(26) MOE_VMCNT_CASE(27) MOE_VMCNT_CASE(28) MOE_VMCNT_CASE(29) MOE_VMCNT_CASE(30)
        MOE_VMCNT_CASE(31) MOE_VMCNT_CASE(32) MOE_VMCNT_CASE(33) MOE_VMCNT_CASE(34) MOE_VMCNT_CASE(35)
        MOE_VMCNT_CASE(36) MOE_VMCNT_CASE(37) MOE_VMCNT_CASE(38) MOE_VMCNT_CASE(39) MOE_VMCNT_CASE(40)
        MOE_VMCNT_CASE(41) MOE_VMCNT_CASE(42) MOE_VMCNT_CASE(43) MOE_VMCNT_CASE(44) MOE_VMCNT_CASE(45)
        MOE_VMCNT_CASE(46) MOE_VMCNT_CASE(47)
#undef MOE_VMCNT_CASE
        default: wait_vmcnt<0>(); break;
    }
}

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma16(const void *g, void *l) {
    __builtin_amdgcn_global_load_lds(g, (lds_void *)l, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void *g, void *l) {
    __builtin_amdgcn_global_load_lds(g, (lds_void *)l, 4, 0, 0);
}

// The same loads through a buffer descriptor: address = base + voff (per lane)
// + soff (wave-uniform), so a step's loads need scalar arithmetic only.  Offsets
// at or past the descriptor's byte count read as zero.
__device__ __forceinline__ void buffer_dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff, void *l) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)l, 16, (int)voff, soff, 0, 0);
}
__device__ __forceinline__ void buffer_dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff, void *l) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)l, 4, (int)voff, soff, 0, 0);
}

// 16-byte loads with the nontemporal cache policy (the `nt` bit): lines they bring
// into L2 are the first to go, which leaves L2 to operands that other workgroups
// read again.  For data one workgroup reads once.
__device__ __forceinline__ void dma16_stream(const void *g, void *l) {
    __builtin_amdgcn_global_load_lds(g, (lds_void *)l, 16, 0, 2);
}
__device__ __forceinline__ void buffer_dma16_stream(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff, void *l) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)l, 16, (int)voff, soff, 0, 2);
}

}  // namespace
}  // namespace moe
