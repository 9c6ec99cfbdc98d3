// Device helpers shared by the HIP kernels of libbitq (gfx950, MI355X).
// Sources are cited by the short names defined in include/bitq.h:
// [RaBiT], [HGF], [ABQ], [BVSR], [BitNet].
//
// Weights come in the packed blob layout of bitq.h: 64-row tiles in which
// each row owns 16 contiguous bytes per plane and 128-input block, so 64
// lanes reading one row each load 1 KB contiguously.  Each kernel's own
// comment gives its work decomposition.  Results never depend on workgroup
// scheduling: integer partial sums are exact, float partials are added in a
// fixed order or, across workgroups, as 64-bit fixed-point integers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "bitq_internal.h"

namespace bitq {

// --------------------------------------------------------------- utilities
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ float load_act(const void* x, int dt, size_t i) {
    if (dt == BITQ_DT_F32) return static_cast<const float*>(x)[i];
    return bf16_to_f32(static_cast<const uint16_t*>(x)[i]);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(h & 0xFFFFu)));
}

// 16-byte load of element i of a global array given by its address as an
// integer (so the load carries no restrict/invariant provenance and stays in
// program order around memory clobbers), as a global (not flat) access.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 global_load16(uintptr_t base, int i) {
    const u32x4_t v = ((const __attribute__((address_space(1))) u32x4_t*)base)[i];
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

template <int DT>
__device__ __forceinline__ float act_at(const void* x, size_t i) {
    if (DT == BITQ_DT_F32) return static_cast<const float*>(x)[i];
    return bf16_to_f32(static_cast<const uint16_t*>(x)[i]);
}

// popcount(v) + acc as one v_bcnt_u32_b32 (keeps the accumulation a chain
// of accumulating popcounts instead of separate popcounts plus adds).
__device__ __forceinline__ int bcnt_acc(uint32_t v, int acc) {
    int r;
    asm("v_bcnt_u32_b32 %0, %1, %2" : "=v"(r) : "v"(v), "v"(acc));
    return r;
}

// Workgroup barrier that first waits until at most N vector-memory loads of
// this wave are still outstanding (loads retire in issue order, so every load
// issued before the last N has landed, including copies into LDS) and all LDS
// accesses are done.  Loads issued after the copies can stay in flight.
template <int N>
__device__ __forceinline__ void barrier_after_loads() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit count");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));  // vmcnt(N) expcnt(7) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// v of another lane of the same quad (DPP quad_perm: lane i of each group of
// 4 takes lane CTRL[2i+1:2i]).
template <int CTRL>
__device__ __forceinline__ uint32_t quad_swap(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

// A wave-uniform value moved to a scalar register (the compiler cannot tell
// that threadIdx.x / 64 is uniform).
__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Horner combination of per-plane popcounts: sum_j c_j a_j.
__device__ __forceinline__ int combine_planes(const int (&a)[8]) {
    int r = -a[7];
#pragma unroll
    for (int j = 6; j >= 0; --j) r = 2 * r + a[j];
    return r;
}

// Buffer loads: a 128-bit descriptor (base address in scalar registers and a
// byte range), a per-lane 32-bit offset and a wave-uniform 32-bit offset.
// The address arithmetic then stays out of the vector ALUs (no 64-bit
// per-lane adds).  The last descriptor word is the raw-buffer format word of
// the CDNA family.  Callers keep every access inside [base, base + bytes).
// (base and range pass through readfirstlane: they are wave-uniform, and
// the compiler then keeps the descriptor in scalar registers instead of
// looping over the lanes' values at each load)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
    void* ub = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ub, static_cast<short>(0),
                                             static_cast<int>(__builtin_amdgcn_readfirstlane(bytes)), 0x00020000);
}
// A byte count as a descriptor range (at most 2^32 - 16), in integer
// arithmetic (a min() over size_t here went through fp64 compares).
__device__ __forceinline__ uint32_t range_u32(size_t bytes) {
    return bytes < 0xFFFFFFF0u ? static_cast<uint32_t>(bytes) : 0xFFFFFFF0u;
}
__device__ __forceinline__ uint32_t buffer_load_u32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(voff), static_cast<int>(soff), 0);
}
__device__ __forceinline__ uint4 buffer_load_u128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), static_cast<int>(soff), 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

}  // namespace bitq
