// Device-side building blocks shared by the normfwd kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace normfwd {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- memory

// Streaming accesses: data touched once are loaded and stored with the
// nontemporal hint so they do not displace reused lines (affine tensors,
// partial moments) from L2.
template <typename T>
__device__ __forceinline__ T ld_nt(const T* p) { return __builtin_nontemporal_load(p); }
template <typename T>
__device__ __forceinline__ void st_nt(T v, T* p) { __builtin_nontemporal_store(v, p); }

// ---------------------------------------------------------------- DPP / cross-lane

// v from the lane whose index differs in bit 0 / bit 1 (DPP quad_perm, no LDS).
__device__ __forceinline__ float dpp_xor1(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
}

// Butterfly sum over aligned groups of L consecutive lanes (L a power of
// two, 1..64); every lane of a group ends with the same total, and the
// order of additions is fixed (so the result is deterministic).
template <int L>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (L >= 2) v += dpp_xor1(v);
    if constexpr (L >= 4) v += dpp_xor2(v);
    if constexpr (L >= 8) v += __shfl_xor(v, 4);
    if constexpr (L >= 16) v += __shfl_xor(v, 8);
    if constexpr (L >= 32) v += __shfl_xor(v, 16);
    if constexpr (L >= 64) v += __shfl_xor(v, 32);
    return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) v += __shfl_xor(v, m);
    return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<kWave>(v); }

// ---------------------------------------------------------------- XCD-aware order

// Workgroups are dispatched to the 8 XCDs round-robin by index, so in index
// order neighbouring workgroups land on different XCDs (each with its own L2
// and TLB).  This remap hands XCD k the k-th contiguous eighth of the grid
// (a bijection when the grid is a multiple of 8; identity otherwise).
__device__ __forceinline__ int64_t xcd_contiguous(int64_t blk, int64_t nblocks)
{
    if (nblocks % 8 != 0) return blk;
    return (blk & 7) * (nblocks >> 3) + (blk >> 3);
}

// ---------------------------------------------------------------- helpers

__host__ __device__ __forceinline__ int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

__device__ __forceinline__ bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace normfwd
