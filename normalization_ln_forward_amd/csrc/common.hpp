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

// v of the first lane of the aligned group of L consecutive lanes this lane
// belongs to (L a power of two, 1..64): DPP quad_perm broadcasts for L <= 4,
// a lane permute beyond.
template <int L>
__device__ __forceinline__ float group_first(float v) {
    if constexpr (L == 1) {
        return v;
    } else if constexpr (L == 2) {
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xA0, 0xF, 0xF, false));  // [0,0,2,2]
    } else if constexpr (L == 4) {
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x00, 0xF, 0xF, false));  // [0,0,0,0]
    } else {
        return __shfl(v, (int)(threadIdx.x & (kWave - 1)) & ~(L - 1));
    }
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) v += __shfl_xor(v, m);
    return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<kWave>(v); }

// Wave total of one value per lane, uniform on return: DPP butterflies
// inside each quad, rotations inside each 16-lane row, then the four row
// sums read from lanes 0, 16, 32, 48 and added as (r0 + r1) + (r2 + r3).  No
// LDS traffic and no lane-address registers; the order of additions is
// fixed, so every call on the same values gives the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)b, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ float lane_f32(float v, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ double lane_f64(double v, int l)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
template <typename T>
__device__ __forceinline__ T wave_total(T v)
{
    if constexpr (sizeof(T) == 4) {
        v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
        v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
        v += dpp_f32<0x124>(v);  // row_ror:4
        v += dpp_f32<0x128>(v);  // row_ror:8
        return (lane_f32(v, 0) + lane_f32(v, 16)) + (lane_f32(v, 32) + lane_f32(v, 48));
    } else {
        v += dpp_f64<0xB1>(v);
        v += dpp_f64<0x4E>(v);
        v += dpp_f64<0x124>(v);
        v += dpp_f64<0x128>(v);
        return (lane_f64(v, 0) + lane_f64(v, 16)) + (lane_f64(v, 32) + lane_f64(v, 48));
    }
}

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
