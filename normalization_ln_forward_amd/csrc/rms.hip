// RMSNorm along the channel dim of a [B, C, S] tensor
// (RMS page "Kimi-K2.6 l1_p36", turns 1-2: y = x / sqrt(mean_c x^2 + eps)).
//
// Layout: one position (b, s) has its C values S elements apart, so a lane
// that owns a position walks the channels with stride S while the 64 lanes
// of a wave own consecutive positions and read each channel row together
// (RMS page, turn 2, the lane-per-position idea; turn 4 widens it to four
// positions per lane with 128-bit loads).
//
// gfx950 design: a workgroup owns a tile of 64*VEC consecutive positions of
// one sample.  Its W waves split the C channels, CPW each, and hold their
// CPW values of the tile in VGPRs, so x is read from HBM exactly once:
//   1. each wave issues its CPW 128-bit loads (64 lanes x 16 B = one 1 KiB
//      row segment per channel, fully coalesced), then sums squares;
//   2. per-lane partial sums cross waves through LDS (W x 64 x 16 B), each
//      wave adds them in wave order (fixed order: deterministic);
//   3. each wave scales its held values by 1/sqrt(ms + eps) and writes them
//      with nontemporal 128-bit stores.
// Channel counts beyond what fits in registers use a streaming kernel that
// reads x twice (the second read is served by L2 / MALL when it hits).
//
// Strided views (RMS page, turn 2 reasons about the layout and the
// wrapper's contiguity handling): the kernels take the batch and channel
// strides of x and y separately (the positions of one channel row stay
// contiguous), so a channel slice or a batch-strided view is normalized in
// place of a copy; rstd (1 / sqrt(ms + eps) per position, [B, S]) is
// written when asked for.
#include "common.hpp"
#include "internal.hpp"

#include <algorithm>

// Channels per wave and 64-lane position segments per lane for the
// register-held kernel (C = 64: 16 waves of 4 channels, 1 KiB per channel
// row segment; the fastest of the shapes measured on MI355X in steady
// state: 3% ahead of 8 waves of 8 channels with 2 KiB segments).
#ifndef NORMFWD_RMS_CPW
#define NORMFWD_RMS_CPW 4
#endif
#ifndef NORMFWD_RMS_PPL
#define NORMFWD_RMS_PPL 1
#endif
#ifndef NORMFWD_RMS_XCD
#define NORMFWD_RMS_XCD 1
#endif
// Streaming (nontemporal) hints on the x loads and y stores.
#ifndef NORMFWD_RMS_NT_LOAD
#define NORMFWD_RMS_NT_LOAD 1
#endif
#ifndef NORMFWD_RMS_NT_STORE
#define NORMFWD_RMS_NT_STORE 1
#endif

namespace normfwd {

template <int VEC>
struct VecOf;
template <>
struct VecOf<4> { using T = f4; };
template <>
struct VecOf<1> { using T = float; };

// Register budget per lane is CPW * PPL vectors; the block-size bound keeps
// the compiler's VGPR limit (512 / waves-per-SIMD) above that.
constexpr int hold_max_threads(int vecs) { return vecs <= 16 ? 1024 : vecs <= 32 ? 512 : 256; }

// The register-held kernel's body.  NORM = false: the same loads, stores,
// grid and workgroup order with the arithmetic left out (y = x), a
// measurement reference for what this access pattern costs by itself
// (rms_copy_pattern_kernel).
template <int CPW, int PPL, int VEC, bool NORM>
__device__ __forceinline__ void rms_hold_body(const float* x, float* y, int C, int64_t S, int64_t tiles, float eps,
                                              RmsStrides L, float* rstd)
{
    using V = typename VecOf<VEC>::T;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    V* part = reinterpret_cast<V*>(smem_raw);  // [nwaves][PPL][64]

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nwaves = blockDim.x / kWave;
    // each XCD walks one contiguous eighth of the tiles (measured +5% over index order)
    const int64_t blk = NORMFWD_RMS_XCD ? xcd_contiguous(blockIdx.x, gridDim.x) : blockIdx.x;
    const int64_t b = blk / tiles;
    const int64_t tile = blk - b * tiles;
    // position of (lane, j): the wave reads PPL adjacent 64*VEC-position segments per channel
    const int64_t s0 = tile * (kWave * PPL * VEC) + (int64_t)lane * VEC;
    const int c0 = wave * CPW;
    const int64_t base = b * L.xsb + (int64_t)c0 * L.xsc + s0;   // x
    const int64_t ybase = b * L.ysb + (int64_t)c0 * L.ysc + s0;  // y

    V v[CPW][PPL];
    // Interior tiles (every position and channel of this wave in range, the
    // common case) load without per-element guards, so all CPW * PPL loads
    // issue back to back.
    const bool interior = (tile + 1) * (kWave * PPL * VEC) <= S && c0 + CPW <= C;
    if (interior) {
#pragma unroll
        for (int k = 0; k < CPW; ++k)
#pragma unroll
            for (int j = 0; j < PPL; ++j) {
                const V* src = reinterpret_cast<const V*>(x + base + (int64_t)k * L.xsc + j * kWave * VEC);
                v[k][j] = NORMFWD_RMS_NT_LOAD ? ld_nt(src) : *src;
            }
    } else {
#pragma unroll
        for (int k = 0; k < CPW; ++k)
#pragma unroll
            for (int j = 0; j < PPL; ++j) {
                const bool ok = (s0 + j * kWave * VEC < S) && (c0 + k < C);  // VEC == 4 implies S % 4 == 0
                const V* src = reinterpret_cast<const V*>(x + base + (int64_t)k * L.xsc + j * kWave * VEC);
                v[k][j] = ok ? (NORMFWD_RMS_NT_LOAD ? ld_nt(src) : *src) : V(0.0f);
            }
    }
    V acc[PPL];
    if constexpr (NORM) {
#pragma unroll
        for (int j = 0; j < PPL; ++j) {
            acc[j] = V(0.0f);
#pragma unroll
            for (int k = 0; k < CPW; ++k) acc[j] += v[k][j] * v[k][j];
            part[(wave * PPL + j) * kWave + lane] = acc[j];
        }
        __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < PPL; ++j) {
        V tot = V(0.0f);
        if constexpr (NORM) {
            tot = part[j * kWave + lane];
            for (int w = 1; w < nwaves; ++w) tot += part[(w * PPL + j) * kWave + lane];
        }
        V inv;
        if constexpr (!NORM) {
            inv = V(1.0f);
        } else if constexpr (VEC == 4) {
            inv.x = 1.0f / sqrtf(tot.x / (float)C + eps);
            inv.y = 1.0f / sqrtf(tot.y / (float)C + eps);
            inv.z = 1.0f / sqrtf(tot.z / (float)C + eps);
            inv.w = 1.0f / sqrtf(tot.w / (float)C + eps);
        } else {
            inv = 1.0f / sqrtf(tot / (float)C + eps);
        }
        const bool okj = interior || s0 + j * kWave * VEC < S;
        if (NORM && rstd && wave == 0 && okj) *reinterpret_cast<V*>(rstd + b * S + s0 + j * kWave * VEC) = inv;
#pragma unroll
        for (int k = 0; k < CPW; ++k) {
            if (okj && (interior || c0 + k < C)) {
                V* dst = reinterpret_cast<V*>(y + ybase + (int64_t)k * L.ysc + j * kWave * VEC);
                const V o = NORM ? v[k][j] * inv : v[k][j];
                if (NORMFWD_RMS_NT_STORE)
                    st_nt(o, dst);
                else
                    *dst = o;
            }
        }
    }
}

template <int CPW, int PPL, int VEC>
__global__ void __launch_bounds__(hold_max_threads(CPW * PPL))
rms_ch_hold_kernel(const float* x, float* y, int C, int64_t S, int64_t tiles, float eps, RmsStrides L, float* rstd)
{
    rms_hold_body<CPW, PPL, VEC, true>(x, y, C, S, tiles, eps, L, rstd);
}

template <int CPW, int PPL, int VEC>
__global__ void __launch_bounds__(hold_max_threads(CPW * PPL))
rms_copy_pattern_kernel(const float* x, float* y, int C, int64_t S, int64_t tiles, float eps, RmsStrides L,
                        float* rstd)
{
    rms_hold_body<CPW, PPL, VEC, false>(x, y, C, S, tiles, eps, L, rstd);
}

// Streaming variant for large C: 4 waves split the channels; pass 1 sums
// squares, pass 2 re-reads x and writes y.
template <int VEC>
__global__ void __launch_bounds__(256)
rms_ch_stream_kernel(const float* x, float* y, int C, int64_t S, int64_t tiles, float eps, RmsStrides L, float* rstd)
{
    using V = typename VecOf<VEC>::T;
    __shared__ V part[4][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t b = blockIdx.x / tiles;
    const int64_t tile = blockIdx.x - b * tiles;
    const int64_t s = (tile * kWave + lane) * VEC;
    const bool active = s < S;
    const int per = (int)ceil_div(C, 4);
    const int c_begin = wave * per;
    const int c_end = min(C, c_begin + per);

    V acc = V(0.0f);
    if (active) {
        for (int c = c_begin; c < c_end; ++c) {
            V v = *reinterpret_cast<const V*>(x + b * L.xsb + (int64_t)c * L.xsc + s);
            acc += v * v;
        }
    }
    part[wave][lane] = acc;
    __syncthreads();
    V tot = part[0][lane] + part[1][lane] + part[2][lane] + part[3][lane];
    V inv;
    if constexpr (VEC == 4) {
        inv.x = 1.0f / sqrtf(tot.x / (float)C + eps);
        inv.y = 1.0f / sqrtf(tot.y / (float)C + eps);
        inv.z = 1.0f / sqrtf(tot.z / (float)C + eps);
        inv.w = 1.0f / sqrtf(tot.w / (float)C + eps);
    } else {
        inv = 1.0f / sqrtf(tot / (float)C + eps);
    }
    if (active) {
        if (rstd && wave == 0) *reinterpret_cast<V*>(rstd + b * S + s) = inv;
        for (int c = c_begin; c < c_end; ++c) {
            V v = *reinterpret_cast<const V*>(x + b * L.xsb + (int64_t)c * L.xsc + s);
            st_nt(v * inv, reinterpret_cast<V*>(y + b * L.ysb + (int64_t)c * L.ysc + s));
        }
    }
}

// Larger tensors are launched in batches of whole samples (samples_per_launch).

template <int CPW, int PPL, int VEC, bool NORM = true>
static hipError_t launch_hold(const float* x, float* y, int64_t B, int64_t C, int64_t S, float eps,
                              const RmsStrides& L, float* rstd, hipStream_t st)
{
    const int nwaves = (int)ceil_div(C, CPW);
    const int64_t tiles = ceil_div(S, (int64_t)kWave * PPL * VEC);
    const size_t lds = (size_t)nwaves * PPL * kWave * sizeof(typename VecOf<VEC>::T);
    const int64_t per_launch = samples_per_launch(tiles * nwaves * kWave);
    for (int64_t b0 = 0; b0 < B; b0 += per_launch) {
        const int64_t nb = std::min(per_launch, B - b0);
        const float* xb = x + b0 * L.xsb;
        float* yb = y + b0 * L.ysb;
        float* rb = rstd ? rstd + b0 * S : nullptr;
        const hipError_t e =
            NORM ? launch_kernel((rms_ch_hold_kernel<CPW, PPL, VEC>), dim3((unsigned)(nb * tiles)),
                                 dim3(nwaves * kWave), lds, st, xb, yb, (int)C, S, tiles, eps, L, rb)
                 : launch_kernel((rms_copy_pattern_kernel<CPW, PPL, VEC>), dim3((unsigned)(nb * tiles)),
                                 dim3(nwaves * kWave), lds, st, xb, yb, (int)C, S, tiles, eps, L, rb);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int VEC>
static hipError_t launch_stream(const float* x, float* y, int64_t B, int64_t C, int64_t S, float eps,
                                const RmsStrides& L, float* rstd, hipStream_t st)
{
    const int64_t tiles = ceil_div(S, (int64_t)kWave * VEC);
    const int64_t per_launch = samples_per_launch(tiles * 256);
    for (int64_t b0 = 0; b0 < B; b0 += per_launch) {
        const int64_t nb = std::min(per_launch, B - b0);
        const hipError_t e = launch_kernel((rms_ch_stream_kernel<VEC>), dim3((unsigned)(nb * tiles)), dim3(256), 0,
                                           st, x + b0 * L.xsb, y + b0 * L.ysb, (int)C, S, tiles, eps, L,
                                           rstd ? rstd + b0 * S : nullptr);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int VEC>
static hipError_t launch_vec(const float* x, float* y, int64_t B, int64_t C, int64_t S, float eps,
                             const RmsStrides& L, float* rstd, hipStream_t st)
{
    // Register-held kernel: the tuned shape when its waves fit one block,
    // 16 channels per wave (up to 16 waves) beyond that, streaming above.
    constexpr int cpw = NORMFWD_RMS_CPW, ppl = NORMFWD_RMS_PPL;
    if (ceil_div(C, cpw) * kWave <= hold_max_threads(cpw * ppl))
        return launch_hold<cpw, ppl, VEC>(x, y, B, C, S, eps, L, rstd, st);
    if (C <= 16 * 16) return launch_hold<16, 1, VEC>(x, y, B, C, S, eps, L, rstd, st);
    return launch_stream<VEC>(x, y, B, C, S, eps, L, rstd, st);
}

hipError_t launch_rms_ch(const float* x, float* y, int64_t B, int64_t C, int64_t S, float eps, const RmsStrides& L,
                         float* rstd, hipStream_t st)
{
    auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    const bool vec4 = S % 4 == 0 && al(x) && al(y) && (!rstd || al(rstd)) && L.xsb % 4 == 0 && L.xsc % 4 == 0 &&
                      L.ysb % 4 == 0 && L.ysc % 4 == 0;
    return vec4 ? launch_vec<4>(x, y, B, C, S, eps, L, rstd, st) : launch_vec<1>(x, y, B, C, S, eps, L, rstd, st);
}

// Measurement reference: rmsnorm_ch_forward's access pattern on [B, C, S]
// (the tuned register-held kernel: same grid, order, loads and stores) as a
// plain copy.  Needs 16-byte aligned tensors, S % 4 == 0 and C <= 64.
hipError_t launch_rms_copy_pattern(const float* x, float* y, int64_t B, int64_t C, int64_t S, hipStream_t st)
{
    constexpr int cpw = NORMFWD_RMS_CPW, ppl = NORMFWD_RMS_PPL;
    if (S % 4 != 0 || (reinterpret_cast<uintptr_t>(x) & 15) || (reinterpret_cast<uintptr_t>(y) & 15) ||
        ceil_div(C, cpw) * kWave > hold_max_threads(cpw * ppl))
        return hipErrorInvalidValue;
    return launch_hold<cpw, ppl, 4, false>(x, y, B, C, S, 0.0f, RmsStrides{C * S, S, C * S, S}, nullptr, st);
}

}  // namespace normfwd
