// GroupNorm -> LeakyReLU -> x + x on an [N, C] tensor
// (GN page "Kimi-K2.6 l2_p62", turn 1: num_groups groups of M = C/G
// contiguous channels, per-(row, group) mean and population variance, eps
// inside the square root, per-channel gamma/beta, LeakyReLU(negative_slope),
// then the tensor added to itself).
//
// gfx950 fast path (M a multiple of 4 with M/4 a power of two <= 64, 16-byte
// aligned tensors): lanes own consecutive float4s of a row, so L = M/4
// adjacent lanes hold one group (GN page, turn 2 puts one group on adjacent
// lanes; turn 5 adds float4 so four lanes cover a 16-channel group).  A wave
// owns a tile of ITEMS*64 float4s of one row (ITEMS*256 channels; the whole
// 8192-channel row when ITEMS = 32, i.e. one wave per row) and
//   1. issues all ITEMS 128-bit loads up front (the row stays in VGPRs),
//   2. shifts the group by its first element K (broadcast from the group's
//      first lane), reduces the group's sum of d = x - K across its L lanes
//      with DPP quad_perm (L = 4: two row-local DPP adds, no LDS traffic) and
//      forms mean_d (the mean is K + mean_d; the shift keeps the sum exact
//      to fp32 rounding of the deviations, not of the values, so a group far
//      from 0, e.g. after a large fc bias, keeps its accuracy),
//   3. reduces the sum of squared deviations e = d - mean_d the same way
//      (two-pass in registers), forms rstd,
//   4. applies gamma/beta (read through L2: 32 KiB each, shared by all
//      rows), LeakyReLU and the doubling, and writes y with nontemporal
//      128-bit stores.
// x is read from HBM once and y written once.  Other shapes use a generic
// kernel: one lane per group for M <= 32, one wave per group beyond.
#include "common.hpp"
#include "internal.hpp"

#include <algorithm>

#ifndef NORMFWD_GN_ITEMS
#define NORMFWD_GN_ITEMS 8
#endif
#ifndef NORMFWD_GN_XCD
#define NORMFWD_GN_XCD 0
#endif
// Streaming (nontemporal) hints on the x loads and y stores.
#ifndef NORMFWD_GN_NT_LOAD
#define NORMFWD_GN_NT_LOAD 1
#endif
#ifndef NORMFWD_GN_NT_STORE
#define NORMFWD_GN_NT_STORE 1
#endif

namespace normfwd {

__device__ __forceinline__ float lrelu_x2(float z, float slope)
{
    const float a = z > 0.0f ? z : slope * z;
    return a + a;
}

template <int L, int ITEMS>
__global__ void __launch_bounds__(256)
gn_fast_kernel(const float* x, const float* __restrict__ gamma, const float* __restrict__ beta, float* y,
               int64_t n_tiles, int64_t tiles_per_row, int64_t C4, int M, float eps, float slope, float* mean_out,
               float* rstd_out)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t blk = NORMFWD_GN_XCD ? xcd_contiguous(blockIdx.x, gridDim.x) : blockIdx.x;
    const int64_t tile = blk * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (tile >= n_tiles) return;  // whole wave leaves together
    const int64_t row = tile / tiles_per_row;
    const int64_t c4_0 = (tile - row * tiles_per_row) * (ITEMS * kWave) + lane;
    const f4* xr = reinterpret_cast<const f4*>(x) + row * C4;
    f4* yr = reinterpret_cast<f4*>(y) + row * C4;
    const f4* g4 = reinterpret_cast<const f4*>(gamma);
    const f4* b4 = reinterpret_cast<const f4*>(beta);
    const float inv_m = 1.0f / (float)M;

    f4 v[ITEMS];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        const int64_t c4 = c4_0 + i * kWave;
        v[i] = c4 < C4 ? (NORMFWD_GN_NT_LOAD ? ld_nt(xr + c4) : xr[c4]) : f4(0.0f);
    }
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        const int64_t c4 = c4_0 + i * kWave;
        const float K = group_first<L>(v[i].x);
        const f4 dk = v[i] - K;
        const float md = group_sum<L>((dk.x + dk.y) + (dk.z + dk.w)) * inv_m;
        const f4 d = dk - md;
        const float ssd = group_sum<L>((d.x * d.x + d.y * d.y) + (d.z * d.z + d.w * d.w));
        const float rstd = 1.0f / sqrtf(ssd * inv_m + eps);
        if (mean_out && c4 < C4 && c4 % L == 0) {  // the group's first lane: statistics of (row, group)
            const int64_t gi = row * (C4 / L) + c4 / L;
            mean_out[gi] = K + md;
            rstd_out[gi] = rstd;
        }
        if (c4 < C4) {
            const f4 g = gamma ? g4[c4] : f4(1.0f);
            const f4 bb = beta ? b4[c4] : f4(0.0f);
            const f4 z = d * rstd * g + bb;
            f4 o;
            o.x = lrelu_x2(z.x, slope);
            o.y = lrelu_x2(z.y, slope);
            o.z = lrelu_x2(z.z, slope);
            o.w = lrelu_x2(z.w, slope);
            if (NORMFWD_GN_NT_STORE)
                st_nt(o, yr + c4);
            else
                yr[c4] = o;
        }
    }
}

// Generic: one lane per (row, group); two passes over the group's M
// channels for the statistics (around the group's first element K, as in
// the fast kernel), a third for the output.
__global__ void __launch_bounds__(256)
gn_lane_kernel(const float* x, const float* __restrict__ gamma, const float* __restrict__ beta, float* y,
               int64_t n_groups_total, int64_t G, int64_t C, int M, float eps, float slope, float* mean_out,
               float* rstd_out)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n_groups_total) return;
    const int64_t row = t / G, g = t - row * G;
    const int64_t base = row * C + g * M;
    const float K = x[base];
    float sum = 0.0f;
    for (int j = 0; j < M; ++j) sum += x[base + j] - K;
    const float md = sum / (float)M;
    float ssd = 0.0f;
    for (int j = 0; j < M; ++j) {
        const float d = (x[base + j] - K) - md;
        ssd += d * d;
    }
    const float rstd = 1.0f / sqrtf(ssd / (float)M + eps);
    if (mean_out) {
        mean_out[t] = K + md;
        rstd_out[t] = rstd;
    }
    for (int j = 0; j < M; ++j) {
        const int64_t c = g * M + j;
        float z = ((x[base + j] - K) - md) * rstd;
        if (gamma) z = z * gamma[c];
        if (beta) z = z + beta[c];
        y[base + j] = lrelu_x2(z, slope);
    }
}

// Generic: one wave per (row, group) for large M; lanes stride the group.
__global__ void __launch_bounds__(256)
gn_wave_kernel(const float* x, const float* __restrict__ gamma, const float* __restrict__ beta, float* y,
               int64_t n_groups_total, int64_t G, int64_t C, int64_t M, float eps, float slope, float* mean_out,
               float* rstd_out)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (t >= n_groups_total) return;
    const int64_t row = t / G, g = t - row * G;
    const int64_t base = row * C + g * M;
    const float K = x[base];  // shift: the group's first element
    float sum = 0.0f;
    for (int64_t j = lane; j < M; j += kWave) sum += x[base + j] - K;
    const float md = wave_sum(sum) / (float)M;
    float ssd = 0.0f;
    for (int64_t j = lane; j < M; j += kWave) {
        const float d = (x[base + j] - K) - md;
        ssd += d * d;
    }
    const float rstd = 1.0f / sqrtf(wave_sum(ssd) / (float)M + eps);
    if (mean_out && lane == 0) {
        mean_out[t] = K + md;
        rstd_out[t] = rstd;
    }
    // Every lane has finished reading the group before any lane writes it
    // (wave_sum is a wave-wide exchange), which keeps y == x safe.
    for (int64_t j = lane; j < M; j += kWave) {
        const int64_t c = g * M + j;
        float z = ((x[base + j] - K) - md) * rstd;
        if (gamma) z = z * gamma[c];
        if (beta) z = z + beta[c];
        y[base + j] = lrelu_x2(z, slope);
    }
}

template <int L, int ITEMS>
static hipError_t launch_fast(const float* x, const float* gamma, const float* beta, float* y, int64_t N,
                              int64_t C, int64_t M, float eps, float slope, float* mo, float* ro, hipStream_t st)
{
    const int64_t C4 = C / 4;
    const int64_t tiles_per_row = ceil_div(C4, (int64_t)ITEMS * kWave);
    const int64_t per = samples_per_launch(tiles_per_row * kWave);
    for (int64_t r0 = 0; r0 < N; r0 += per) {
        const int64_t nr = std::min(per, N - r0);
        const int64_t n_tiles = nr * tiles_per_row;
        const int64_t G = C / M;
        const hipError_t e = launch_kernel((gn_fast_kernel<L, ITEMS>), dim3((unsigned)ceil_div(n_tiles, 4)), dim3(256),
                                           0, st, x + r0 * C, gamma, beta, y + r0 * C, n_tiles, tiles_per_row, C4,
                                           (int)M, eps, slope, mo ? mo + r0 * G : nullptr, ro ? ro + r0 * G : nullptr);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int L>
static hipError_t launch_fast_items(const float* x, const float* gamma, const float* beta, float* y,
                                    int64_t N, int64_t C, int64_t M, float eps, float slope, float* mo, float* ro,
                                    hipStream_t st)
{
    // A wave's tile never needs to be longer than the row.
    constexpr int items = NORMFWD_GN_ITEMS;
#define NORMFWD_GN_FAST(I) return launch_fast<L, I>(x, gamma, beta, y, N, C, M, eps, slope, mo, ro, st)
    if (C / 4 <= 1 * kWave || items <= 1) NORMFWD_GN_FAST(1);
    if (C / 4 <= 2 * kWave || items <= 2) NORMFWD_GN_FAST(2);
    if (C / 4 <= 4 * kWave || items <= 4) NORMFWD_GN_FAST(4);
    if (C / 4 <= 8 * kWave || items <= 8) NORMFWD_GN_FAST(8);
    if (C / 4 <= 16 * kWave || items <= 16) NORMFWD_GN_FAST(16);
    NORMFWD_GN_FAST(32);
#undef NORMFWD_GN_FAST
}

bool gn_fast_path_applies(const float* x, const float* gamma, const float* beta, const float* y, int64_t C,
                          int64_t M)
{
    auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    if (M % 4 != 0 || M > 4 * kWave) return false;
    const int64_t L = M / 4;
    if ((L & (L - 1)) != 0) return false;
    (void)C;
    return al(x) && al(y) && (!gamma || al(gamma)) && (!beta || al(beta));
}

hipError_t launch_gn_lrelu_x2(const float* x, const float* gamma, const float* beta, float* y, int64_t N,
                              int64_t C, int64_t G, float eps, float slope, float* mo, float* ro, hipStream_t st)
{
    const int64_t M = C / G;
    if (gn_fast_path_applies(x, gamma, beta, y, C, M)) {
        switch (M / 4) {
            case 1: return launch_fast_items<1>(x, gamma, beta, y, N, C, M, eps, slope, mo, ro, st);
            case 2: return launch_fast_items<2>(x, gamma, beta, y, N, C, M, eps, slope, mo, ro, st);
            case 4: return launch_fast_items<4>(x, gamma, beta, y, N, C, M, eps, slope, mo, ro, st);
            case 8: return launch_fast_items<8>(x, gamma, beta, y, N, C, M, eps, slope, mo, ro, st);
            case 16: return launch_fast_items<16>(x, gamma, beta, y, N, C, M, eps, slope, mo, ro, st);
            case 32: return launch_fast_items<32>(x, gamma, beta, y, N, C, M, eps, slope, mo, ro, st);
            case 64: return launch_fast_items<64>(x, gamma, beta, y, N, C, M, eps, slope, mo, ro, st);
            default: break;
        }
    }
    // one lane (M <= 32) or one wave per (row, group)
    const int64_t per = samples_per_launch(M <= 32 ? G : G * kWave);
    for (int64_t r0 = 0; r0 < N; r0 += per) {
        const int64_t total = std::min(per, N - r0) * G;
        float* mb = mo ? mo + r0 * G : nullptr;
        float* rb = ro ? ro + r0 * G : nullptr;
        const hipError_t e =
            M <= 32 ? launch_kernel(gn_lane_kernel, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0, st, x + r0 * C,
                                    gamma, beta, y + r0 * C, total, G, C, (int)M, eps, slope, mb, rb)
                    : launch_kernel(gn_wave_kernel, dim3((unsigned)ceil_div(total, 4)), dim3(256), 0, st, x + r0 * C,
                                    gamma, beta, y + r0 * C, total, G, C, M, eps, slope, mb, rb);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace normfwd
