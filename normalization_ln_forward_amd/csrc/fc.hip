// fc -> GroupNorm -> LeakyReLU -> x + x
// (GN page "Kimi-K2.6 l2_p62", turn 1: h = x W^T + b with x [N, K] and W
// [C, K] row-major, then the GroupNorm epilogue on h).
//
// The fc is an fp32 GEMM on the matrix cores (v_mfma_f32_32x32x2_f32, exact
// fp32 products with fp32 accumulation; no reduced-precision inputs).  Both
// operands are K-contiguous, so a workgroup stages a BM x BK tile of x and a
// BN x BK tile of W in LDS (rows padded by 4 floats against bank conflicts)
// and each of its waves computes a 64 x 64 block of h as 2 x 2 MFMA tiles;
// LDS is double-buffered so the next K slice loads during the MFMAs.
// Within one MFMA the two k values a lane pair contributes are free to
// choose as long as x and W agree, so each lane reads 4 consecutive k of its
// row with one 128-bit LDS read and feeds them to 4 successive MFMAs.
// With 16- or 32-channel groups the GroupNorm epilogue runs on the
// accumulators and y is written directly; otherwise h goes to the
// workspace and the GroupNorm kernel reads it back.
#include "common.hpp"
#include "internal.hpp"

namespace normfwd {

typedef float f16v __attribute__((ext_vector_type(16)));

#ifndef NORMFWD_FC_BK
#define NORMFWD_FC_BK 32
#endif
#ifndef NORMFWD_FC_PAD
#define NORMFWD_FC_PAD 4
#endif
// GroupNorm epilogue inside the GEMM for 16- and 32-channel groups.
#ifndef NORMFWD_FC_FUSE
#define NORMFWD_FC_FUSE 1
#endif
#ifndef NORMFWD_FC_WM
#define NORMFWD_FC_WM 4
#endif
constexpr int kBN = 128, kBK = NORMFWD_FC_BK, kPad = NORMFWD_FC_PAD;
constexpr int kLdsRow = kBK + kPad;
constexpr int kVecsPerRow = kBK / 4;

// Workgroup of WM x 2 waves, each computing 64 x 64 of h: a BM = 64 WM by
// BN = 128 output tile.  One K slice is BM x BK of x and BN x BK of W.
template <int WM>
struct Tile {
    static constexpr int kThreads = 128 * WM;
    static constexpr int kBM = 64 * WM;
    static constexpr int kVecsA = kBM * kBK / 4 / kThreads;
    static constexpr int kVecsB = kBN * kBK / 4 / kThreads;
};

template <bool VEC>
__device__ __forceinline__ f4 load_row_vec(const float* __restrict__ p, int rows, int K, int r, int k)
{
    f4 v = f4(0.0f);
    if constexpr (VEC) {  // K % 4 == 0 and 16-byte aligned rows
        if (r < rows && k < K) v = *reinterpret_cast<const f4*>(p + (int64_t)r * K + k);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (r < rows && k + q < K) v[q] = p[(int64_t)r * K + k + q];
    }
    return v;
}

template <bool VEC, int WM>
__device__ __forceinline__ void load_slice(const float* __restrict__ x, const float* __restrict__ W, int M, int N,
                                           int K, int m0, int n0, int k0, f4 (&a)[Tile<WM>::kVecsA],
                                           f4 (&b)[Tile<WM>::kVecsB])
{
    using T = Tile<WM>;
#pragma unroll
    for (int u = 0; u < T::kVecsA; ++u) {
        const int idx = threadIdx.x + T::kThreads * u;
        a[u] = load_row_vec<VEC>(x, M, K, m0 + idx / kVecsPerRow, k0 + (idx % kVecsPerRow) * 4);
    }
#pragma unroll
    for (int u = 0; u < T::kVecsB; ++u) {
        const int idx = threadIdx.x + T::kThreads * u;
        b[u] = load_row_vec<VEC>(W, N, K, n0 + idx / kVecsPerRow, k0 + (idx % kVecsPerRow) * 4);
    }
}

template <int WM>
__device__ __forceinline__ void store_slice(float* As, float* Bs, const f4 (&a)[Tile<WM>::kVecsA],
                                            const f4 (&b)[Tile<WM>::kVecsB])
{
    using T = Tile<WM>;
#pragma unroll
    for (int u = 0; u < T::kVecsA; ++u) {
        const int idx = threadIdx.x + T::kThreads * u;
        *reinterpret_cast<f4*>(As + (idx / kVecsPerRow) * kLdsRow + (idx % kVecsPerRow) * 4) = a[u];
    }
#pragma unroll
    for (int u = 0; u < T::kVecsB; ++u) {
        const int idx = threadIdx.x + T::kThreads * u;
        *reinterpret_cast<f4*>(Bs + (idx / kVecsPerRow) * kLdsRow + (idx % kVecsPerRow) * 4) = b[u];
    }
}

// Sum over the 16 lanes of a DPP row (lanes 16r .. 16r+15), fixed order,
// every lane gets the total: quad butterflies, then rotations by 4 and 8
// within the row.
__device__ __forceinline__ float row16_sum(float v)
{
    v += dpp_xor1(v);
    v += dpp_xor2(v);
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xF, 0xF, false));  // row_ror:4
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false));  // row_ror:8
    return v;
}

// Sum over the GM lanes (channels) of a group inside one 32-lane half:
// GM <= 8 butterflies (group_sum), 16 one DPP row, 32 two DPP rows.  Fixed
// order, every lane of the group gets the total.
template <int GM>
__device__ __forceinline__ float group_lanes_sum(float v)
{
    if constexpr (GM <= 8) {
        return group_sum<GM>(v);
    } else {
        v = row16_sum(v);
        if constexpr (GM == 32) v += __shfl_xor(v, 16);
        return v;
    }
}

// One output element of the epilogue: GroupNorm with the group's statistics
// (mean m, rstd r), gamma g, beta be, then LeakyReLU and the doubling.
__device__ __forceinline__ float gn_out(float d, float rstd, float g, float be, float slope)
{
    const float z = d * rstd * g + be;
    const float a = z > 0.0f ? z : slope * z;
    return a + a;
}

// Epilogue of a wave's 64 x 64 block of h (rows m0w.., columns n0w..).
// D layout of a 32 x 32 tile: lane holds column (lane % 32); register r holds
// row (r / 4) * 8 + (lane / 32) * 4 + r % 4.
template <int GM>
__device__ __forceinline__ void fc_epilogue(f16v (&acc)[2][2], const float* __restrict__ bias,
                                            const float* __restrict__ gamma, const float* __restrict__ beta,
                                            float* __restrict__ out, int M, int N, int m0w, int n0w, int li, int lh,
                                            float eps, float slope, float* __restrict__ mean_out,
                                            float* __restrict__ rstd_out)
{
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0w + j * 32 + li;
            const bool col_ok = col < N;
            const float bb = (bias && col_ok) ? bias[col] : 0.0f;
            if constexpr (GM == 0) {
                if (!col_ok) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = m0w + i * 32 + (r >> 2) * 8 + lh * 4 + (r & 3);
                    if (row < M) out[(int64_t)row * N + col] = acc[i][j][r] + bb;
                }
            } else if constexpr (GM <= 32) {
                const float g = (gamma && col_ok) ? gamma[col] : 1.0f;
                const float be = (beta && col_ok) ? beta[col] : 0.0f;
                constexpr float inv_m = 1.0f / GM;
                // statistics around the group's first channel k: h_c - h_k =
                // (acc_c - acc_k) + (b_c - b_k), so neither a large bias nor
                // an offset of the group from 0 is ever rounded at its own
                // magnitude (h itself never exists in fp32 here)
                const float bk = group_first<GM>(bb);
                const float db = bb - bk;
                // the group's first lane writes the (row, group) statistics
                const bool stats = mean_out && col_ok && (li & (GM - 1)) == 0;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float ak = group_first<GM>(acc[i][j][r]);
                    const float hk = (acc[i][j][r] - ak) + db;
                    const float s1 = group_lanes_sum<GM>(hk);
                    const float md = s1 * inv_m;
                    const float d = hk - md;
                    const float s2 = group_lanes_sum<GM>(d * d);
                    const float rstd = 1.0f / sqrtf(s2 * inv_m + eps);
                    const int row = m0w + i * 32 + (r >> 2) * 8 + lh * 4 + (r & 3);
                    if (row < M && col_ok) out[(int64_t)row * N + col] = gn_out(d, rstd, g, be, slope);
                    if (stats && row < M) {
                        const int64_t gi = (int64_t)row * (N / GM) + col / GM;
                        mean_out[gi] = (ak + bk) + md;
                        rstd_out[gi] = rstd;
                    }
                }
            }
        }
    if constexpr (GM == 64) {
        // a 64-channel group is the wave's two 32-channel tiles: each row's
        // sums are the two tiles' 32-lane sums, added in tile order
        const int c0 = n0w + li, c1 = n0w + 32 + li;
        const bool ok0 = c0 < N, ok1 = c1 < N;
        const float bb0 = (bias && ok0) ? bias[c0] : 0.0f, bb1 = (bias && ok1) ? bias[c1] : 0.0f;
        const float g0 = (gamma && ok0) ? gamma[c0] : 1.0f, g1 = (gamma && ok1) ? gamma[c1] : 1.0f;
        const float be0 = (beta && ok0) ? beta[c0] : 0.0f, be1 = (beta && ok1) ? beta[c1] : 0.0f;
        constexpr float inv_m = 1.0f / 64.0f;
        // around the group's first channel k (tile 0, this half's first lane),
        // as for the smaller groups: h_c - h_k = (acc_c - acc_k) + (b_c - b_k)
        const float bk = group_first<32>(bb0);
        const float db0 = bb0 - bk, db1 = bb1 - bk;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float ak = group_first<32>(acc[i][0][r]);
                const float h0 = (acc[i][0][r] - ak) + db0, h1 = (acc[i][1][r] - ak) + db1;
                const float s1 = group_lanes_sum<32>(h0) + group_lanes_sum<32>(h1);
                const float d0 = h0 - s1 * inv_m, d1 = h1 - s1 * inv_m;
                const float s2 = group_lanes_sum<32>(d0 * d0) + group_lanes_sum<32>(d1 * d1);
                const float rstd = 1.0f / sqrtf(s2 * inv_m + eps);
                const int row = m0w + i * 32 + (r >> 2) * 8 + lh * 4 + (r & 3);
                if (row < M) {
                    if (ok0) out[(int64_t)row * N + c0] = gn_out(d0, rstd, g0, be0, slope);
                    if (ok1) out[(int64_t)row * N + c1] = gn_out(d1, rstd, g1, be1, slope);
                    if (mean_out && ok0 && li == 0) {  // the group's first lane: (row, group) statistics
                        const int64_t gi = (int64_t)row * (N / 64) + c0 / 64;
                        mean_out[gi] = (ak + bk) + s1 * inv_m;
                        rstd_out[gi] = rstd;
                    }
                }
            }
    }
}

// GM = 0: write h = x W^T + b to `out`.  GM = 4, 8, 16, 32 or 64 (channels
// per group): the GroupNorm -> LeakyReLU -> x + x epilogue runs on the
// accumulators and `out` receives y; h never goes to memory.  In a 32 x 32
// MFMA tile a lane holds one column (channel) for 16 rows, so the 16
// channels of a group are the 16 lanes of one DPP row (GM = 32: two
// adjacent DPP rows; GM = 4, 8: part of one; GM = 64: both of the wave's
// tiles), and each row's group statistics are a lane reduction per
// register, two-pass in registers.
//
// Software pipeline over K: while the waves multiply slice k out of one LDS
// buffer, the loads of slice k+1 are in flight into registers; they are
// written to the other buffer afterwards, so one barrier per slice
// suffices.  (Prefetching two slices ahead doubled the register footprint
// and halved occupancy; measured slower.)
template <bool VEC, int GM, int WM>
__global__ void __launch_bounds__(Tile<WM>::kThreads)
fc_mfma_kernel(const float* __restrict__ x, const float* __restrict__ W, const float* __restrict__ bias,
               const float* __restrict__ gamma, const float* __restrict__ beta, float* __restrict__ out, int M,
               int N, int K, float eps, float slope, float* __restrict__ mean_out, float* __restrict__ rstd_out)
{
    using T = Tile<WM>;
    __shared__ __attribute__((aligned(16))) float As[2][T::kBM * kLdsRow];
    __shared__ __attribute__((aligned(16))) float Bs[2][kBN * kLdsRow];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * T::kBM;
    const int n0 = blockIdx.x * kBN;
    const int li = lane & 31;  // row / column inside a 32 x 32 tile
    const int lh = lane >> 5;  // which half of the k pair

    f16v acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f16v(0.0f);

    f4 ra[T::kVecsA], rb[T::kVecsB];
    load_slice<VEC, WM>(x, W, M, N, K, m0, n0, 0, ra, rb);
    store_slice<WM>(As[0], Bs[0], ra, rb);
    __syncthreads();

    const int nk = (K + kBK - 1) / kBK;
    for (int it = 0; it < nk; ++it) {
        const int cur = it & 1;
        if (it + 1 < nk) load_slice<VEC, WM>(x, W, M, N, K, m0, n0, (it + 1) * kBK, ra, rb);
        const float* A = As[cur];
        const float* B = Bs[cur];
#pragma unroll
        for (int kq = 0; kq < kBK / 8; ++kq) {
            f4 av[2], bv[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                av[t] = *reinterpret_cast<const f4*>(A + (wm * 64 + t * 32 + li) * kLdsRow + kq * 8 + lh * 4);
                bv[t] = *reinterpret_cast<const f4*>(B + (wn * 64 + t * 32 + li) * kLdsRow + kq * 8 + lh * 4);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i][e], bv[j][e], acc[i][j], 0, 0, 0);
        }
        if (it + 1 < nk) store_slice<WM>(As[cur ^ 1], Bs[cur ^ 1], ra, rb);
        __syncthreads();
    }

    fc_epilogue<GM>(acc, bias, gamma, beta, out, M, N, m0 + wm * 64, n0 + wn * 64, li, lh, eps, slope, mean_out,
                    rstd_out);
}

// Direct-to-LDS variant (K a multiple of 32, 16-byte aligned rows): the
// K slices of x and W are copied from global memory straight into LDS with
// gfx950's global_load_lds_dwordx4 (lane l of a wave fills bytes
// [16 l, 16 l + 16) of the wave's 1 KiB destination), so no VGPRs stage
// them and no ds_write is issued.  Three LDS stages (3 x 48 KiB): slices
// it+1 and it+2 are in flight while slice it is multiplied, and one barrier
// per slice, placed before its last k step, hands slice it's stage to the
// copies of slice it+3.  LDS rows are 128 bytes
// (32 floats, eight 16-byte chunks) without padding; chunk c of row r is
// stored at position c ^ (r & 7), so the eight rows a group of lanes reads
// at one k land in eight different bank groups.  Rows beyond M or N read a
// clamped (valid) row; their results are never stored.
#ifndef NORMFWD_FC_DMA
#define NORMFWD_FC_DMA 1
#endif
constexpr int kDmaStages = 3;
constexpr int kDmaBM = 256, kDmaThreads = 512;
constexpr int kDmaStageFloats = (kDmaBM + kBN) * 32;
typedef __attribute__((address_space(3))) void lds_void_t;

template <int GM>
__global__ void __launch_bounds__(kDmaThreads)
fc_dma_kernel(const float* __restrict__ x, const float* __restrict__ W, const float* __restrict__ bias,
              const float* __restrict__ gamma, const float* __restrict__ beta, float* __restrict__ out, int M, int N,
              int K, float eps, float slope, float* __restrict__ mean_out, float* __restrict__ rstd_out)
{
    __shared__ __attribute__((aligned(16))) float lds[kDmaStages * kDmaStageFloats];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * kDmaBM;
    const int n0 = blockIdx.x * kBN;
    const int li = lane & 31;  // row / column inside a 32 x 32 tile
    const int lh = lane >> 5;  // which half of the k pair
    const int nk = K / 32;

    // This wave's share of one slice: A chunks q = (i * 8 + wave) * 64 + lane
    // for i < 4 (256 rows x 8 chunks), B chunks likewise for i < 2.
    auto issue = [&](int slice, int stage) __attribute__((always_inline)) {
        float* base = lds + stage * kDmaStageFloats;
        const int k0 = slice * 32;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = (i * 8 + wave) * 64 + lane;
            const int row = q >> 3, chunk = (q & 7) ^ (row & 7);
            const int grow = min(m0 + row, M - 1);
            __builtin_amdgcn_global_load_lds(x + (int64_t)grow * K + k0 + chunk * 4,
                                             (lds_void_t*)(base + (i * 8 + wave) * 256), 16, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int q = (i * 8 + wave) * 64 + lane;
            const int row = q >> 3, chunk = (q & 7) ^ (row & 7);
            const int grow = min(n0 + row, N - 1);
            __builtin_amdgcn_global_load_lds(W + (int64_t)grow * K + k0 + chunk * 4,
                                             (lds_void_t*)(base + kDmaBM * 32 + (i * 8 + wave) * 256), 16, 0, 0);
        }
    };

    f16v acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f16v(0.0f);

    // byte offset of this lane's 16 bytes for logical chunk c of its rows: rows
    // r = w*64 + t*32 + li have r & 7 == li & 7
    const int swz = li & 7;
    // Slice it's last k step is multiplied after the barrier, so the first
    // operand reads of slice it+1 (issued right after the barrier) land while
    // those MFMAs run; slice it+3 goes into slice it's stage, whose reads
    // have all completed (lgkmcnt(0) before the barrier).
    f4 av[2][2], bv[2][2];
    auto read = [&](const float* A, int kq, int buf) __attribute__((always_inline)) {
        const float* B = A + kDmaBM * 32;
        const int chunk = ((kq * 2 + lh) ^ swz) * 4;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            av[buf][t] = *reinterpret_cast<const f4*>(A + (wm * 64 + t * 32 + li) * 32 + chunk);
            bv[buf][t] = *reinterpret_cast<const f4*>(B + (wn * 64 + t * 32 + li) * 32 + chunk);
        }
    };
    auto mfma_step = [&](int cb) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[cb][i][e], bv[cb][j][e], acc[i][j], 0, 0, 0);
    };
    issue(0, 0);
    issue(nk > 1 ? 1 : 0, 1);
    issue(nk > 2 ? 2 : nk - 1, 2);
    asm volatile("s_waitcnt vmcnt(12)\n\ts_barrier" ::: "memory");  // slice 0 is in LDS
    read(lds, 0, 0);
    for (int it = 0; it < nk; ++it) {
        const float* A = lds + (it % kDmaStages) * kDmaStageFloats;
#pragma unroll
        for (int kq = 0; kq < 3; ++kq) {
            read(A, kq + 1, (kq + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
            mfma_step(kq & 1);
        }
        // this wave's copies of slice it+1 are done (slice it+2's, 6 more,
        // may be in flight) and its reads of slice it have landed; after the
        // barrier the same holds for every wave
        asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        issue(it + 3 < nk ? it + 3 : nk - 1, it % kDmaStages);
        if (it + 1 < nk) read(lds + ((it + 1) % kDmaStages) * kDmaStageFloats, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        mfma_step(1);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no copy outlives the workgroup's LDS
    fc_epilogue<GM>(acc, bias, gamma, beta, out, M, N, m0 + wm * 64, n0 + wn * 64, li, lh, eps, slope, mean_out,
                    rstd_out);
}

template <int GM>
static hipError_t launch_gemm(bool vec, const float* x, const float* W, const float* b, const float* gamma,
                              const float* beta, float* out, int64_t N, int64_t K, int64_t C, float eps, float slope,
                              float* mo, float* ro, hipStream_t st)
{
    if (NORMFWD_FC_DMA && vec && K >= 32 && K % 32 == 0) {
        const dim3 g((unsigned)ceil_div(C, kBN), (unsigned)ceil_div(N, kDmaBM));
        return launch_kernel((fc_dma_kernel<GM>), g, dim3(kDmaThreads), 0, st, x, W, b, gamma, beta, out, (int)N,
                             (int)C, (int)K, eps, slope, mo, ro);
    }
    constexpr int WM = NORMFWD_FC_WM;
    using T = Tile<WM>;
    const dim3 grid((unsigned)ceil_div(C, kBN), (unsigned)ceil_div(N, T::kBM));
    if (vec)
        return launch_kernel((fc_mfma_kernel<true, GM, WM>), grid, dim3(T::kThreads), 0, st, x, W, b, gamma, beta,
                             out, (int)N, (int)C, (int)K, eps, slope, mo, ro);
    return launch_kernel((fc_mfma_kernel<false, GM, WM>), grid, dim3(T::kThreads), 0, st, x, W, b, gamma, beta, out,
                         (int)N, (int)C, (int)K, eps, slope, mo, ro);
}

hipError_t launch_fc_gn(const float* x, const float* W, const float* b, const float* gamma, const float* beta,
                        float* y, int64_t N, int64_t K, int64_t C, int64_t G, float eps, float slope, void* ws,
                        float* mo, float* ro, hipStream_t st)
{
    // The tile loader reads 16-byte vectors along K when rows allow it.
    auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    const bool vec = K % 4 == 0 && al(x) && al(W);
    const int64_t M = C / G;
    // Groups of 4 to 64 channels (powers of two) fit in the GEMM epilogue: a
    // wave's block is 64 channels wide in two 32-channel tiles and starts at
    // a multiple of 64, so no group straddles waves.
    if (NORMFWD_FC_FUSE) {
        switch (M) {
            case 4: return launch_gemm<4>(vec, x, W, b, gamma, beta, y, N, K, C, eps, slope, mo, ro, st);
            case 8: return launch_gemm<8>(vec, x, W, b, gamma, beta, y, N, K, C, eps, slope, mo, ro, st);
            case 16: return launch_gemm<16>(vec, x, W, b, gamma, beta, y, N, K, C, eps, slope, mo, ro, st);
            case 32: return launch_gemm<32>(vec, x, W, b, gamma, beta, y, N, K, C, eps, slope, mo, ro, st);
            case 64: return launch_gemm<64>(vec, x, W, b, gamma, beta, y, N, K, C, eps, slope, mo, ro, st);
            default: break;
        }
    }
    float* h = static_cast<float*>(ws);
    hipError_t e = launch_gemm<0>(vec, x, W, b, nullptr, nullptr, h, N, K, C, eps, slope, nullptr, nullptr, st);
    if (e != hipSuccess) return e;
    return launch_gn_lrelu_x2(h, gamma, beta, y, N, C, G, eps, slope, mo, ro, st);
}

}  // namespace normfwd
