// fc -> GroupNorm -> LeakyReLU -> x + x
// (GN page "Kimi-K2.6 l2_p62", turn 1: h = x W^T + b with x [N, K] and W
// [C, K] row-major, then the GroupNorm epilogue on h).
//
// The fc is an fp32 GEMM on the matrix cores (v_mfma_f32_32x32x2_f32, exact
// fp32 products with fp32 accumulation; no reduced-precision inputs).  Both
// operands are K-contiguous, so a workgroup stages a BM x BK tile of x and a
// BN x BK tile of W in LDS (rows padded by 4 floats against bank conflicts)
// and each of its four waves computes a 64 x 64 block of h as 2 x 2 MFMA
// tiles.  Within one MFMA the two k values a lane pair contributes are free
// to choose as long as x and W agree, so each lane reads 4 consecutive k of
// its row with one 128-bit LDS read and feeds them to 4 successive MFMAs.
// h goes to the workspace; the GroupNorm kernel then reads it back.
#include "common.hpp"
#include "internal.hpp"

namespace normfwd {

typedef float f16v __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 128, kBK = 32, kPad = 4;
constexpr int kLdsRow = kBK + kPad;

template <bool VEC>
__global__ void __launch_bounds__(256)
fc_mfma_kernel(const float* __restrict__ x, const float* __restrict__ W, const float* __restrict__ bias,
               float* __restrict__ h, int M, int N, int K)
{
    __shared__ __attribute__((aligned(16))) float As[kBM * kLdsRow];
    __shared__ __attribute__((aligned(16))) float Bs[kBN * kLdsRow];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * kBM;
    const int n0 = blockIdx.x * kBN;
    const int li = lane & 31;  // row / column inside a 32 x 32 tile
    const int lh = lane >> 5;  // which half of the k pair

    f16v acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f16v(0.0f);

    for (int k0 = 0; k0 < K; k0 += kBK) {
        // stage: each of A and B is 128 rows x 8 float4
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int idx = tid + 256 * u;
            const int r = idx >> 3, c = (idx & 7) * 4;
            const int k = k0 + c;
            f4 a = f4(0.0f), b = f4(0.0f);
            if constexpr (VEC) {  // K % 4 == 0 and 16-byte aligned rows
                if (m0 + r < M && k < K) a = *reinterpret_cast<const f4*>(x + (int64_t)(m0 + r) * K + k);
                if (n0 + r < N && k < K) b = *reinterpret_cast<const f4*>(W + (int64_t)(n0 + r) * K + k);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (m0 + r < M && k + q < K) a[q] = x[(int64_t)(m0 + r) * K + k + q];
                    if (n0 + r < N && k + q < K) b[q] = W[(int64_t)(n0 + r) * K + k + q];
                }
            }
            *reinterpret_cast<f4*>(As + r * kLdsRow + c) = a;
            *reinterpret_cast<f4*>(Bs + r * kLdsRow + c) = b;
        }
        __syncthreads();
#pragma unroll
        for (int kq = 0; kq < kBK / 8; ++kq) {
            f4 av[2], bv[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                av[t] = *reinterpret_cast<const f4*>(As + (wm * 64 + t * 32 + li) * kLdsRow + kq * 8 + lh * 4);
                bv[t] = *reinterpret_cast<const f4*>(Bs + (wn * 64 + t * 32 + li) * kLdsRow + kq * 8 + lh * 4);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i][e], bv[j][e], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }

    // D layout of a 32 x 32 tile: lane holds column (lane % 32); register r
    // holds row (r / 4) * 8 + (lane / 32) * 4 + r % 4.
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + wn * 64 + j * 32 + li;
            if (col >= N) continue;
            const float bb = bias ? bias[col] : 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + lh * 4 + (r & 3);
                if (row < M) h[(int64_t)row * N + col] = acc[i][j][r] + bb;
            }
        }
}

hipError_t launch_fc_gn(const float* x, const float* W, const float* b, const float* gamma, const float* beta,
                        float* y, int64_t N, int64_t K, int64_t C, int64_t G, float eps, float slope, void* ws,
                        hipStream_t st)
{
    // The tile loader reads 16-byte vectors along K when rows allow it.
    auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    const bool vec = K % 4 == 0 && al(x) && al(W);
    float* h = static_cast<float*>(ws);
    const dim3 grid((unsigned)ceil_div(C, kBN), (unsigned)ceil_div(N, kBM));
    if (vec)
        hipLaunchKernelGGL(fc_mfma_kernel<true>, grid, dim3(256), 0, st, x, W, b, h, (int)N, (int)C, (int)K);
    else
        hipLaunchKernelGGL(fc_mfma_kernel<false>, grid, dim3(256), 0, st, x, W, b, h, (int)N, (int)C, (int)K);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_gn_lrelu_x2(h, gamma, beta, y, N, C, G, eps, slope, st);
}

}  // namespace normfwd
