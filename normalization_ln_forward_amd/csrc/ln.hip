// LayerNorm over the trailing `inner` elements of each of `outer` samples
// (LN page "Kimi-K2.6 l1_p40", turn 1: population mean and variance per
// sample, y = (x - mean) / sqrt(var + eps) * weight + bias with elementwise
// weight and bias).
//
// One sample is 4,194,304 floats (16 MiB) in the LN page's problem, far
// more than one workgroup should reduce, so each sample is split into P
// contiguous chunks (LN page, turn 2: many blocks per sample write partial
// moments to a workspace, a small step reduces them per sample, a third
// pass normalizes).
//
// Numerics (the page's own one-pass E[x^2] - mean^2 loses everything when
// |mean| >> std, e.g. N(100, 0.01) data):
//   * lanes accumulate d = x - K, with K the sample's first element, in fp32
//     (for data clustered around K the subtraction is exact), one sum and
//     one sum of squares per float4 component;
//   * lane sums are widened to fp64 and reduced over the workgroup in a fixed
//     order; the chunk's moments (n, mean, M2) are stored in fp64;
//   * chunk moments are merged with Chan's pairwise update (LN page, turn 2
//     derives the same merge for Welford partials) in chunk order;
//   * the mean is handed to the normalize pass as an fp32 pair hi + lo, so
//     (x - hi) - lo keeps ~48 bits of the mean.
//
// Two schedules of the same arithmetic:
//   split  (variant 0): ln_partial_kernel -> ln_merge_kernel -> ln_normalize_kernel.
//   single (variant 1): one cooperative launch, one workgroup per chunk
//          index p; the last workgroup to deliver a sample's partial merges
//          it and publishes the statistics with an agent-scope release (LN
//          page, turn 6: last-block-done with a counter), the others wait
//          for it with acquire loads.  Workgroups run phase 1 of sample t and
//          phase 2 of sample t-1 back to back, so the second read of a
//          chunk follows the first by one sample (16 MiB of chip-wide
//          traffic) and is served from L2 / MALL instead of HBM.
#include "common.hpp"
#include "internal.hpp"

#include <algorithm>
#include <mutex>

namespace normfwd {

struct alignas(32) Partial {
    double n, mean, m2, pad;
};

struct LnCtrl {
    uint32_t gen;    // generation: incremented by the last workgroup of each single-kernel launch
    uint32_t done;   // completion counter of the current launch (returns to 0)
    uint32_t error;  // set to 1 if a wait ran past its spin limit
    uint32_t pad[61];
};
static_assert(sizeof(LnCtrl) == 256, "control block is 256 bytes");

constexpr int kLnThreads = 256;
constexpr int kLnUnroll = 4;
constexpr uint32_t kSpinLimit = 1u << 22;

static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

LnLayout ln_layout(int64_t outer, int64_t inner)
{
    LnLayout L{};
    L.P = std::min<int64_t>(1024, std::max<int64_t>(1, ceil_div(inner, 16384)));
    L.chunk = ceil_div(ceil_div(inner, L.P), 4) * 4;
    L.P_cap = std::min<int64_t>(1024, std::max<int64_t>(1, ceil_div(inner, 1024)));
    size_t off = 0;
    L.off_ctrl = off;
    off += sizeof(LnCtrl);
    L.off_counter = off;
    off += align256(4 * (size_t)outer);
    L.off_flag = off;
    off += align256(4 * (size_t)outer);
    L.off_stats = off;
    off += align256(16 * (size_t)outer);
    L.off_part = off;
    off += align256(sizeof(Partial) * (size_t)outer * (size_t)L.P_cap);
    L.total = off;
    return L;
}

// ---------------------------------------------------------------- device pieces

__device__ __forceinline__ void chan_merge(double& n, double& m, double& m2, double nb, double mb, double m2b)
{
    if (nb == 0.0) return;
    if (n == 0.0) {
        n = nb;
        m = mb;
        m2 = m2b;
        return;
    }
    const double nn = n + nb;
    const double d = mb - m;
    m = m + d * (nb / nn);
    m2 = m2 + m2b + d * d * (n * nb / nn);
    n = nn;
}

// Sum and sum of squares of (x - K) over xs[0, n), reduced over the
// workgroup; the result is valid in thread 0.  red: LDS of 2*(NT/64) doubles.
template <int VEC>
__device__ __forceinline__ void chunk_moments(const float* xs, int64_t n, float K, double* red, double& s1,
                                              double& s2)
{
    f4 a1 = f4(0.0f), a2 = f4(0.0f);
    if constexpr (VEC == 4) {
        const f4* x4 = reinterpret_cast<const f4*>(xs);
        const int64_t nv = n / 4;
        for (int64_t i = threadIdx.x; i < nv; i += kLnThreads * kLnUnroll) {
            f4 v[kLnUnroll];
#pragma unroll
            for (int u = 0; u < kLnUnroll; ++u) {
                const int64_t j = i + (int64_t)u * kLnThreads;
                v[u] = j < nv ? x4[j] : f4(K);
            }
#pragma unroll
            for (int u = 0; u < kLnUnroll; ++u) {
                const f4 d = v[u] - K;
                a1 += d;
                a2 += d * d;
            }
        }
    } else {
        for (int64_t i = threadIdx.x; i < n; i += kLnThreads) {
            const float d = xs[i] - K;
            a1.x += d;
            a2.x += d * d;
        }
    }
    double t1 = ((double)a1.x + (double)a1.y) + ((double)a1.z + (double)a1.w);
    double t2 = ((double)a2.x + (double)a2.y) + ((double)a2.z + (double)a2.w);
    t1 = wave_sum(t1);
    t2 = wave_sum(t2);
    const int wave = threadIdx.x / kWave;
    __syncthreads();  // red may still be read from a previous use
    if ((threadIdx.x & (kWave - 1)) == 0) {
        red[2 * wave] = t1;
        red[2 * wave + 1] = t2;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        s1 = red[0];
        s2 = red[1];
        for (int w = 1; w < kLnThreads / kWave; ++w) {
            s1 += red[2 * w];
            s2 += red[2 * w + 1];
        }
    }
}

__device__ __forceinline__ Partial make_partial(int64_t n, float K, double s1, double s2)
{
    Partial p{};
    if (n > 0) {
        const double dn = (double)n;
        p.n = dn;
        p.mean = (double)K + s1 / dn;
        p.m2 = fmax(s2 - s1 * (s1 / dn), 0.0);
    }
    return p;
}

// Merge parts[0, P) in a fixed order (thread t folds t, t+NT, ... then a
// fixed tree over threads); writes (mean hi, mean lo, rstd) for the sample.
// lds: 3*NT doubles.
__device__ void merge_and_publish(const Partial* parts, int64_t P, float eps, double* lds, f4* stats_b,
                                  float* mean_out_b, float* rstd_out_b)
{
    double n = 0.0, m = 0.0, m2 = 0.0;
    for (int64_t j = threadIdx.x; j < P; j += kLnThreads) {
        const Partial q = parts[j];
        chan_merge(n, m, m2, q.n, q.mean, q.m2);
    }
    double* ln_ = lds;
    double* lm = lds + kLnThreads;
    double* lm2 = lds + 2 * kLnThreads;
    __syncthreads();
    ln_[threadIdx.x] = n;
    lm[threadIdx.x] = m;
    lm2[threadIdx.x] = m2;
    __syncthreads();
    for (int stride = kLnThreads / 2; stride > 0; stride >>= 1) {
        if ((int)threadIdx.x < stride) {
            chan_merge(n, m, m2, ln_[threadIdx.x + stride], lm[threadIdx.x + stride], lm2[threadIdx.x + stride]);
            ln_[threadIdx.x] = n;
            lm[threadIdx.x] = m;
            lm2[threadIdx.x] = m2;
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const double var = n > 0.0 ? m2 / n : 0.0;
        const double rstd = 1.0 / sqrt(var + (double)eps);
        const float hi = (float)m;
        const float lo = (float)(m - (double)hi);
        *stats_b = f4{hi, lo, (float)rstd, 0.0f};
        if (mean_out_b) *mean_out_b = hi;
        if (rstd_out_b) *rstd_out_b = (float)rstd;
    }
}

// y = (((x - hi) - lo) * rstd) * w + b over xs/ys[0, n); w/b already
// offset to the same position in the sample.
template <int VEC>
__device__ __forceinline__ void normalize_range(const float* xs, const float* ws, const float* bs, float* ys,
                                                int64_t n, f4 st)
{
    const float hi = st.x, lo = st.y, rs = st.z;
    if constexpr (VEC == 4) {
        const f4* x4 = reinterpret_cast<const f4*>(xs);
        const f4* w4 = reinterpret_cast<const f4*>(ws);
        const f4* b4 = reinterpret_cast<const f4*>(bs);
        f4* y4 = reinterpret_cast<f4*>(ys);
        const int64_t nv = n / 4;
        for (int64_t i = threadIdx.x; i < nv; i += kLnThreads * kLnUnroll) {
            f4 v[kLnUnroll], wv[kLnUnroll], bv[kLnUnroll];
#pragma unroll
            for (int u = 0; u < kLnUnroll; ++u) {
                const int64_t j = i + (int64_t)u * kLnThreads;
                if (j < nv) {
                    v[u] = ld_nt(x4 + j);
                    wv[u] = ws ? w4[j] : f4(1.0f);
                    bv[u] = bs ? b4[j] : f4(0.0f);
                }
            }
#pragma unroll
            for (int u = 0; u < kLnUnroll; ++u) {
                const int64_t j = i + (int64_t)u * kLnThreads;
                if (j < nv) {
                    const f4 t = ((v[u] - hi) - lo) * rs;
                    st_nt(t * wv[u] + bv[u], y4 + j);
                }
            }
        }
    } else {
        for (int64_t i = threadIdx.x; i < n; i += kLnThreads) {
            const float t = ((xs[i] - hi) - lo) * rs;
            const float wv = ws ? ws[i] : 1.0f;
            const float bv = bs ? bs[i] : 0.0f;
            ys[i] = t * wv + bv;
        }
    }
}

// ---------------------------------------------------------------- split variant

template <int VEC>
__global__ void __launch_bounds__(kLnThreads)
ln_partial_kernel(const float* x, int64_t inner, int64_t chunk, int64_t P, int64_t P_cap, Partial* parts)
{
    __shared__ double red[2 * kLnThreads / kWave];
    const int64_t b = blockIdx.x / P;
    const int64_t p = blockIdx.x - b * P;
    const int64_t start = p * chunk;
    const int64_t n = std::max<int64_t>(0, std::min<int64_t>(inner, start + chunk) - start);
    const float* xb = x + b * inner;
    const float K = xb[0];
    double s1 = 0.0, s2 = 0.0;
    chunk_moments<VEC>(xb + start, n, K, red, s1, s2);
    if (threadIdx.x == 0) parts[b * P_cap + p] = make_partial(n, K, s1, s2);
}

__global__ void __launch_bounds__(kLnThreads)
ln_merge_kernel(const Partial* parts, int64_t P, int64_t P_cap, float eps, f4* stats, float* mean_out,
                float* rstd_out)
{
    __shared__ double lds[3 * kLnThreads];
    const int64_t b = blockIdx.x;
    merge_and_publish(parts + b * P_cap, P, eps, lds, stats + b, mean_out ? mean_out + b : nullptr,
                      rstd_out ? rstd_out + b : nullptr);
}

// Blocks are mapped so that the blocks one XCD runs back to back share the
// same chunk q of weight/bias across samples (workgroups go to the 8 XCDs
// round-robin by index): the XCD fetches that chunk of w/b into its L2 once
// and reuses it for every sample.
template <int VEC>
__global__ void __launch_bounds__(kLnThreads)
ln_normalize_kernel(const float* x, const float* w, const float* bias, float* y, int64_t outer, int64_t inner,
                    int64_t Q, int64_t cq, int xcd_map, const f4* stats)
{
    int64_t b, q;
    const int64_t i = blockIdx.x;
    if (xcd_map) {
        const int64_t xcd = i & 7, r = i >> 3;
        b = r % outer;
        q = (r / outer) * 8 + xcd;
    } else {
        b = i / Q;
        q = i - b * Q;
    }
    const int64_t start = q * cq;
    const int64_t n = std::max<int64_t>(0, std::min<int64_t>(inner, start + cq) - start);
    const f4 st = stats[b];
    const int64_t o = b * inner + start;
    normalize_range<VEC>(x + o, w ? w + start : nullptr, bias ? bias + start : nullptr, y + o, n, st);
}

// ---------------------------------------------------------------- single-kernel variant

template <int VEC>
__global__ void __launch_bounds__(kLnThreads)
ln_single_kernel(const float* x, const float* w, const float* bias, float* y, int64_t outer, int64_t inner,
                 int64_t chunk, int64_t P_cap, float eps, LnCtrl* ctrl, uint32_t* counter, uint32_t* flag,
                 f4* stats, Partial* parts, float* mean_out, float* rstd_out)
{
    __shared__ double lds[3 * kLnThreads];
    __shared__ int s_last;
    const int64_t P = gridDim.x;
    const int64_t p = blockIdx.x;
    const int64_t start = p * chunk;
    const int64_t n = std::max<int64_t>(0, std::min<int64_t>(inner, start + chunk) - start);
    const uint32_t target = __hip_atomic_load(&ctrl->gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;

    for (int64_t t = 0; t <= outer; ++t) {
        if (t < outer) {
            // phase 1: moments of chunk p of sample t
            const float* xb = x + t * inner;
            const float K = xb[0];
            double s1 = 0.0, s2 = 0.0;
            chunk_moments<VEC>(xb + start, n, K, lds, s1, s2);
            if (threadIdx.x == 0) {
                parts[t * P_cap + p] = make_partial(n, K, s1, s2);
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                const uint32_t old =
                    __hip_atomic_fetch_add(&counter[t], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
                s_last = (old == (uint32_t)(P - 1));
            }
            __syncthreads();
            if (s_last) {
                // every partial of sample t has been released: merge in chunk order
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                merge_and_publish(parts + t * P_cap, P, eps, lds, stats + t, mean_out ? mean_out + t : nullptr,
                                  rstd_out ? rstd_out + t : nullptr);
                if (threadIdx.x == 0) {
                    __hip_atomic_store(&counter[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                    __hip_atomic_store(&flag[t], target, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
        if (t >= 1) {
            // phase 2: normalize chunk p of sample t-1 once its statistics are published
            const int64_t s = t - 1;
            if (threadIdx.x == 0) {
                uint32_t it = 0;
                while (__hip_atomic_load(&flag[s], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) != target) {
                    __builtin_amdgcn_s_sleep(1);
                    if (++it > kSpinLimit) {
                        __hip_atomic_store(&ctrl->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                }
            }
            __syncthreads();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            const f4 st = stats[s];
            const int64_t o = s * inner + start;
            normalize_range<VEC>(x + o, w ? w + start : nullptr, bias ? bias + start : nullptr, y + o, n, st);
        }
    }
    // completion: the last workgroup out resets the counter and advances the generation
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&ctrl->done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (old == (uint32_t)(P - 1)) {
            __hip_atomic_store(&ctrl->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&ctrl->gen, target, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ---------------------------------------------------------------- launchers

__global__ void __launch_bounds__(256) zero_words_kernel(uint32_t* p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

hipError_t launch_zero_words(void* p, size_t bytes, hipStream_t st)
{
    const int64_t n = (int64_t)(bytes / 4);
    const int64_t blocks = std::min<int64_t>(1024, std::max<int64_t>(1, ceil_div(n, 256)));
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)blocks), dim3(256), 0, st, static_cast<uint32_t*>(p), n);
    return hipGetLastError();
}

static bool is_aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

hipError_t launch_ln_stats(const float* x, int64_t outer, int64_t inner, float eps, void* ws,
                           const LnLayout& lay, float* mean_out, float* rstd_out, hipStream_t st)
{
    char* base = static_cast<char*>(ws);
    Partial* parts = reinterpret_cast<Partial*>(base + lay.off_part);
    f4* stats = reinterpret_cast<f4*>(base + lay.off_stats);
    const bool vec4 = (inner % 4 == 0) && is_aligned16(x);
    const dim3 grid((unsigned)(outer * lay.P));
    if (vec4)
        hipLaunchKernelGGL(ln_partial_kernel<4>, grid, dim3(kLnThreads), 0, st, x, inner, lay.chunk, lay.P,
                           lay.P_cap, parts);
    else
        hipLaunchKernelGGL(ln_partial_kernel<1>, grid, dim3(kLnThreads), 0, st, x, inner, lay.chunk, lay.P,
                           lay.P_cap, parts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(ln_merge_kernel, dim3((unsigned)outer), dim3(kLnThreads), 0, st, parts, lay.P, lay.P_cap,
                       eps, stats, mean_out, rstd_out);
    return hipGetLastError();
}

hipError_t launch_ln_apply(const float* x, const float* w, const float* b, float* y, int64_t outer,
                           int64_t inner, const void* ws, const LnLayout& lay, hipStream_t st)
{
    const f4* stats = reinterpret_cast<const f4*>(static_cast<const char*>(ws) + lay.off_stats);
    const bool vec4 = (inner % 4 == 0) && is_aligned16(x) && is_aligned16(y) && is_aligned16(w) && is_aligned16(b);
    // Q blocks per sample, each over a contiguous range of cq elements (a
    // multiple of 4); Q is a multiple of 8 when the XCD mapping is used.
    int64_t Q = std::max<int64_t>(1, ceil_div(inner, 16384));
    int xcd_map = 0;
    if (Q >= 8) {
        Q = ceil_div(Q, 8) * 8;
        xcd_map = 1;
    }
    const int64_t cq = ceil_div(ceil_div(inner, Q), 4) * 4;
    const dim3 grid((unsigned)(outer * Q));
    if (vec4)
        hipLaunchKernelGGL(ln_normalize_kernel<4>, grid, dim3(kLnThreads), 0, st, x, w, b, y, outer, inner, Q, cq,
                           xcd_map, stats);
    else
        hipLaunchKernelGGL(ln_normalize_kernel<1>, grid, dim3(kLnThreads), 0, st, x, w, b, y, outer, inner, Q, cq,
                           xcd_map, stats);
    return hipGetLastError();
}

// Co-resident workgroups of ln_single_kernel per device (queried once).
static int single_capacity(bool vec4)
{
    static std::mutex mu;
    static int cap[2][64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lock(mu);
    int& c = cap[vec4 ? 1 : 0][dev];
    if (c == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        const void* fn = vec4 ? reinterpret_cast<const void*>(&ln_single_kernel<4>)
                              : reinterpret_cast<const void*>(&ln_single_kernel<1>);
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kLnThreads, 0) != hipSuccess) return 0;
        c = cus * per_cu;
    }
    return c;
}

hipError_t launch_ln_single(const float* x, const float* w, const float* b, float* y, int64_t outer,
                            int64_t inner, float eps, void* ws, const LnLayout& lay, float* mean_out,
                            float* rstd_out, hipStream_t st)
{
    char* base = static_cast<char*>(ws);
    LnCtrl* ctrl = reinterpret_cast<LnCtrl*>(base + lay.off_ctrl);
    uint32_t* counter = reinterpret_cast<uint32_t*>(base + lay.off_counter);
    uint32_t* flag = reinterpret_cast<uint32_t*>(base + lay.off_flag);
    f4* stats = reinterpret_cast<f4*>(base + lay.off_stats);
    Partial* parts = reinterpret_cast<Partial*>(base + lay.off_part);
    const bool vec4 = (inner % 4 == 0) && is_aligned16(x) && is_aligned16(y) && is_aligned16(w) && is_aligned16(b);
    const int cap = single_capacity(vec4);
    if (cap <= 0) return hipErrorInvalidDevice;
    // One workgroup per chunk index; at most the co-resident count, at most
    // the workspace's partial slots, and chunks of at least 1024 elements.
    int64_t P = std::min<int64_t>({(int64_t)cap, lay.P_cap, std::max<int64_t>(1, ceil_div(inner, 1024))});
    // Prefer a multiple of 256 workgroups (whole waves of CUs) when large.
    if (P > 256) P = (P / 256) * 256;
    const int64_t chunk = ceil_div(ceil_div(inner, P), 4) * 4;
    int64_t pcap = lay.P_cap;
    void* args[] = {(void*)&x, (void*)&w, (void*)&b, (void*)&y, (void*)&outer, (void*)&inner, (void*)&chunk,
                    (void*)&pcap, (void*)&eps, (void*)&ctrl, (void*)&counter, (void*)&flag, (void*)&stats,
                    (void*)&parts, (void*)&mean_out, (void*)&rstd_out};
    const void* fn = vec4 ? reinterpret_cast<const void*>(&ln_single_kernel<4>)
                          : reinterpret_cast<const void*>(&ln_single_kernel<1>);
    hipError_t e = hipLaunchCooperativeKernel(fn, dim3((unsigned)P), dim3(kLnThreads), args, 0, st);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace normfwd
