// Measurement references, not part of the normalization API: plain copies
// that price an access pattern by itself, so that each normalization
// kernel's HBM rate can be compared with what a copy of the same bytes
// reaches on the same device in the same run.
#include "common.hpp"
#include "internal.hpp"

#include <algorithm>

namespace normfwd {

// One float4 per thread, consecutive workgroups on consecutive 4 KiB
// blocks, nontemporal (streaming) loads and stores.
__global__ void __launch_bounds__(256) copy_dense_kernel(const f4* __restrict__ src, f4* __restrict__ dst, int64_t n4)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n4) st_nt(ld_nt(src + i), dst + i);
}

hipError_t launch_copy_dense(const float* src, float* dst, int64_t n, hipStream_t st)
{
    if (n % 4 != 0 || (reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(dst) & 15))
        return hipErrorInvalidValue;
    const int64_t n4 = n / 4;
    const int64_t per = max_grid_items() / 256 * 256;  // float4s per launch
    for (int64_t i0 = 0; i0 < n4; i0 += per) {
        const int64_t m = std::min(per, n4 - i0);
        const hipError_t e = launch_kernel(copy_dense_kernel, dim3((unsigned)ceil_div(m, 256)), dim3(256), 0, st,
                                           reinterpret_cast<const f4*>(src) + i0, reinterpret_cast<f4*>(dst) + i0, m);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace normfwd
