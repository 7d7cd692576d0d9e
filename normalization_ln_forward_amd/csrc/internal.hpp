// Host-side launchers behind the C ABI (one translation unit per operation).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace normfwd {

// Events armed by normfwd_time_next_kernel on the calling thread; taking
// them disarms them.
struct LaunchEvents {
    hipEvent_t start;
    hipEvent_t stop;
};
LaunchEvents take_launch_events();

// Work-items per grid dimension of one launch are a 32-bit count, so every
// launcher splits larger problems into batches of whole samples / rows of at
// most max_grid_items() work-items (2^31; the environment variable
// NORMFWD_MAX_GRID_ITEMS, read once, can lower it so that tests exercise the
// batching on small tensors).
int64_t max_grid_items();

// Every kernel launch of the library goes through here: it refuses a grid
// whose work-item count does not fit 32 bits (instead of letting it wrap),
// and an armed pair of events is recorded by the first launch after arming
// (hipExtLaunchKernel stamps the kernel's own start and end; no marker
// packets are added).
template <typename F, typename... Args>
inline hipError_t launch_kernel(F kernel, const dim3& grid, const dim3& block, uint32_t shmem, hipStream_t st,
                                Args... args)
{
    constexpr uint64_t kMax = 0xFFFFFFFFull;
    if ((uint64_t)grid.x * block.x > kMax || (uint64_t)grid.y * block.y > kMax || (uint64_t)grid.z * block.z > kMax ||
        grid.x == 0 || grid.y == 0 || grid.z == 0)
        return hipErrorInvalidConfiguration;
    const LaunchEvents ev = take_launch_events();
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, ev.start, ev.stop, 0u, args...);
    return hipGetLastError();
}

// Samples (rows) per launch when one sample needs `items_per_sample`
// work-items: at least 1, at most what keeps a launch under max_grid_items().
inline int64_t samples_per_launch(int64_t items_per_sample)
{
    return items_per_sample >= max_grid_items() ? 1 : max_grid_items() / items_per_sample;
}

// Element strides of a [B, C, S] view whose S positions of one (b, c) are
// contiguous: x at b * xsb + c * xsc + s, y at b * ysb + c * ysc + s.
struct RmsStrides {
    int64_t xsb, xsc, ysb, ysc;
};
// rstd: [B, S] (1 / sqrt(ms + eps) per position) or NULL.
hipError_t launch_rms_ch(const float* x, float* y, int64_t B, int64_t C, int64_t S, float eps, const RmsStrides& L,
                         float* rstd, hipStream_t st);

// mean_out, rstd_out: [N, G] or NULL (both or neither).
hipError_t launch_gn_lrelu_x2(const float* x, const float* gamma, const float* beta, float* y, int64_t N,
                              int64_t C, int64_t G, float eps, float slope, float* mean_out, float* rstd_out,
                              hipStream_t st);

// LayerNorm workspace: byte offsets of each region (all 256-byte aligned).
struct LnLayout {
    int64_t P;        // partial-moment workgroups per sample, split variant
    int64_t P_cap;    // partial-moment slots per sample (>= chunks of either variant)
    size_t off_ctrl;  // control block: generation, completion counter, error word
    size_t off_counter;  // single kernel: ring of arrival counters
    size_t off_split_counter;  // split schedule: per-sample arrival counters (128-byte lines)
    size_t off_stats;
    size_t off_part;
    size_t off_xchg;  // control-wave kernel's exchange: per sample, P_cap tagged means then P_cap tagged M2s
    size_t off_lbd;   // control-wave kernel, last workgroup merging: per sample, tagged mean and rstd (fp64)
    size_t off_lbdx;  // ... and its workgroups' moments: per sample, P_cap tagged means then P_cap tagged M2s
    size_t total;
};
// Byte offset, in an LN workspace, of the word the single kernels set when
// a wait gives up (the control block starts every LN workspace).
constexpr size_t kLnErrorWordOffset = 8;
// Byte offset of the control-wave kernel's count of workgroup sums that a
// reader computed itself (after waiting past its spin limit, or forced).
constexpr size_t kLnRecomputedWordOffset = 12;
// Byte offset of the control-wave kernel's generation (launches so far on
// the workspace, mod 255); its exchange tags derive from it.
constexpr size_t kLnCtlGenWordOffset = 16;
// Test knob, read once from NORMFWD_LN_FORCE_RECOMPUTE (0 = off): a power of
// two k makes the control-wave kernel ignore the published sums of every
// workgroup j with j % k == k - 1 and compute them from x instead, which
// must give bitwise the same result (other values are ignored).
uint32_t ln_force_recompute();
LnLayout ln_layout(int64_t outer, int64_t inner);

hipError_t launch_ln_stats(const float* x, int64_t outer, int64_t inner, float eps, void* ws,
                           const LnLayout& lay, float* mean_out, float* rstd_out, hipStream_t st);
hipError_t launch_ln_apply(const float* x, const float* w, const float* b, float* y, int64_t outer,
                           int64_t inner, const void* ws, const LnLayout& lay, hipStream_t st);
// One workgroup per sample when the sample fits its registers (inner <=
// 8192 with 128-bit access, <= 2048 otherwise); false if it does not.
bool launch_ln_rows(const float* x, const float* w, const float* b, float* y, int64_t outer, int64_t inner, float eps,
                    float* mean_out, float* rstd_out, hipStream_t st, hipError_t& err);
// ln_single_ctl_kernel with its control wave running protocol 1 (the
// generation-tagged gather, an ordinary launch) or 2 (the last workgroup of
// a sample merges it, a cooperative launch).  Shapes the kernel cannot hold
// run the split schedule.
hipError_t launch_ln_single(const float* x, const float* w, const float* b, float* y, int64_t outer,
                            int64_t inner, float eps, void* ws, const LnLayout& lay, float* mean_out,
                            float* rstd_out, int protocol, hipStream_t st);

// ln_forward variant 3: the schedule measured fastest for this shape on this
// device (1 = the control-wave single kernel, else 0 = split).
int ln_auto_variant(const float* x, const float* w, const float* b, const float* y, int64_t outer, int64_t inner);

// Fill bytes/4 32-bit words with zero (a kernel, not a memset, so the call
// can sit inside a captured HIP graph).
hipError_t launch_zero_words(void* p, size_t bytes, hipStream_t st);

// Measurement references (plain copies): a dense streaming copy of n
// floats, and rmsnorm_ch_forward's access pattern without its arithmetic.
hipError_t launch_copy_dense(const float* src, float* dst, int64_t n, hipStream_t st);
hipError_t launch_rms_copy_pattern(const float* x, float* y, int64_t B, int64_t C, int64_t S, hipStream_t st);

hipError_t launch_fc_gn(const float* x, const float* W, const float* b, const float* gamma, const float* beta,
                        float* y, int64_t N, int64_t K, int64_t C, int64_t G, float eps, float slope, void* ws,
                        float* mean_out, float* rstd_out, hipStream_t st);

}  // namespace normfwd
