// C ABI of libnormfwd: argument validation, status reporting and dispatch
// to the per-operation launchers.  Declarations and contracts are in
// include/normfwd.h.
#include "normfwd.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <mutex>
#include <utility>

#include "internal.hpp"

namespace {

thread_local char g_last_error[512] = "";

normfwd_status fail(normfwd_status st, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

normfwd_status ok()
{
    g_last_error[0] = '\0';
    return NORMFWD_OK;
}

normfwd_status hip_status(hipError_t e, const char* what)
{
    if (e == hipSuccess) return ok();
    return fail(NORMFWD_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

// Largest element count one tensor may have: grid sizes and 32-bit block
// indices stay in range below this, with headroom.
constexpr int64_t kMaxElems = (int64_t)1 << 40;

bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255) == 0; }

normfwd_status check_ln(const float* x, const float* y, int64_t outer, int64_t inner, float eps)
{
    if (!x || !y) return fail(NORMFWD_ERR_INVALID, "ln: x and y must not be NULL");
    if (outer <= 0 || inner <= 0) return fail(NORMFWD_ERR_INVALID, "ln: outer (%lld) and inner (%lld) must be > 0",
                                               (long long)outer, (long long)inner);
    if (outer > kMaxElems / inner) return fail(NORMFWD_ERR_UNSUPPORTED, "ln: outer*inner too large");
    if (outer > ((int64_t)1 << 22)) return fail(NORMFWD_ERR_UNSUPPORTED, "ln: outer > 2^22 samples");
    if (inner > ((int64_t)1 << 31)) return fail(NORMFWD_ERR_UNSUPPORTED, "ln: inner > 2^31 elements per sample");
    if (!(eps >= 0.0f)) return fail(NORMFWD_ERR_INVALID, "ln: eps must be >= 0");
    return ok();
}

normfwd_status check_ws(const void* ws, size_t bytes, size_t need, const char* who)
{
    if (!ws) return fail(NORMFWD_ERR_WORKSPACE, "%s: workspace is NULL", who);
    if (!aligned256(ws)) return fail(NORMFWD_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", who);
    if (bytes < need)
        return fail(NORMFWD_ERR_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", who, bytes, need);
    return ok();
}

}  // namespace

namespace normfwd {

thread_local LaunchEvents g_armed{nullptr, nullptr};

int64_t max_grid_items()
{
    static const int64_t limit = [] {
        int64_t lim = (int64_t)1 << 31;
        if (const char* e = std::getenv("NORMFWD_MAX_GRID_ITEMS")) {
            const long long v = std::atoll(e);
            if (v >= 4096 && v < lim) lim = v;
        }
        return lim;
    }();
    return limit;
}

uint32_t ln_force_recompute()
{
    static const uint32_t k = [] {
        uint32_t v = 0;
        if (const char* e = std::getenv("NORMFWD_LN_FORCE_RECOMPUTE")) {
            const long long n = std::atoll(e);
            if (n > 0 && n <= (1ll << 30) && (n & (n - 1)) == 0) v = (uint32_t)n;
        }
        return v;
    }();
    return k;
}

LaunchEvents take_launch_events()
{
    const LaunchEvents e = g_armed;
    g_armed = LaunchEvents{nullptr, nullptr};
    return e;
}

}  // namespace normfwd

namespace {

// One ln_forward call on a workspace of the layout `lay`: one workgroup per
// sample for short samples, else the schedule `variant` selects.
normfwd_status ln_dispatch(const float* x, const float* weight, const float* bias, float* y, int64_t outer,
                           int64_t inner, float eps, void* workspace, const normfwd::LnLayout& lay, float* mean_out,
                           float* rstd_out, int variant, hipStream_t st)
{
    hipError_t re = hipSuccess;
    if (normfwd::launch_ln_rows(x, weight, bias, y, outer, inner, eps, mean_out, rstd_out, st, re))
        return hip_status(re, "ln_forward (one workgroup per sample) launch");
    if (variant == 3) variant = normfwd::ln_auto_variant(x, weight, bias, y, outer, inner);
    if (variant != 0) {
        const hipError_t e = normfwd::launch_ln_single(x, weight, bias, y, outer, inner, eps, workspace, lay,
                                                       mean_out, rstd_out, variant, st);
        // The runtime grants cooperative launches on a GPU to one process
        // at a time: once a process has made one, the same launch from
        // another process is refused until the first process exits
        // (measured on MI355X: the refused launch returns
        // hipErrorIllegalState; the first process keeps launching).
        if (e == hipErrorIllegalState)
            return fail(NORMFWD_ERR_UNSUPPORTED,
                        "ln_forward: the cooperative launch of the last-workgroup-merges kernel was refused "
                        "(hipErrorIllegalState): another process that is still running has made a cooperative "
                        "launch on this GPU; only variant 2 in place uses one");
        return hip_status(e, "ln_forward (single kernel) launch");
    }
    hipError_t e = normfwd::launch_ln_stats(x, outer, inner, eps, workspace, lay, mean_out, rstd_out, st);
    if (e != hipSuccess) return hip_status(e, "ln_forward stats launch");
    return hip_status(normfwd::launch_ln_apply(x, weight, bias, y, outer, inner, workspace, lay, st),
                      "ln_forward normalize launch");
}

// ln_forward_noalloc's workspace: a file-scope device array, one copy per
// GPU, kept until the process ends.  Host code never passes `scratch` itself
// to a kernel (on the host that name is only a stand-in for the symbol);
// it uses the device address hipGetSymbolAddress returns for the current
// device, looked up on the first call on that device.
constexpr size_t kLnScratchBytes = NORMFWD_LN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kLnScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchState {
    void* ptr = nullptr;  // device address of `scratch` on this device
    int64_t outer = -1;   // shape the scratch was last laid out for
    int64_t inner = -1;
};
std::mutex g_scratch_mu;
ScratchState g_scratch[kMaxDevices];

}  // namespace

extern "C" {

normfwd_status normfwd_time_next_kernel(void* start_event, void* stop_event)
{
    normfwd::g_armed = normfwd::LaunchEvents{static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event)};
    return ok();
}

const char* normfwd_status_string(normfwd_status s)
{
    switch (s) {
        case NORMFWD_OK: return "NORMFWD_OK";
        case NORMFWD_ERR_INVALID: return "NORMFWD_ERR_INVALID: invalid argument";
        case NORMFWD_ERR_UNSUPPORTED: return "NORMFWD_ERR_UNSUPPORTED: arguments valid but not supported";
        case NORMFWD_ERR_WORKSPACE: return "NORMFWD_ERR_WORKSPACE: workspace missing, misaligned or too small";
        case NORMFWD_ERR_HIP: return "NORMFWD_ERR_HIP: HIP runtime error";
        case NORMFWD_ERR_INCOMPLETE: return "NORMFWD_ERR_INCOMPLETE: a single-kernel launch gave up waiting";
        default: return "unknown status";
    }
}

const char* normfwd_last_error(void) { return g_last_error; }

size_t ln_forward_workspace_size(int64_t outer, int64_t inner)
{
    if (outer <= 0 || inner <= 0) return 0;
    return normfwd::ln_layout(outer, inner).total;
}

normfwd_status ln_forward_workspace_init(void* workspace, size_t workspace_bytes, void* stream)
{
    if (!workspace || workspace_bytes < 256 || !aligned256(workspace))
        return fail(NORMFWD_ERR_WORKSPACE, "ln_forward_workspace_init: need a 256-byte aligned workspace of >= 256 bytes");
    // The whole workspace is cleared: control block, counters and exchange words.
    (void)hipGetLastError();
    return hip_status(normfwd::launch_zero_words(workspace, workspace_bytes, (hipStream_t)stream),
                      "ln_forward_workspace_init launch");
}

normfwd_status ln_forward_workspace_check(void* workspace, size_t workspace_bytes, void* stream)
{
    if (!workspace || workspace_bytes < 256 || !aligned256(workspace))
        return fail(NORMFWD_ERR_WORKSPACE, "ln_forward_workspace_check: need a 256-byte aligned workspace of >= 256 bytes");
    (void)hipGetLastError();
    hipStream_t st = (hipStream_t)stream;
    char* word_ptr = static_cast<char*>(workspace) + normfwd::kLnErrorWordOffset;
    uint32_t word = 0;
    hipError_t e = hipMemcpyAsync(&word, word_ptr, sizeof(word), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_status(e, "ln_forward_workspace_check: reading the error word");
    if (word == 0) return ok();
    const uint32_t zero = 0;
    e = hipMemcpyAsync(word_ptr, &zero, sizeof(zero), hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_status(e, "ln_forward_workspace_check: clearing the error word");
    return fail(NORMFWD_ERR_INCOMPLETE,
                "a single-kernel ln_forward on this workspace gave up waiting for another workgroup; "
                "its output is not valid");
}

normfwd_status ln_forward_stats(const float* x, int64_t outer, int64_t inner, float eps, void* workspace,
                                size_t workspace_bytes, float* mean_out, float* rstd_out, void* stream)
{
    if (outer == 0 && inner >= 0) return ok();  // empty batch: nothing to do
    normfwd_status s = check_ln(x, x, outer, inner, eps);
    if (s != NORMFWD_OK) return s;
    const normfwd::LnLayout lay = normfwd::ln_layout(outer, inner);
    s = check_ws(workspace, workspace_bytes, lay.total, "ln_forward_stats");
    if (s != NORMFWD_OK) return s;
    (void)hipGetLastError();
    return hip_status(normfwd::launch_ln_stats(x, outer, inner, eps, workspace, lay, mean_out, rstd_out,
                                               (hipStream_t)stream),
                      "ln_forward_stats launch");
}

normfwd_status ln_forward_apply(const float* x, const float* weight, const float* bias, float* y, int64_t outer,
                                int64_t inner, const void* workspace, size_t workspace_bytes, void* stream)
{
    if (outer == 0 && inner >= 0) return ok();  // empty batch: nothing to do
    normfwd_status s = check_ln(x, y, outer, inner, 0.0f);
    if (s != NORMFWD_OK) return s;
    const normfwd::LnLayout lay = normfwd::ln_layout(outer, inner);
    s = check_ws(workspace, workspace_bytes, lay.total, "ln_forward_apply");
    if (s != NORMFWD_OK) return s;
    (void)hipGetLastError();
    return hip_status(normfwd::launch_ln_apply(x, weight, bias, y, outer, inner, workspace, lay, (hipStream_t)stream),
                      "ln_forward_apply launch");
}

normfwd_status ln_forward(const float* x, const float* weight, const float* bias, float* y, int64_t outer,
                          int64_t inner, float eps, void* workspace, size_t workspace_bytes, float* mean_out,
                          float* rstd_out, int variant, void* stream)
{
    if (outer == 0 && inner >= 0 && variant >= 0 && variant <= 3) return ok();  // empty batch: nothing to do
    normfwd_status s = check_ln(x, y, outer, inner, eps);
    if (s != NORMFWD_OK) return s;
    if (variant < 0 || variant > 3) return fail(NORMFWD_ERR_INVALID, "ln_forward: variant must be 0, 1, 2 or 3");
    const normfwd::LnLayout lay = normfwd::ln_layout(outer, inner);
    s = check_ws(workspace, workspace_bytes, lay.total, "ln_forward");
    if (s != NORMFWD_OK) return s;
    (void)hipGetLastError();
    return ln_dispatch(x, weight, bias, y, outer, inner, eps, workspace, lay, mean_out, rstd_out, variant,
                       (hipStream_t)stream);
}

normfwd_status ln_forward_noalloc(const float* x, const float* weight, const float* bias, float* y, int64_t outer,
                                  int64_t inner, float eps, float* mean_out, float* rstd_out, int variant,
                                  void* stream)
{
    if (outer == 0 && inner >= 0 && variant >= 0 && variant <= 3) return ok();  // empty batch: nothing to do
    normfwd_status s = check_ln(x, y, outer, inner, eps);
    if (s != NORMFWD_OK) return s;
    if (variant < 0 || variant > 3)
        return fail(NORMFWD_ERR_INVALID, "ln_forward_noalloc: variant must be 0, 1, 2 or 3");
    const normfwd::LnLayout lay = normfwd::ln_layout(outer, inner);
    if (lay.total > kLnScratchBytes)
        return fail(NORMFWD_ERR_UNSUPPORTED,
                    "ln_forward_noalloc: shape [%lld, %lld] needs %zu bytes of workspace, more than the %zu bytes "
                    "of the library's static scratch; use ln_forward with a caller workspace",
                    (long long)outer, (long long)inner, lay.total, kLnScratchBytes);
    (void)hipGetLastError();
    hipStream_t st = (hipStream_t)stream;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "ln_forward_noalloc: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(NORMFWD_ERR_UNSUPPORTED, "ln_forward_noalloc: device index %d", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ScratchState& sc = g_scratch[dev];
    if (!sc.ptr) {
        // once per device, with that device current: each GPU holds its own
        // copy of `scratch`, at its own address
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol,
                                                     "ln_forward_noalloc: hipGetSymbolAddress(scratch)");
        sc.ptr = p;
    }
    if (sc.outer != outer || sc.inner != inner) {
        // The workspace regions sit at offsets that depend on the shape: a new
        // shape starts from a zeroed scratch (a kernel, not a memset)
        e = normfwd::launch_zero_words(sc.ptr, lay.total, st);
        if (e != hipSuccess) return hip_status(e, "ln_forward_noalloc: zeroing the scratch");
        sc.outer = outer;
        sc.inner = inner;
    }
    return ln_dispatch(x, weight, bias, y, outer, inner, eps, sc.ptr, lay, mean_out, rstd_out, variant, st);
}

normfwd_status gn_lrelu_x2_forward(const float* x, const float* gamma, const float* beta, float* y, int64_t N,
                                   int64_t C, int64_t num_groups, float eps, float negative_slope, float* mean_out,
                                   float* rstd_out, void* stream)
{
    if (N == 0 && C > 0 && num_groups > 0 && C % num_groups == 0) return ok();  // no rows: nothing to do
    if (!x || !y) return fail(NORMFWD_ERR_INVALID, "gn_lrelu_x2_forward: x and y must not be NULL");
    if (N <= 0 || C <= 0 || num_groups <= 0)
        return fail(NORMFWD_ERR_INVALID, "gn_lrelu_x2_forward: N, C and num_groups must be > 0");
    if (C % num_groups != 0)
        return fail(NORMFWD_ERR_INVALID, "gn_lrelu_x2_forward: C (%lld) must be a multiple of num_groups (%lld)",
                    (long long)C, (long long)num_groups);
    if (N > kMaxElems / C || C > ((int64_t)1 << 30))
        return fail(NORMFWD_ERR_UNSUPPORTED, "gn_lrelu_x2_forward: N*C too large or C > 2^30");
    if (N * num_groups > ((int64_t)1 << 38))
        return fail(NORMFWD_ERR_UNSUPPORTED, "gn_lrelu_x2_forward: too many groups");
    if (C / num_groups > std::numeric_limits<int>::max())
        return fail(NORMFWD_ERR_UNSUPPORTED, "gn_lrelu_x2_forward: group too large");
    if (!(eps >= 0.0f)) return fail(NORMFWD_ERR_INVALID, "gn_lrelu_x2_forward: eps must be >= 0");
    if (!mean_out != !rstd_out)
        return fail(NORMFWD_ERR_INVALID, "gn_lrelu_x2_forward: give both mean_out and rstd_out, or neither");
    (void)hipGetLastError();
    return hip_status(normfwd::launch_gn_lrelu_x2(x, gamma, beta, y, N, C, num_groups, eps, negative_slope, mean_out,
                                                  rstd_out, (hipStream_t)stream),
                      "gn_lrelu_x2_forward launch");
}

normfwd_status rmsnorm_ch_forward(const float* x, float* y, int64_t B, int64_t C, int64_t S, float eps, void* stream)
{
    if ((B == 0 || S == 0) && B >= 0 && S >= 0 && C > 0) return ok();  // no positions: nothing to do
    if (!x || !y) return fail(NORMFWD_ERR_INVALID, "rmsnorm_ch_forward: x and y must not be NULL");
    if (B <= 0 || C <= 0 || S <= 0) return fail(NORMFWD_ERR_INVALID, "rmsnorm_ch_forward: B, C and S must be > 0");
    if (C > std::numeric_limits<int>::max() || S > ((int64_t)1 << 26) || B > kMaxElems / (C * S))
        return fail(NORMFWD_ERR_UNSUPPORTED, "rmsnorm_ch_forward: shape too large (C < 2^31, S <= 2^26)");
    if (!(eps >= 0.0f)) return fail(NORMFWD_ERR_INVALID, "rmsnorm_ch_forward: eps must be >= 0");
    (void)hipGetLastError();
    return hip_status(normfwd::launch_rms_ch(x, y, B, C, S, eps, normfwd::RmsStrides{C * S, S, C * S, S}, nullptr,
                                             (hipStream_t)stream),
                      "rmsnorm_ch_forward launch");
}

normfwd_status rmsnorm_ch_forward_strided(const float* x, float* y, int64_t B, int64_t C, int64_t S,
                                          int64_t x_batch_stride, int64_t x_channel_stride, int64_t y_batch_stride,
                                          int64_t y_channel_stride, float eps, float* rstd_out, void* stream)
{
    if ((B == 0 || S == 0) && B >= 0 && S >= 0 && C > 0) return ok();  // no positions: nothing to do
    if (!x || !y) return fail(NORMFWD_ERR_INVALID, "rmsnorm_ch_forward_strided: x and y must not be NULL");
    if (B <= 0 || C <= 0 || S <= 0)
        return fail(NORMFWD_ERR_INVALID, "rmsnorm_ch_forward_strided: B, C and S must be > 0");
    if (x_batch_stride < 0 || x_channel_stride < 0 || y_batch_stride < 0 || y_channel_stride < 0)
        return fail(NORMFWD_ERR_UNSUPPORTED, "rmsnorm_ch_forward_strided: negative strides are not supported");
    if (C > std::numeric_limits<int>::max() || S > ((int64_t)1 << 26) || B > kMaxElems / S || C > kMaxElems / S)
        return fail(NORMFWD_ERR_UNSUPPORTED, "rmsnorm_ch_forward_strided: shape too large (C < 2^31, S <= 2^26)");
    // the last element each tensor addresses must stay below 2^40
    auto span = [&](int64_t sb, int64_t sc) {
        const int64_t lim = kMaxElems;
        if (B > 1 && sb > (lim - S) / (B - 1)) return lim;
        if (C > 1 && sc > (lim - S) / (C - 1)) return lim;
        const int64_t a = (B - 1) * sb, c = (C - 1) * sc;
        return a > lim - S - c ? lim : a + c + S;
    };
    if (span(x_batch_stride, x_channel_stride) >= kMaxElems || span(y_batch_stride, y_channel_stride) >= kMaxElems)
        return fail(NORMFWD_ERR_UNSUPPORTED, "rmsnorm_ch_forward_strided: a view spans 2^40 elements or more");
    // y's rows of S positions must not overlap one another: ordered by
    // stride, the smaller one (if its extent is > 1) is at least S and the
    // larger one (if its extent is > 1) at least that row block
    {
        int64_t s1 = y_batch_stride, n1 = B, s2 = y_channel_stride, n2 = C;
        if (n1 == 1 || (n2 > 1 && s2 < s1)) {
            std::swap(s1, s2);
            std::swap(n1, n2);
        }
        const int64_t block = n1 > 1 ? s1 * n1 : S;
        const bool ok1 = n1 == 1 || s1 >= S;
        const bool ok2 = n2 == 1 || s2 >= block;
        if (!ok1 || !ok2)
            return fail(NORMFWD_ERR_INVALID, "rmsnorm_ch_forward_strided: y's strides make its rows overlap");
    }
    if (!(eps >= 0.0f)) return fail(NORMFWD_ERR_INVALID, "rmsnorm_ch_forward_strided: eps must be >= 0");
    (void)hipGetLastError();
    return hip_status(
        normfwd::launch_rms_ch(x, y, B, C, S, eps,
                               normfwd::RmsStrides{x_batch_stride, x_channel_stride, y_batch_stride, y_channel_stride},
                               rstd_out, (hipStream_t)stream),
        "rmsnorm_ch_forward_strided launch");
}

normfwd_status normfwd_copy_reference(const float* src, float* dst, int64_t B, int64_t C, int64_t S, int pattern,
                                      void* stream)
{
    if (!src || !dst) return fail(NORMFWD_ERR_INVALID, "normfwd_copy_reference: src and dst must not be NULL");
    if (B <= 0 || C <= 0 || S <= 0 || B > kMaxElems / C || B * C > kMaxElems / S)
        return fail(NORMFWD_ERR_INVALID, "normfwd_copy_reference: B, C, S must be > 0 (at most 2^40 elements)");
    if (pattern != 0 && pattern != 1) return fail(NORMFWD_ERR_INVALID, "normfwd_copy_reference: pattern must be 0 or 1");
    const bool al = !(reinterpret_cast<uintptr_t>(src) & 15) && !(reinterpret_cast<uintptr_t>(dst) & 15);
    if (!al || (pattern == 0 && (B * C * S) % 4 != 0) || (pattern == 1 && (S % 4 != 0 || C > 64 || S > ((int64_t)1 << 26))))
        return fail(NORMFWD_ERR_UNSUPPORTED,
                    "normfwd_copy_reference: needs 16-byte aligned buffers and a multiple of 4 floats (pattern 1: "
                    "S %% 4 == 0, C <= 64, S <= 2^26)");
    (void)hipGetLastError();
    hipStream_t st = (hipStream_t)stream;
    return hip_status(pattern == 0 ? normfwd::launch_copy_dense(src, dst, B * C * S, st)
                                   : normfwd::launch_rms_copy_pattern(src, dst, B, C, S, st),
                      "normfwd_copy_reference launch");
}

size_t fc_gn_forward_workspace_size(int64_t N, int64_t K, int64_t C)
{
    (void)K;
    if (N <= 0 || C <= 0) return 0;
    return ((size_t)N * (size_t)C * sizeof(float) + 255) & ~(size_t)255;
}

normfwd_status fc_gn_forward(const float* x, const float* W, const float* b, const float* gamma, const float* beta,
                             float* y, int64_t N, int64_t K, int64_t C, int64_t num_groups, float eps,
                             float negative_slope, void* workspace, size_t workspace_bytes, float* mean_out,
                             float* rstd_out, void* stream)
{
    if (N == 0 && K >= 0 && C > 0 && num_groups > 0 && C % num_groups == 0) return ok();  // no rows: nothing to do
    if (!x && K > 0) return fail(NORMFWD_ERR_INVALID, "fc_gn_forward: x must not be NULL");
    if ((!W && K > 0) || !y) return fail(NORMFWD_ERR_INVALID, "fc_gn_forward: W and y must not be NULL");
    if (N <= 0 || K < 0 || C <= 0 || num_groups <= 0)
        return fail(NORMFWD_ERR_INVALID, "fc_gn_forward: N, C and num_groups must be > 0 and K >= 0");
    if (C % num_groups != 0)
        return fail(NORMFWD_ERR_INVALID, "fc_gn_forward: C (%lld) must be a multiple of num_groups (%lld)",
                    (long long)C, (long long)num_groups);
    const int64_t K1 = K > 0 ? K : 1;
    if (N > kMaxElems / C || C > kMaxElems / K1 || N > kMaxElems / K1 || N > (1 << 23) || C > (1 << 24))
        return fail(NORMFWD_ERR_UNSUPPORTED, "fc_gn_forward: shape too large");
    if (!(eps >= 0.0f)) return fail(NORMFWD_ERR_INVALID, "fc_gn_forward: eps must be >= 0");
    if (!mean_out != !rstd_out)
        return fail(NORMFWD_ERR_INVALID, "fc_gn_forward: give both mean_out and rstd_out, or neither");
    normfwd_status s = check_ws(workspace, workspace_bytes, fc_gn_forward_workspace_size(N, K, C), "fc_gn_forward");
    if (s != NORMFWD_OK) return s;
    (void)hipGetLastError();
    return hip_status(normfwd::launch_fc_gn(x, W, b, gamma, beta, y, N, K, C, num_groups, eps, negative_slope,
                                            workspace, mean_out, rstd_out, (hipStream_t)stream),
                      "fc_gn_forward launch");
}

}  // extern "C"
