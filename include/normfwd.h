/*
 * normfwd — forward passes of three normalization layers on AMD MI355X
 * (gfx950), as a C ABI over hand-written HIP kernels.
 *
 * Sources (three POPCORNBENCH agent transcripts; a "turn" is one agent
 * message on a page):
 *   LN page  "Kimi-K2.6 l1_p40": LayerNorm over normalized_shape (64,256,256)
 *   GN page  "Kimi-K2.6 l2_p62": fc -> GroupNorm(512) -> LeakyReLU -> x + x
 *   RMS page "Kimi-K2.6 l1_p36": RMSNorm along dim 1 of an NCHW tensor
 *
 * Conventions shared by every entry point:
 *   - Tensors are fp32, contiguous, row-major, in device memory (HBM).  The
 *     caller owns every buffer; the library never allocates or frees.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     All work is enqueued on it; calls return as soon as the work is
 *     enqueued.
 *   - Any alignment and any length are accepted.  128-bit vector paths are
 *     taken when pointers are 16-byte aligned and the contiguous extent is a
 *     multiple of 4; otherwise a scalar path computes the same result.
 *   - In place (y == x) is allowed: every element is read before the same
 *     lane writes it (LayerNorm in place runs the split schedule under
 *     variants 1 and 3).  Partial overlap of inputs and outputs is
 *     undefined.
 *   - Results are run-to-run bitwise deterministic: no floating-point
 *     atomics, every reduction has a fixed order.
 *   - Size limits (beyond them NORMFWD_ERR_UNSUPPORTED): at most 2^40
 *     elements per tensor; LayerNorm outer <= 2^22 and inner <= 2^31;
 *     GroupNorm C <= 2^30; RMSNorm C < 2^31 and S <= 2^26; fc N <= 2^23 and
 *     C <= 2^24.  Problems whose grid would exceed the 32-bit work-item
 *     count of one launch are enqueued as several launches of whole samples
 *     (rows), in order, on the same stream.
 *   - Empty work is a no-op that returns NORMFWD_OK without inspecting the
 *     pointers: ln with outer == 0, gn with N == 0, rms with B == 0 or
 *     S == 0, fc with N == 0 (fc with K == 0 computes h = b).
 *   - Only ln_forward_workspace_check synchronizes (it reads a result back).
 *   - Errors are returned, never thrown: arguments are validated before
 *     anything is enqueued, so a non-OK return from validation means nothing
 *     was launched.  normfwd_last_error() then describes the failure
 *     (thread-local, valid until the next call on the same thread).
 *   - Two environment variables, read once per process, exist for testing
 *     and change no result: NORMFWD_MAX_GRID_ITEMS (>= 4096) lowers the
 *     work-items per launch so that small problems also take the
 *     several-launch path; NORMFWD_LN_FORCE_RECOMPUTE = k (a power of two)
 *     makes every k-th workgroup of the single-read LayerNorm kernel
 *     (ln_forward variant 1, not in place) have its moments computed by the
 *     other workgroups, the path taken when a workgroup is not resident.
 */
#ifndef NORMFWD_H
#define NORMFWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int normfwd_status;
#define NORMFWD_OK 0
#define NORMFWD_ERR_INVALID 1     /* bad shape, null required pointer, bad enum value   */
#define NORMFWD_ERR_UNSUPPORTED 2 /* valid arguments the library does not handle       */
#define NORMFWD_ERR_WORKSPACE 3   /* workspace null or smaller than the size query says */
#define NORMFWD_ERR_HIP 4         /* a HIP runtime call or kernel launch failed         */
#define NORMFWD_ERR_INCOMPLETE 5  /* a single-kernel LayerNorm gave up waiting (below)  */

/* Static string naming a status code ("unknown status" for other values). */
const char* normfwd_status_string(normfwd_status status);

/* Message describing the last non-OK return on this thread ("" if none). */
const char* normfwd_last_error(void);

/* Measurement hook.  Arms two hipEvent_t handles (created by the caller with
 * timing enabled; either may be NULL) for the next kernel this library
 * launches from the calling thread: that launch records its own start and
 * end time into them (hipExtLaunchKernel), so hipEventElapsedTime gives the
 * kernel's duration with no marker packets between kernels.  For an entry
 * point that launches several kernels, the first one is timed (ln_forward
 * variant 0: the moments kernel; use ln_forward_apply to time the normalize
 * kernel).  The cooperative launch of ln_forward variant 2 in place cannot
 * carry events; there they are recorded as markers just before and after it.  The
 * events stay armed until a launch takes them or this is called again
 * (NULL, NULL disarms).  Always NORMFWD_OK. */
normfwd_status normfwd_time_next_kernel(void* start_event, void* stop_event);

/* ------------------------------------------------------------------------
 * LayerNorm (LN page, turn 1: per sample, mean and population variance over
 * all elements of normalized_shape; y = (x - mean) / sqrt(var + eps) * weight
 * + bias, weight and bias elementwise of normalized_shape.  Turn 2 splits
 * each sample over many workgroups that write partial moments, reduces them
 * per sample, then normalizes.  Turn 6 lets the last workgroup to finish a
 * sample do that reduction, which the single-kernel variant does.)
 *
 *   x, y      [outer, inner] fp32; inner = prod(normalized_shape)
 *   weight    [inner] fp32 or NULL (= all ones)
 *   bias      [inner] fp32 or NULL (= all zeros)
 *   eps       added to the variance inside the square root
 *   mean_out  [outer] fp32 or NULL: the sample mean, rounded to fp32
 *   rstd_out  [outer] fp32 or NULL: 1 / sqrt(var + eps), rounded to fp32
 *   workspace device buffer of at least ln_forward_workspace_size(outer,
 *             inner) bytes, 256-byte aligned, zeroed by
 *             ln_forward_workspace_init() before its first use with a given
 *             (outer, inner); each call leaves it ready for the next call of
 *             the same (outer, inner).  Where its regions lie depends on the
 *             shape, so before a workspace serves another shape it must be
 *             zeroed again.  It holds per-workgroup partial moments,
 *             per-sample statistics and the arrival counters the kernels
 *             synchronize on.  One workspace must not be used by two calls
 *             that may run concurrently.
 *   variant   0 = split: a partial-moments kernel, a per-sample merge of
 *                 the partials, then a normalize kernel.  With fewer than
 *                 16384 moments workgroups the merge is done by the last
 *                 workgroup of each sample to finish (LN page, turn 6;
 *                 nothing waits, so any grid size works), otherwise by a
 *                 merge kernel;
 *             1 = single kernel: one launch of at most one workgroup per
 *                 CU in which every workgroup keeps its share of each
 *                 sample in registers between the moments pass and the
 *                 normalize pass (x is read from HBM once).  When a sample
 *                 spreads over fewer workgroups than fit on the GPU, the
 *                 grid holds several groups of workgroups, each taking every
 *                 groups-th sample.  A control wave
 *                 per workgroup exchanges the workgroups' moments of each
 *                 sample through generation-tagged words (no atomics) while
 *                 the data waves stream the next samples.  It is an
 *                 ordinary launch: if a workgroup is not resident (another
 *                 kernel holds its CU), the others wait for its moments
 *                 for at most 256 polls (~0.3-0.5 ms, which absorbs a
 *                 kernel running alongside on another stream), then compute
 *                 them from x themselves, bit for bit the same, and publish
 *                 them for the other readers; later waits of that launch
 *                 last at most 32 polls.  The result never depends on
 *                 residency (GPU tests check it bitwise, with workgroups
 *                 forced silent and beside other kernels on other
 *                 streams).  Since readers need x intact until the end, in
 *                 place (y == x) this variant runs the split schedule;
 *             2 = single kernel in which the last workgroup to arrive at
 *                 a sample, by an atomic count, merges every workgroup's
 *                 partial of it and announces the statistics (LN page,
 *                 turn 6: last-block-done), the others waiting for them (a
 *                 control wave per workgroup does the exchange beside the
 *                 data waves of variant 1, which read x once; partials
 *                 carry the launch's generation tag, so arrivals are
 *                 counted iterations ahead and the merger polls until
 *                 every partial is current).  Not in place it is an
 *                 ordinary launch: if a workgroup is not resident (so it
 *                 never arrives and no merger is elected), a workgroup that
 *                 has waited for a sample's statistics for the same bounded
 *                 number of polls as in variant 1 merges the sample itself,
 *                 computing the missing moments from x, with the same bits
 *                 whoever merges.  In place (y == x) it is a cooperative
 *                 launch, every workgroup resident, since x may be
 *                 overwritten by then.  The runtime grants cooperative
 *                 launches on a GPU to one process at a time: after
 *                 another, still running process has made one, an in-place
 *                 call of this variant returns NORMFWD_ERR_UNSUPPORTED and
 *                 launches nothing.
 *             3 = automatic: variant 1 wherever it can run (it measured
 *                 faster than the split, or within 1 us of it on calls of
 *                 ~10 us, at every shape tried), otherwise variant 0 (also
 *                 in place).  The choice depends only on the shape, the
 *                 pointers (alignment, y == x) and the device, so it is the
 *                 same on every call with the same tensors.
 *             Shapes a single kernel cannot hold (inner % 4 != 0, unaligned
 *             pointers, more rows than co-resident workgroups can keep) run
 *             the split schedule instead.
 *
 * Statistics are exact to about 1e-7 relative even when |mean| >> std and
 * whatever the values of particular elements: every sum of squares is taken
 * around a shift that lies inside the data it sums (a wave's own mean in
 * the single-kernel variants, a thread's own first value in the split's
 * moments pass), partial moments travel in fp64 and are merged in a fixed
 * order (Chan's pairwise update), and the mean is applied as an fp32 hi +
 * lo pair.
 * ---------------------------------------------------------------------- */
size_t ln_forward_workspace_size(int64_t outer, int64_t inner);

/* Zero `workspace` (enqueued on `stream`, as a kernel: safe inside a
 * captured HIP graph).  Required before a workspace's first use with each
 * (outer, inner). */
normfwd_status ln_forward_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* Health check of the last-workgroup-merges kernel (ln_forward variant 2).
 * Its workgroups wait for one another; each wait gives up after a bounded
 * number of polls (a fraction of a second), which can only happen if the
 * workgroups of its cooperative launch (in place) were not all resident,
 * and then records the failure in the workspace instead of hanging.
 * (Variant 1, and variant 2 not in place, never record one: moments that
 * do not arrive are computed by the waiting workgroups.)  This call waits
 * for the work queued on `stream` (it synchronizes, unlike every other entry
 * point, so it cannot be captured in a graph), reads that record and clears
 * it.  Returns NORMFWD_OK if no launch that used `workspace` since the last
 * check (or since ln_forward_workspace_init) gave up, NORMFWD_ERR_INCOMPLETE
 * if one did (its y and statistics are not valid), NORMFWD_ERR_WORKSPACE for
 * a null, misaligned or short buffer, NORMFWD_ERR_HIP if the copy fails. */
normfwd_status ln_forward_workspace_check(void* workspace, size_t workspace_bytes, void* stream);

normfwd_status ln_forward(const float* x, const float* weight, const float* bias, float* y,
                          int64_t outer, int64_t inner, float eps,
                          void* workspace, size_t workspace_bytes,
                          float* mean_out, float* rstd_out, int variant, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): ln_forward
 * without a workspace argument.  The workspace is a static array inside the
 * library, one per GPU, of 8 MiB (NORMFWD_LN_NOALLOC_SCRATCH_BYTES), which
 * each GPU the library runs on holds until the process ends.  The call
 * allocates and frees nothing and otherwise behaves exactly as ln_forward
 * (same kernels, same results, bit for bit) with the same arguments.
 *   - Shapes whose workspace (ln_forward_workspace_size(outer, inner)) is
 *     larger than the scratch return NORMFWD_ERR_UNSUPPORTED before anything
 *     is enqueued; samples of up to 8192 elements need no workspace at all.
 *   - Every call on one GPU shares that GPU's scratch, which keeps the last
 *     call's contents.  When a call's (outer, inner) differs from the last
 *     call's on that GPU, the call first clears the part it uses, with a
 *     kernel enqueued on `stream` ahead of its own work.
 *   - Calls that may run concurrently on one GPU (different streams without
 *     ordering between them, or different host threads) race on the scratch
 *     and give wrong results: order them.
 *   - The first call on each GPU looks up the scratch's device address
 *     (hipGetSymbolAddress) with that GPU current; a failure there returns
 *     NORMFWD_ERR_HIP. */
#define NORMFWD_LN_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
normfwd_status ln_forward_noalloc(const float* x, const float* weight, const float* bias, float* y,
                                  int64_t outer, int64_t inner, float eps,
                                  float* mean_out, float* rstd_out, int variant, void* stream);

/* The split variant's two halves, for callers that want the statistics
 * alone or want to time the phases: ln_forward_stats runs the moments
 * kernel and the merge and leaves per-sample (mean hi, mean lo, rstd) in
 * the workspace;
 * ln_forward_apply runs the normalize kernel from them.  Calling stats then
 * apply on one stream equals ln_forward(..., variant 0, ...). */
normfwd_status ln_forward_stats(const float* x, int64_t outer, int64_t inner, float eps,
                                void* workspace, size_t workspace_bytes,
                                float* mean_out, float* rstd_out, void* stream);
normfwd_status ln_forward_apply(const float* x, const float* weight, const float* bias, float* y,
                                int64_t outer, int64_t inner,
                                const void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * GroupNorm -> LeakyReLU -> x + x (GN page, turn 1: the [N, C] fc output is
 * split into num_groups groups of M = C / num_groups contiguous channels;
 * each (row, group) is normalized with its own mean and population variance
 * (eps inside the square root), then scaled by gamma[c] and shifted by
 * beta[c]; then LeakyReLU with negative_slope; then the result is added to
 * itself.)
 *
 *   x, y          [N, C] fp32
 *   gamma, beta   [C] fp32, or NULL (= ones / zeros)
 *   mean_out, rstd_out
 *                 [N, num_groups] fp32, both or neither (one alone is
 *                 NORMFWD_ERR_INVALID): each (row, group)'s mean and
 *                 1 / sqrt(var + eps), rounded to fp32, the statistics the
 *                 framework layer keeps for its backward pass (GN page,
 *                 turn 1)
 *   C % num_groups != 0 -> NORMFWD_ERR_INVALID (the GN page checks the same)
 * Statistics are taken around each group's first element, so groups far
 * from 0 (e.g. after a large fc bias) keep their accuracy.
 * ---------------------------------------------------------------------- */
normfwd_status gn_lrelu_x2_forward(const float* x, const float* gamma, const float* beta, float* y,
                                   int64_t N, int64_t C, int64_t num_groups, float eps,
                                   float negative_slope, float* mean_out, float* rstd_out, void* stream);

/* ------------------------------------------------------------------------
 * RMSNorm along dim 1 (RMS page, turns 1-2: rms = sqrt(mean over the
 * feature dim of x^2 + eps), y = x / rms, no affine).  The tensor is viewed
 * as [B, C, S] with S the product of the trailing dims, so one position's C
 * values sit S elements apart.
 *
 *   x, y   [B, C, S] fp32 (B * C * S may exceed 2^31)
 * ---------------------------------------------------------------------- */
normfwd_status rmsnorm_ch_forward(const float* x, float* y, int64_t B, int64_t C, int64_t S,
                                  float eps, void* stream);

/* The same on strided views (the RMS page, turn 2, weighs the tensor's
 * layout and its wrapper's contiguity handling; a channel slice or a
 * batch-strided view is normalized here without a copy).  Element (b, c, s)
 * of x is at x[b * x_batch_stride + c * x_channel_stride + s], of y at
 * y[b * y_batch_stride + c * y_channel_stride + s]: the S positions of one
 * (b, c) stay contiguous, strides are in elements and >= 0.  y's rows must
 * not overlap one another (NORMFWD_ERR_INVALID otherwise); x may be any
 * view, and y may be x itself with the same strides.
 *   rstd_out  [B, S] fp32 or NULL: 1 / sqrt(mean over C of x^2 + eps) per
 *             position, contiguous
 * The 128-bit path needs 16-byte aligned pointers, S and every stride a
 * multiple of 4; otherwise a scalar path computes the same result.
 * rmsnorm_ch_forward(x, y, B, C, S, ...) equals this call with strides
 * (C * S, S, C * S, S) and no rstd_out. */
normfwd_status rmsnorm_ch_forward_strided(const float* x, float* y, int64_t B, int64_t C, int64_t S,
                                          int64_t x_batch_stride, int64_t x_channel_stride,
                                          int64_t y_batch_stride, int64_t y_channel_stride,
                                          float eps, float* rstd_out, void* stream);

/* ------------------------------------------------------------------------
 * fc followed by GroupNorm -> LeakyReLU -> x + x (GN page, turn 1: h = x W^T
 * + b with x [N, K], W [C, K], b [C]; then the GN epilogue above on h).
 *
 *   workspace  device buffer of at least fc_gn_forward_workspace_size(N, K,
 *              C) bytes (holds h, [N, C] fp32, for group sizes the GEMM's
 *              epilogue does not handle itself), 256-byte aligned
 *   b, gamma, beta may be NULL.
 *   mean_out, rstd_out  as for gn_lrelu_x2_forward: the statistics of h's
 *              (row, group)s, [N, num_groups] fp32, both or neither.
 * ---------------------------------------------------------------------- */
size_t fc_gn_forward_workspace_size(int64_t N, int64_t K, int64_t C);
normfwd_status fc_gn_forward(const float* x, const float* W, const float* b,
                             const float* gamma, const float* beta, float* y,
                             int64_t N, int64_t K, int64_t C, int64_t num_groups, float eps,
                             float negative_slope, void* workspace, size_t workspace_bytes,
                             float* mean_out, float* rstd_out, void* stream);

/* ------------------------------------------------------------------------
 * Measurement references (not normalization operations): plain copies with
 * the access patterns of the kernels above, so that each kernel's HBM rate
 * can be set beside what a copy of the same bytes reaches on the same
 * device in the same run.
 *
 *   pattern 0   dense streaming copy of B * C * S floats (one 128-bit load
 *               and nontemporal store per thread, consecutive workgroups on
 *               consecutive addresses)
 *   pattern 1   rmsnorm_ch_forward's access pattern on [B, C, S] (the same
 *               grid, workgroup order, loads and stores), dst = src
 *   src, dst    device buffers of B * C * S floats, 16-byte aligned, not
 *               overlapping
 * Other shapes than those the patterns cover (a multiple of 4 floats;
 * pattern 1: S % 4 == 0, C <= 64, S <= 2^26) return NORMFWD_ERR_UNSUPPORTED.
 * ---------------------------------------------------------------------- */
normfwd_status normfwd_copy_reference(const float* src, float* dst, int64_t B, int64_t C, int64_t S,
                                      int pattern, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NORMFWD_H */
