// LayerNorm over the trailing `inner` elements of each of `outer` samples
// (LN page "Kimi-K2.6 l1_p40", turn 1: population mean and variance per
// sample, y = (x - mean) / sqrt(var + eps) * weight + bias with elementwise
// weight and bias).
//
// One sample is 4,194,304 floats (16 MiB) in the LN page's problem, far
// more than one workgroup should reduce, so each sample is spread over P
// workgroups (LN page, turn 2: many blocks per sample write partial moments
// to a workspace, a small step reduces them per sample, a third pass
// normalizes).
//
// Numerics (the page's own one-pass E[x^2] - mean^2 loses everything when
// |mean| >> std, e.g. N(100, 0.01) data, and a sum of squares around a shift
// that is not typical of the data loses as much; LN page, turn 2 asks for
// per-thread moments merged pairwise for this reason):
//   * every sum of squares is taken around a shift that lies inside the data
//     it sums: in the single-read kernels each wave first takes its mean in
//     fp32 (a wave sum of its registers) and then sums d = x - mean_w and d^2
//     (a true two-pass over registers); in the split moments pass every
//     float4 component of a thread shifts by the first value it reads (a
//     member of the very set it sums); the one-workgroup-per-sample kernel
//     takes two passes and corrects the mean with the second pass's sum;
//   * lane sums are widened to fp64 and reduced in a fixed order; moments
//     (n, mean, M2) travel in fp64;
//   * moments of different parts are merged with the pairwise (Chan) update,
//     in its k-way form around one part's mean, in a fixed order (LN page,
//     turn 2 derives the same merge for Welford partials);
//   * the mean is handed to the normalize pass as an fp32 pair hi + lo, so
//     (x - hi) - lo keeps ~48 bits of the mean.
// No statistic depends on which element a kernel reads first: tests plant
// outliers at the first element of the sample, of workgroups' and of waves'
// shares.
//
// Schedules of the same arithmetic:
//   split (variant 0): ln_partial_kernel (-> ln_merge_kernel from 1024
//          moments workgroups on; below that the last workgroup of each
//          sample merges it) -> ln_normalize_rows_kernel (or
//          ln_normalize_kernel for short samples); x is read twice.
//   single kernels (variants 1 and 2): one launch of at most one workgroup
//          per CU; workgroup p keeps its rows of every sample (variant 1: of
//          every sample of its group, when the grid holds several groups of
//          workgroups that take every G-th sample) in VGPRs from the moments
//          pass to the normalize pass, so x is read once, and the
//          workgroups exchange each sample's moments in the middle:
//          ln_single_ctl_kernel (variant 1, an ordinary launch): a control
//          wave per workgroup publishes generation-tagged moments and
//          gathers everyone's, while the data waves stream the next samples;
//          moments that do not arrive within a bounded wait (their workgroup
//          is not resident) are computed by the reader from x, with the same
//          bits (so it never runs in place: y == x takes the split);
//          variant 2: the last workgroup to arrive at a sample (an atomic
//          count, issued LAG - 1 iterations ahead) merges every workgroup's
//          generation-tagged partial of it and announces the statistics as
//          tagged words (LN page, turn 6: last-block-done; the tags serve as
//          the flags), done by the control wave of ln_single_ctl_kernel
//          (ctl_wave_last_block) beside the same data waves; an ordinary
//          launch in which a sample nobody announces (a workgroup that is
//          not resident never arrives) is merged by whoever waited for it,
//          from x where moments are missing; in place a cooperative launch.
//          Samples too large for the kernel's co-resident grid take the
//          split under every variant.
//   automatic (variant 3): ln_auto_variant picks variant 1 or the split by
//          shape, from measurements (the split in place).
//   short samples (inner <= 8192): ln_row_kernel, one workgroup per sample.
// Cross-workgroup data is only ever accessed with device-coherent atomic
// loads and stores (see the protocol notes below), never with fences.
#include "common.hpp"
#include "internal.hpp"
#include "ln_tag.hpp"

#include <algorithm>
#include <cstddef>
#include <type_traits>
#include <mutex>

namespace normfwd {

struct alignas(32) Partial {
    double n, mean, m2, pad;
};

struct LnCtrl {
    uint32_t gen;    // last-workgroup-merges kernel: launches so far (its statistics words carry the next value's tag)
    uint32_t done;   // completion counter of the current single-kernel launch (returns to 0)
    uint32_t error;  // set to 1 if a wait ran past its spin limit (last-workgroup-merges kernel)
    uint32_t recomputed;  // control-wave kernel: workgroup moments computed by a reader instead (diagnostic)
    uint32_t gen_ctl;     // control-wave kernel: launches so far mod 255 (its exchange tags derive from the next value)
    uint32_t pad[59];
};
static_assert(sizeof(LnCtrl) == 256, "control block is 256 bytes");
static_assert(offsetof(LnCtrl, error) == kLnErrorWordOffset, "error word where the API reads it");
static_assert(offsetof(LnCtrl, recomputed) == kLnRecomputedWordOffset, "recompute count where the tests read it");
static_assert(offsetof(LnCtrl, gen_ctl) == kLnCtlGenWordOffset, "control-wave generation where the tests read it");

constexpr int kLnThreads = 256;
// The single kernel's arrival counters: a ring of kRing, each on its own
// 128-byte line (atomics that meet on one line serialize).
constexpr int kCounterStride = 32;  // uint32 words
constexpr int kRing = 8;
// Polls before a wait gives up (sets the control block's error word and
// goes on): ~0.3-0.5 s, thousands of times the longest wait of a healthy
// launch, so a launch whose workgroups are not all resident ends instead of
// hanging.
constexpr uint32_t kSpinLimit = 1u << 18;
// The control-wave kernel needs no co-residency for its result: a reader
// that has polled this often for a workgroup's moments (~0.3-0.5 ms, tens of
// samples' streaming time, far beyond the skew of a healthy launch) computes
// them from x itself; once one wait has run out, later waits give up after
// kSpinLimitAfterMiss polls, since the missing workgroup is most likely
// still not resident.
constexpr uint32_t kCtlSpinLimit = 1u << 8;
constexpr uint32_t kSpinLimitAfterMiss = 1u << 5;

// Split schedule tuning: elements per partial-moment workgroup, rows in
// flight per thread in the moments pass, XCD-aware row order in the
// normalize pass.
#ifndef NORMFWD_LN_SPLIT_CHUNK
#define NORMFWD_LN_SPLIT_CHUNK 16384
#endif
#ifndef NORMFWD_LN_PARTIAL_UNROLL
#define NORMFWD_LN_PARTIAL_UNROLL 4
#endif
#ifndef NORMFWD_LN_PARTIAL_NT
#define NORMFWD_LN_PARTIAL_NT 0
#endif
#ifndef NORMFWD_LN_NORM_ROWS
#define NORMFWD_LN_NORM_ROWS 1
#endif
#ifndef NORMFWD_LN_NORM_NT_STORE
#define NORMFWD_LN_NORM_NT_STORE 1
#endif
// Normalize pass: 1 = sample loop (ln_normalize_rows_kernel), 0 = one row
// per workgroup in XCD order (ln_normalize_kernel); samples in flight per
// thread in the sample loop.
#ifndef NORMFWD_LN_NORM_MODE
#define NORMFWD_LN_NORM_MODE 1
#endif
#ifndef NORMFWD_LN_NORM_SAMPLE_UNROLL
#define NORMFWD_LN_NORM_SAMPLE_UNROLL 2
#endif
#ifndef NORMFWD_LN_XCD_CONTIG
#define NORMFWD_LN_XCD_CONTIG 0
#endif
#ifndef NORMFWD_LN_XCD_MAP
#define NORMFWD_LN_XCD_MAP 1
#endif
// Split schedule: below NORMFWD_LN_FUSE_BELOW moments workgroups in all,
// the last workgroup of a sample to finish merges its partials (no separate
// merge launch); from there on ln_merge_kernel does (0 = always the kernel).
// Measured on MI355X, step per call, fused against the merge kernel: 64-512
// workgroups ([16, 65536], [8, 2^20]) 0.6-1.2 us faster; [16, 2^22] (4096)
// 135.3-136.3 against 137.0-137.8 us, [32, 2^22] (8192) 270.0-270.4 against
// 274.4-277.0, [128, 2^20] (8192) 267.2-268.0 against 265.3-269.3, [8, 2^22],
// [4, 2^22], [16, 2^20], [64, 2^18] within 0.3 us; [64, 2^22] (16384)
// 593.2-595.0 against 575.5-577.3.  (With the compiler's atomic optimizer
// on, which waited for each counter atomic where it was issued, fusing had
// cost 0.6-1.5 us at 1024-4096 workgroups.)
// Single-read kernel tiles: DW data waves (plus the control wave) of F4PT
// float4 per thread, i.e. a workgroup holds F4PT rows of 64 DW float4 of
// every sample.  Measured on MI355X at [16, 4M] (kernel duration, one call,
// three alternations, on two boxes): 11 x 6 96.3-97.0 us, 10 x 7 97.1-97.7,
// 8 x 8 99.1-100.4, 9 x 8 99.2-99.7, 12 x 6 100.7-101.1, 13/14/15 x 5
// 99.7-100.5, 7 x 10 99.2-100.2 (DW x F4PT; tiles whose rows of weight and
// bias overflow LDS or whose grid exceeds 256 workgroups were not run).
// The wide tile (11 x 6) streams a sample faster but costs more to start
// and with sample groups: against 8 x 8 (kernel us, one call) [32, 4M]
// 181.5 vs 188.3, [16, 4M] 97.0 vs 99.4, [12, 4M] 75.0 vs 76.3, [8, 4M]
// 53.7 vs 54.6, [4, 4M] 30.4 vs 30.4, [2, 4M] 22.0 vs 20.4, [1, 4M] 15.2 vs
// 14.2, [16, 3M] 77.3 vs 76.3, [32, 3M] 147.0 vs 146.5, [16, 2M] 52.8 vs
// 50.0, [32, 1M] 52.6 vs 49.4, [8, 1M] 21.4 vs 17.1, [256, 16K] 12.1 vs
// 11.6.  With the store/refill interleave (both tiles; kernel us, median of
// 40 launches, one shared output buffer): [1, 4M] 14.8 vs 14.4, [2, 4M] 19.2
// vs 18.2, [3, 4M] 22.1 vs 22.0, [4, 4M] 26.8 vs 27.5, [5, 4M] 31.0 vs 34.3,
// [6, 4M] 37.3 vs 39.5, [7, 4M] 42.9 vs 45.9, [4, 4000000] 25.4 vs 28.7,
// [6, 3900000] 35.3 vs 39.7, [16, 3.5M] 83.2 vs 83.6, [16, 3M] 74.1 vs 74.9,
// [8, 3M] 38.7 vs 39.6, [32, 3M] 144.3 vs 142.7, [16, 2.5M] 68.4 vs 67.2.
// So the wide tile runs where a sample fills at least 90% of the
// co-resident grid (one group) and there are at least 4 samples, and where
// the 8 x 8 tile cannot hold a sample.  The choice depends on the shape and
// the device only, as the tagged exchange needs (a workspace of one shape
// always sees the same tile).
// LAG: iterations between a sample's moments and its normalize (register
// tiles LAG + 2).  The wide tile has room for a lag of 3 (152 VGPRs, no
// spills) or 4 (166): kernel us for lags 2 / 3 / 4, one call: [64, 4M]
// 352.7 / 352.1 / 364.0, [32, 4M] 183.5 / 182.9 / 185.4, [16, 4M] 96.9 /
// 96.2 / 96.3, [8, 4M] 53.6 / 50.1 / 49.4 (last-workgroup merges at [16,
// 4M]: 167-168 / 164-165 us per call).  The 8 x 8 tile spills with 3.
// (Those figures predate the store/refill interleave.  With it, at [16, 4M]:
// 11 x 6 with lags 2 / 3 / 4 95.1 / 93.2 / 93.3 us, 10 x 7 with lags 2 / 3
// 95.7 / 94.3, 13 x 5 with a lag of 3 93.5, 8 x 8 with a lag of 2 94.8;
// 12 x 6, 8 x 8 with a lag of 3 and 13 x 5 with 4 spill.)
constexpr int kLnTileWaves = 8;
constexpr int kLnTileF4 = 8;
constexpr int kLnTileLag = 2;
constexpr int kLnWideWaves = 11;
constexpr int kLnWideF4 = 6;
constexpr int kLnWideLag = 3;


// Doubles per workgroup in the control-wave kernel's exchange region (0:
// all means of a sample, then all M2s).  Measured on MI355X at [16, 4M]
// (kernel duration, one call, three alternations): 4 (32 bytes, the mean
// and M2 words then padding) 99.1-99.5 us, 8 99.2-99.6, 16 101.4-101.8, 0
// 101.6-102.2: packing many workgroups' words into one line (fewer poll
// requests) or giving each its own 128-byte line is slower.
#ifndef NORMFWD_LN_XCHG_SLOT
#define NORMFWD_LN_XCHG_SLOT 4
#endif

#ifndef NORMFWD_LN_FUSE_BELOW
#define NORMFWD_LN_FUSE_BELOW 16384
#endif


// uint32 words of the single kernel's arrival-counter ring (kRing slots x
// 128 bytes).
constexpr size_t kLnCounterWords = (size_t)kRing * 32;

static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

LnLayout ln_layout(int64_t outer, int64_t inner)
{
    LnLayout L{};
    L.P = std::min<int64_t>(1024, std::max<int64_t>(1, ceil_div(inner, NORMFWD_LN_SPLIT_CHUNK)));
    L.P_cap = std::min<int64_t>(1024, std::max<int64_t>(1, ceil_div(inner, 1024)));
    size_t off = 0;
    L.off_ctrl = off;
    off += sizeof(LnCtrl);
    L.off_counter = off;
    off += align256(4 * (size_t)kLnCounterWords);
    L.off_split_counter = off;
    off += align256(4 * (size_t)kCounterStride * (size_t)outer);
    L.off_stats = off;
    off += align256(16 * (size_t)outer);
    L.off_part = off;
    off += align256(sizeof(Partial) * (size_t)outer * (size_t)L.P_cap);
    L.off_xchg = off;
    off += align256((NORMFWD_LN_XCHG_SLOT ? NORMFWD_LN_XCHG_SLOT : 2) * sizeof(double) * (size_t)outer * (size_t)L.P_cap);
    L.off_lbd = off;
    off += align256(2 * sizeof(double) * (size_t)outer);
    L.off_lbdx = off;
    off += align256(2 * sizeof(double) * (size_t)outer * (size_t)L.P_cap);
    L.total = off;
    return L;
}

// ---------------------------------------------------------------- device pieces

// Sum of one double per thread over the workgroup, fixed order; valid in
// every thread on return.  red: LDS of NT/64 + 1 doubles.
__device__ __forceinline__ double block_sum(double v, double* red)
{
    v = wave_sum(v);
    const int wave = threadIdx.x / kWave;
    __syncthreads();  // red may still be read from a previous use
    if ((threadIdx.x & (kWave - 1)) == 0) red[wave] = v;
    __syncthreads();
    double t = red[0];
    for (int w = 1; w < kLnThreads / kWave; ++w) t += red[w];
    return t;
}

// Cross-workgroup protocol.  The 8 XCDs have their own L2s, which are not
// coherent with each other for ordinary accesses; agent-scope release and
// acquire fences make them coherent by writing back / invalidating the
// whole L2 (buffer_wbl2 / buffer_inv), which measured ~100 us over one
// LayerNorm launch.  The protocol below avoids them: every location that
// crosses workgroups (partial moments, statistics, counters, exchange
// words) is only ever accessed with agent-scope atomic loads and stores,
// which the gfx950 code generator issues as device-coherent accesses (sc1)
// served at the device's coherence point.  In the split schedule's fused
// tail a writer waits for its partial's stores to complete (s_waitcnt
// vmcnt(0)) before it counts its arrival, so the workgroup that sees the
// last arrival reads every partial.  The single kernels exchange words that
// announce themselves instead (generation-tagged, see ln_tag.hpp), which
// need no flag and no such wait: an aligned 8-byte store is seen whole, and
// a reader takes a word only when it carries the current tag.
//
// Arrival counters of the single kernel live in a ring of kRing slots
// (sample t uses slot t % kRing), each on its own 128-byte line, and are
// never reset (see ctl_wave_last_block for why reuse is safe).

// Wait until this thread's earlier vector-memory accesses have completed.
__device__ __forceinline__ void vmem_drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <typename T>
__device__ __forceinline__ void dev_store(T* p, T v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T dev_load(const T* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Publish this workgroup's partial and count its arrival on `counter`
// (thread 0 only); true for the last of the P arrivals.
__device__ __forceinline__ bool deliver_partial(Partial* part, const Partial& v, uint32_t* counter, int64_t P)
{
    dev_store(&part->n, v.n);
    dev_store(&part->mean, v.mean);
    dev_store(&part->m2, v.m2);
    vmem_drain();
    return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(P - 1);
}

// (mean hi, mean lo, rstd) of a merged sample.
__device__ __forceinline__ f4 finish_stats(double n, double m, double m2, float eps)
{
    const double var = n > 0.0 ? m2 / n : 0.0;
    const double rstd = 1.0 / sqrt(var + (double)eps);
    const float hi = (float)m;
    const float lo = (float)(m - (double)hi);
    return f4{hi, lo, (float)rstd, 0.0f};
}

// ---------------------------------------------------------------- split variant

template <int VEC>
struct LnVec;
template <>
struct LnVec<4> {
    using T = f4;
};
template <>
struct LnVec<1> {
    using T = float;
};

// Measured on MI355X: HBM streams fastest when the loads in flight at any
// moment cover one dense address range (few KiB per workgroup, neighbouring
// workgroups on neighbouring addresses); a workgroup that walks its own
// 64 KiB run leaves the in-flight set scattered 64 KiB apart and loses ~20%.
// So a sample is cut into rows of 256 units (a unit is one float4, or one
// float on the scalar path), and the P workgroups of a sample take the rows
// round-robin: workgroup p owns rows p, p + P, p + 2P, ...  At any moment
// the P workgroups read P adjacent rows.  Any partition of the sample works
// for the moment merge; this one only changes which elements a partial holds.
__device__ __forceinline__ int64_t rows_owned_units(int64_t nu, int64_t p, int64_t P)
{
    const int64_t nrows = ceil_div(nu, (int64_t)kLnThreads);
    if (p >= nrows) return 0;
    const int64_t c = (nrows - 1 - p) / P + 1;
    const int64_t last = nrows - 1;
    const int64_t last_units = nu - last * kLnThreads;
    const bool owns_last = (last - p) % P == 0;
    return owns_last ? (c - 1) * kLnThreads + last_units : c * kLnThreads;
}

// A sample's P partials (n, mean, M2) merged by one wave in the k-way form
// of the pairwise update, around partial 0's mean c: N = sum n_j, A = sum
// n_j (mean_j - c), B = sum (M2_j + n_j (mean_j - c)^2) (lane l takes
// partials l, l + 64, ..., the loads of a block of 256 in flight together;
// wave_total: a fixed order), then mean = c + A / N and M2 = B - A^2 / N.
// One division in all (a pairwise merge takes two per step, on the critical
// path of the sample); uniform on return.  COHERENT: the partials were
// written by other workgroups of the running launch and are read with
// device-coherent loads.
template <bool COHERENT>
__device__ __forceinline__ void kway_merge(const Partial* pb, int64_t P, double& n, double& mean, double& m2)
{
    const int lane = threadIdx.x & (kWave - 1);
    auto ld = [](const double* q) { return COHERENT ? dev_load(q) : *q; };
    const double c = lane_f64(ld(&pb[0].mean), 0);
    double N = 0.0, A = 0.0, B = 0.0;
    for (int64_t j0 = 0; j0 < P; j0 += 4 * kWave) {
        double nj[4], mj[4], qj[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t j = j0 + lane + (int64_t)u * kWave;
            const Partial* pj = pb + (j < P ? j : 0);
            nj[u] = j < P ? ld(&pj->n) : 0.0;
            mj[u] = ld(&pj->mean);
            qj[u] = j < P ? ld(&pj->m2) : 0.0;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const double d = mj[u] - c;
            N += nj[u];
            A += nj[u] * d;
            B += qj[u] + nj[u] * (d * d);
        }
    }
    n = wave_total(N);
    A = wave_total(A);
    B = wave_total(B);
    const double md = n > 0.0 ? A / n : 0.0;
    mean = c + md;
    m2 = fmax(B - A * md, 0.0);
}

__device__ __forceinline__ void store_stats(int64_t b, const f4& st, f4* stats, float* mean_out, float* rstd_out)
{
    stats[b] = st;
    if (mean_out) mean_out[b] = st.x;
    if (rstd_out) rstd_out[b] = st.z;
}

// Moments of workgroup p's rows of sample b, stored as the sample's p-th
// partial (n, mean, M2).  With counters (one per sample, on its own
// 128-byte line, zero on entry) the partial is published with the
// device-coherent protocol above and counted; the workgroup that arrives
// last merges the sample's partials with one wave, writes its statistics
// and puts the counter back to zero for the next launch.  Nothing waits, so
// the launch needs no co-residency.  Without counters the merge is left to
// ln_merge_kernel.
template <int VEC>
__global__ void __launch_bounds__(kLnThreads)
ln_partial_kernel(const float* x, int64_t inner, int64_t P, int64_t P_cap, Partial* parts, uint32_t* counters,
                  float eps, f4* stats, float* mean_out, float* rstd_out)
{
    using V = typename LnVec<VEC>::T;
    constexpr int U = NORMFWD_LN_PARTIAL_UNROLL;
    __shared__ double red[kLnThreads / kWave];
    const int64_t blk = NORMFWD_LN_XCD_CONTIG ? xcd_contiguous(blockIdx.x, gridDim.x) : blockIdx.x;
    const int64_t b = blk / P;
    const int64_t p = blk - b * P;
    const float* xb = x + b * inner;
    const V* xv = reinterpret_cast<const V*>(xb);
    const int64_t nu = inner / VEC;
    const int64_t nrows = ceil_div(nu, (int64_t)kLnThreads);
    // Every float4 component of a thread sums d = x - K and d^2 around its own
    // shift K, the first value it reads: a member of the very set it sums,
    // so the cancellation in M2 = sum d^2 - (sum d)^2 / n costs at most a few
    // fp32 roundings of that set's own M2, whatever its offset from 0.
    // (Positions past the end load K: d = 0, and they are not counted.)
    const int64_t j_first = p * kLnThreads + threadIdx.x;
    const V K = j_first < nu ? xv[j_first] : V(0.0f);
    V a1 = V(0.0f), a2 = V(0.0f);
    int cnt = 0;
    for (int64_t r = p; r < nrows; r += P * U) {
        V v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = (r + (int64_t)u * P) * kLnThreads + threadIdx.x;
            cnt += j < nu;
            v[u] = j < nu ? (NORMFWD_LN_PARTIAL_NT ? ld_nt(xv + j) : xv[j]) : K;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const V d = v[u] - K;
            a1 += d;
            a2 += d * d;
        }
    }
    // Per component: n = cnt, mean_c = K_c + a1_c / n, M2_c = a2_c - a1_c^2 / n;
    // merged over the workgroup in a fixed order: mean = sum n mean_c / N,
    // M2 = sum (M2_c + n (mean_c - mean)^2) (the k-way pairwise update).
    f4 K4, a14, a24;
    if constexpr (VEC == 4) {
        K4 = K;
        a14 = a1;
        a24 = a2;
    } else {
        K4 = f4{K, 0.0f, 0.0f, 0.0f};
        a14 = f4{a1, 0.0f, 0.0f, 0.0f};
        a24 = f4{a2, 0.0f, 0.0f, 0.0f};
    }
    const double nl = (double)cnt;
    double mc[VEC], sum_nm = 0.0;
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
        mc[c] = cnt ? (double)K4[c] + (double)a14[c] / nl : 0.0;
        sum_nm += nl * mc[c];
    }
    const double n_wg = (double)(rows_owned_units(nu, p, P) * VEC);
    const double mean = n_wg > 0.0 ? block_sum(sum_nm, red) / n_wg : 0.0;
    double sum_m2 = 0.0;
    if (cnt) {
#pragma unroll
        for (int c = 0; c < VEC; ++c) {
            const double t1 = (double)a14[c], dm = mc[c] - mean;
            sum_m2 += fmax((double)a24[c] - t1 * (t1 / nl), 0.0) + nl * (dm * dm);
        }
    }
    Partial q{};
    q.n = n_wg;
    q.mean = mean;
    q.m2 = block_sum(sum_m2, red);
    Partial* pb = parts + b * P_cap;
    if (counters == nullptr) {
        if (threadIdx.x == 0) pb[p] = q;
        return;
    }
    __shared__ int last;
    uint32_t* counter = counters + b * kCounterStride;
    // The wave that publishes and counts (and, for the last arrival, merges)
    // at raised priority, ahead of the other workgroups' streaming waves on
    // its SIMD.  Step per call on MI355X: [16, 4M] 134.9-135.3 against
    // 136.5-136.8 us, [32, 4M] 272.2-275.1 against 274.4-274.9, [8, 4M]
    // 73.7-74.2 against 73.3-73.6, [16, 1M] and [64, 256K] within 0.3 us.
    if (threadIdx.x < kWave) __builtin_amdgcn_s_setprio(2);
    if (threadIdx.x == 0) last = deliver_partial(&pb[p], q, counter, P);
    __syncthreads();
    if (!last || threadIdx.x >= kWave) return;
    double n, m, m2;
    kway_merge<true>(pb, P, n, m, m2);
    if (threadIdx.x == 0) {
        store_stats(b, finish_stats(n, m, m2, eps), stats, mean_out, rstd_out);
        dev_store(counter, 0u);
    }
}

// One wave per sample merges its partials (kway_merge); lane 0 writes
// (mean hi, mean lo, rstd).
__global__ void __launch_bounds__(kWave)
ln_merge_kernel(const Partial* parts, int64_t P, int64_t P_cap, float eps, f4* stats, float* mean_out,
                float* rstd_out)
{
    const int64_t b = blockIdx.x;
    double n, m, m2;
    kway_merge<false>(parts + b * P_cap, P, n, m, m2);
    if (threadIdx.x == 0) store_stats(b, finish_stats(n, m, m2, eps), stats, mean_out, rstd_out);
}

// One row of 256 units per workgroup.  With xcd_map the workgroups one XCD
// runs back to back (workgroups go to the 8 XCDs round-robin by index) take
// the same row of every sample in turn, so that XCD's L2 fetches the row of
// weight/bias once and serves it to all samples.
template <int VEC>
__global__ void __launch_bounds__(kLnThreads)
ln_normalize_kernel(const float* x, const float* w, const float* bias, float* y, int64_t outer, int64_t inner,
                    int64_t bps, int xcd_map, const f4* stats)
{
    using V = typename LnVec<VEC>::T;
    constexpr int R = NORMFWD_LN_NORM_ROWS;
    int64_t b, q;
    const int64_t i = blockIdx.x;
    if (xcd_map) {
        const int64_t xcd = i & 7, r = i >> 3;
        b = r % outer;
        q = (r / outer) * 8 + xcd;
    } else {
        b = i / bps;
        q = i - b * bps;
    }
    const int64_t nu = inner / VEC;
    const f4 st = stats[b];
    const V* xv = reinterpret_cast<const V*>(x + b * inner);
    V* yv = reinterpret_cast<V*>(y + b * inner);
    V xr[R], wr[R], br[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t j = (q * R + r) * kLnThreads + threadIdx.x;
        if (j < nu) {
            xr[r] = ld_nt(xv + j);
            wr[r] = w ? reinterpret_cast<const V*>(w)[j] : V(1.0f);
            br[r] = bias ? reinterpret_cast<const V*>(bias)[j] : V(0.0f);
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t j = (q * R + r) * kLnThreads + threadIdx.x;
        if (j < nu) {
            const V o = ((xr[r] - st.x) - st.y) * st.z * wr[r] + br[r];
            if (NORMFWD_LN_NORM_NT_STORE)
                st_nt(o, yv + j);
            else
                yv[j] = o;
        }
    }
}

// Sample-loop order: workgroup q owns row q of every sample; it loads its
// row of weight/bias once and streams the samples through it, so weight and
// bias cross HBM exactly once without relying on L2, and at any moment the
// workgroups in flight cover one dense run of rows per sample.  (Measured:
// 84 us inside the LN step against 92 us for the XCD-ordered one-row
// kernel; part of the second read of x is served by the 256 MB MALL, which
// is why the moments pass keeps ordinary, not streaming, loads.)
template <int VEC>
__global__ void __launch_bounds__(kLnThreads)
ln_normalize_rows_kernel(const float* x, const float* w, const float* bias, float* y, int64_t outer, int64_t inner,
                         const f4* stats)
{
    using V = typename LnVec<VEC>::T;
    constexpr int U = NORMFWD_LN_NORM_SAMPLE_UNROLL;
    const int64_t nu = inner / VEC;
    const int64_t blk = NORMFWD_LN_XCD_CONTIG ? xcd_contiguous(blockIdx.x, gridDim.x) : blockIdx.x;
    const int64_t j = blk * kLnThreads + threadIdx.x;
    if (j >= nu) return;
    const V wv = w ? reinterpret_cast<const V*>(w)[j] : V(1.0f);
    const V bv = bias ? reinterpret_cast<const V*>(bias)[j] : V(0.0f);
    for (int64_t t0 = 0; t0 < outer; t0 += U) {
        V xr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t b = t0 + u;
            if (b < outer) xr[u] = ld_nt(reinterpret_cast<const V*>(x + b * inner) + j);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t b = t0 + u;
            if (b < outer) {
                const f4 st = stats[b];
                const V o = ((xr[u] - st.x) - st.y) * st.z * wv + bv;
                V* dst = reinterpret_cast<V*>(y + b * inner) + j;
                if (NORMFWD_LN_NORM_NT_STORE)
                    st_nt(o, dst);
                else
                    *dst = o;
            }
        }
    }
}

// ---------------------------------------------------------------- one workgroup per sample

// Samples of at most 256 * UPT units (a unit is one float4, or one float
// on the scalar path): one workgroup holds the whole sample in VGPRs, takes
// the two passes over registers (mean of d = x - K with K the sample's first
// element, then the sum of (d - mean_d)^2) and writes y; x is read once and
// no workspace is involved.  This is the shape of LayerNorm used in
// transformer blocks (many samples of a few thousand elements).
template <int VEC, int UPT>
__global__ void __launch_bounds__(kLnThreads)
ln_row_kernel(const float* x, const float* w, const float* bias, float* y, int64_t inner, float eps,
              float* mean_out, float* rstd_out)
{
    using V = typename LnVec<VEC>::T;
    __shared__ double red[kLnThreads / kWave];
    const int64_t row = blockIdx.x;
    const float* xr = x + row * inner;
    const V* xv = reinterpret_cast<const V*>(xr);
    const int64_t nu = inner / VEC;
    const float K = xr[0];
    V v[UPT];
    V a = V(0.0f);
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
        const int64_t j = threadIdx.x + (int64_t)k * kLnThreads;
        v[k] = j < nu ? xv[j] : V(K);
        a += v[k] - K;
    }
    double t;
    if constexpr (VEC == 4)
        t = ((double)a.x + (double)a.y) + ((double)a.z + (double)a.w);
    else
        t = (double)a;
    const double n = (double)inner;
    const double mean_d = block_sum(t, red) / n;
    const float md = (float)mean_d;
    // second pass around K + md, which lies inside the data: the sums of
    // e = (x - K) - md and e^2 are accurate whatever the first pass's rounding
    // (its fp32 sums of d may be far from 0 when K is not typical of the
    // sample), and sum e / n corrects the mean: mean = K + md + sum e / n,
    // var = sum e^2 / n - (sum e / n)^2
    V q = V(0.0f), q1 = V(0.0f);
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
        const V e = (v[k] - K) - md;  // padding lanes hold K: e = -md, masked below
        const int64_t j = threadIdx.x + (int64_t)k * kLnThreads;
        if (j < nu) {
            q1 += e;
            q += e * e;
        }
    }
    double t1;
    if constexpr (VEC == 4) {
        t = ((double)q.x + (double)q.y) + ((double)q.z + (double)q.w);
        t1 = ((double)q1.x + (double)q1.y) + ((double)q1.z + (double)q1.w);
    } else {
        t = (double)q;
        t1 = (double)q1;
    }
    const double de = block_sum(t1, red) / n;
    const double var = fmax(block_sum(t, red) / n - de * de, 0.0);
    const double mean = ((double)K + (double)md) + de;
    const double rstd = 1.0 / sqrt(var + (double)eps);
    const float hi = (float)mean;
    const float lo = (float)(mean - (double)hi);
    const float rs = (float)rstd;
    if (threadIdx.x == 0) {
        if (mean_out) mean_out[row] = hi;
        if (rstd_out) rstd_out[row] = rs;
    }
    V* yv = reinterpret_cast<V*>(y + row * inner);
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
        const int64_t j = threadIdx.x + (int64_t)k * kLnThreads;
        if (j < nu) {
            const V tt = ((v[k] - hi) - lo) * rs;
            const V wv = w ? reinterpret_cast<const V*>(w)[j] : V(1.0f);
            const V bv = bias ? reinterpret_cast<const V*>(bias)[j] : V(0.0f);
            st_nt(tt * wv + bv, yv + j);
        }
    }
}

// ---------------------------------------------------------------- single-kernel variant

// One float4 of d = x - m into a thread's running sums of d and d^2.  Every
// place that must reproduce these sums bit for bit goes through here, so
// they round the same way (the square and the add contract to one fused
// multiply-add on gfx950).
__device__ __forceinline__ void shifted_acc(f4& a1, f4& a2, const f4 d)
{
    a1 += d;
    a2 += d * d;
}

// A wave's sums of its lanes' (a1, a2), widened to fp64, in a fixed order
// (wave_total); uniform on return.
__device__ __forceinline__ void wave_moments(const f4 a1, const f4 a2, double& t1, double& t2)
{
    t1 = wave_total(((double)a1.x + (double)a1.y) + ((double)a1.z + (double)a1.w));
    t2 = wave_total(((double)a2.x + (double)a2.y) + ((double)a2.z + (double)a2.w));
}

// Layout of ln_single_ctl_kernel: DW data waves of 64 threads, F4PT float4
// per thread; thread i of workgroup j holds float4s j*RW + i + k*P*RW (k <
// F4PT, RW = 64 DW) of each sample, where those are < nv.  Elements (fp32
// values) data wave w of workgroup j holds of one sample:
template <int F4PT, int DW>
__device__ __forceinline__ uint32_t ctl_wave_elems(uint32_t j, int w, uint32_t P, int64_t nv)
{
    constexpr int64_t RW = DW * kWave;
    uint32_t n = 0;
#pragma unroll 1
    for (int k = 0; k < F4PT; ++k) {
        const int64_t left = nv - ((int64_t)j * RW + (int64_t)w * kWave + (int64_t)k * P * RW);
        n += (uint32_t)(left <= 0 ? 0 : left >= kWave ? kWave : left);
    }
    return 4u * n;
}
// ... and workgroup j as a whole:
template <int F4PT, int DW>
__device__ __forceinline__ uint32_t ctl_wg_elems(uint32_t j, uint32_t P, int64_t nv)
{
    constexpr int64_t RW = DW * kWave;
    uint32_t n = 0;
#pragma unroll 1
    for (int k = 0; k < F4PT; ++k) {
        const int64_t left = nv - ((int64_t)j * RW + (int64_t)k * P * RW);
        n += (uint32_t)(left <= 0 ? 0 : left >= RW ? RW : left);
    }
    return 4u * n;
}

// Moments of one data wave's share of a sample, two passes over the
// registers that hold it:
//   1. m = the wave's mean in fp32 (a float4 sum per lane over its valid
//      elements, in element order, then wave_shift): only a shift, so its
//      rounding does not matter, but it sits inside the data, so
//   2. the sums of d = x - m and d^2 (shifted_acc per element in element
//      order, fp32 per lane, then wave_moments in fp64) lose nothing to
//      cancellation, whatever the data's offset from 0: the wave's M2 is
//      t2 - t1^2 / n with t1 ~ 0.
// The data waves and a reader that recomputes a missing workgroup's
// moments (ctl_recompute) run these same steps on the same elements, so they
// get the same bits.  (The two loops are written out at both places: a
// helper taking the register tile by reference measured 18 spilled VGPRs in
// the data waves' loop, the loops inline none.)
struct WaveMoments {
    double t1, t2;  // sums of d and d^2 over the wave's elements
    float m;        // the shift
};
// inv_n: 1 / (the wave's element count), or 0 for a wave with none
__device__ __forceinline__ float wave_shift(const f4 s, float inv_n)
{
    return wave_total((s.x + s.y) + (s.z + s.w)) * inv_n;
}
__device__ __forceinline__ float inv_count_f32(uint32_t n) { return n ? 1.0f / (float)n : 0.0f; }
__device__ __forceinline__ double inv_count_f64(uint32_t n) { return n ? 1.0 / (double)n : 0.0; }

// A workgroup's (mean, M2) from its waves' moments (rd[3w .. 3w+2] = t1,
// t2, m of wave w; cnt[w] its element count, inv[w] = inv_count_f64(cnt[w]),
// inv_n the same of their total), merged around c, wave 0's mean (wave 0
// always holds elements): lane w < DW forms mean_w = m_w + t1_w / n_w and
// M2_w = t2_w - t1_w^2 / n_w, then A = sum n_w (mean_w - c) and B = sum
// (M2_w + n_w (mean_w - c)^2) over the lanes (wave_total, a fixed order), and
// mean = c + A / n, M2 = B - A^2 / n (the k-way pairwise update; with c a
// wave mean of the same data the last subtraction loses nothing that
// matters).  A wave with no elements adds nothing.  Called by a whole wave;
// the result is uniform, and every call on the same moments gets the same
// bits.
template <int DW>
__device__ __forceinline__ void merge_wave_moments(const double* rd, const uint32_t* cnt, const double* inv,
                                                   double inv_n, double& mean, double& m2)
{
    const int lane = threadIdx.x & (kWave - 1);
    double mw = 0.0, m2w = 0.0, nw = 0.0;
    if (lane < DW) {
        const double t1 = rd[3 * lane], iw = inv[lane];
        nw = (double)cnt[lane];
        mw = rd[3 * lane + 2] + t1 * iw;
        m2w = fmax(rd[3 * lane + 1] - t1 * (t1 * iw), 0.0);
    }
    const double c = lane_f64(mw, 0);
    const double d = mw - c;
    const double A = wave_total(nw * d);
    const double B = wave_total(m2w + nw * (d * d));
    const double md = A * inv_n;
    mean = c + md;
    m2 = fmax(B - A * md, 0.0);
}

// The (mean, M2) workgroup j of ln_single_ctl_kernel publishes for one
// sample (xs: the sample's float4s), computed by one whole wave from x: for
// each data wave w of j, lane l loads what thread w * 64 + l of j holds and
// takes the same two passes (wave_two_pass), and the wave results are merged
// by merge_wave_moments in wave order, so the result has exactly the bits j itself
// publishes.  Used when j's moments do not arrive.  rc: LDS for 3 DW doubles
// and DW counts, private to the calling wave.
template <int F4PT, int DW>
__device__ void ctl_recompute(const f4* xs, uint32_t j, uint32_t P, int64_t nv, double* rc, uint32_t* rc_cnt,
                              double* rc_inv, double& mean, double& m2)
{
    constexpr uint32_t RW = DW * kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t stride = P * RW;
    // two data waves' elements per batch: twice the loads in flight per round
    // trip, at 2 F4PT float4 registers per lane (with an odd DW the last
    // batch holds one wave)
#pragma unroll 1
    for (int w0 = 0; w0 < DW; w0 += 2) {
        f4 v[2][F4PT];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t off0 = j * RW + (uint32_t)((w0 + h) * kWave + lane);
#pragma unroll
            for (int k = 0; k < F4PT; ++k) {
                const uint32_t idx = off0 + (uint32_t)k * stride;
                v[h][k] = (w0 + h < DW && (int64_t)idx < nv) ? ld_nt(xs + idx) : f4(0.0f);
            }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int w = w0 + h;
            if (w >= DW) break;
            const uint32_t off0 = j * RW + (uint32_t)(w * kWave + lane);
            auto ok = [&](int k) { return (int64_t)(off0 + (uint32_t)k * stride) < nv; };
            const uint32_t n = ctl_wave_elems<F4PT, DW>(j, w, P, nv);
            // the data waves' two passes (see WaveMoments)
            f4 s = f4(0.0f);
#pragma unroll
            for (int k = 0; k < F4PT; ++k) s += ok(k) ? v[h][k] : f4(0.0f);
            WaveMoments r;
            r.m = wave_shift(s, inv_count_f32(n));
            f4 a1 = f4(0.0f), a2 = f4(0.0f);
#pragma unroll
            for (int k = 0; k < F4PT; ++k) shifted_acc(a1, a2, ok(k) ? v[h][k] - r.m : f4(0.0f));
            wave_moments(a1, a2, r.t1, r.t2);
            if (lane == 0) {
                rc[3 * w] = r.t1;
                rc[3 * w + 1] = r.t2;
                rc[3 * w + 2] = (double)r.m;
                rc_cnt[w] = n;
                rc_inv[w] = inv_count_f64(n);
            }
        }
    }
    merge_wave_moments<DW>(rc, rc_cnt, rc_inv, inv_count_f64(ctl_wg_elems<F4PT, DW>(j, P, nv)), mean, m2);
}

// Single-read schedule with a control wave.  DW data waves hold the
// workgroup's rows as above (rows are DW * 64 float4 wide here); one more
// wave holds no data and runs the cross-workgroup exchange, so that the
// data waves never wait on another workgroup and their loads stay in
// flight (a wave's memory counter retires in issue order, so a wave that
// polled memory would also wait for its own prefetch).  One workgroup
// barrier per sample; sample s is normalized LAG iterations after its
// moments:
//   data waves, iteration t:  two-pass moments of their share of sample t
//       (wave_two_pass) -> LDS; barrier t; normalize and store sample t-LAG
//       with the statistics the control wave left in LDS, then load sample
//       t-LAG+NT into the freed registers (NT = LAG + 2 register tiles:
//       sample t+1 is in flight while t is reduced, and t+2 is issued at
//       the end of the iteration; samples t-1 .. t-LAG+1 wait for their
//       statistics).
//   control wave, after barrier t:  merge the data waves' moments of sample
//       t into this workgroup's (mean, M2) (merge_wave_moments) and publish them
//       as two generation-tagged words; then read all P workgroups' words
//       for sample t-LAG+1 until every tag is current, merge them in a fixed
//       order (every workgroup computes the same statistics; the k-way
//       pairwise update around one shift, workgroup 0's mean, in fp64) and
//       leave the statistics in LDS before barrier t+1.
// With LAG >= 2 every workgroup has had a whole iteration to publish the
// moments the control wave gathers, so the gather rarely waits and the data
// waves do not wait for the slowest workgroup each iteration.  No atomics,
// counters or flags.  (The last-workgroup-merges exchange beside the same
// data waves, ctl_wave_last_block below, puts the last arrival's merge and
// announcement and the readers' poll on every sample's path: 98-99 us per
// call at [16, 4M] against 92-93 us.)
//
// Control wave of ln_single_ctl_kernel with the last-workgroup-merges
// exchange (LN page, turn 6: last-block-done), for ln_forward variant 2.
// Not in place it is an ordinary launch (may_recompute): a wait that runs
// out (a workgroup that is not resident neither arrives nor publishes, so
// no merger is elected) is followed by the waiter merging the sample
// itself, computing missing moments from x with the same bits, so the
// result is the same bits whoever merges.  In place it is a cooperative
// launch (x may be overwritten by then; every workgroup is resident) and a
// wait that runs past its spin limit sets the control block's error word
// instead.  The data waves are those of the tagged exchange, unchanged, so
// they never wait on another workgroup.  Each workgroup counts its arrival
// at a sample on that sample's counter (a ring of kRing) AHEAD = LAG - 1
// iterations early, and the arrival that finds P - 1 (mod P) before it
// merges the sample.  After barrier t:
//   take the count returned for sample t (issued AHEAD iterations ago) and
//   issue this workgroup's arrival at sample t + AHEAD;
//   issue the loads of the statistics words of sample g = t - LAG + 1 (they
//   were announced an iteration or more ago, and their round trip overlaps
//   what follows);
//   merge the data waves' moments of sample t into this workgroup's (mean,
//   M2) (merge_wave_moments) and store them as two words tagged with the
//   launch generation in its slot of a region only this kernel and the
//   zeroing kernel write;
//   if elected for sample t, read every workgroup's words, polling any whose
//   tag is not yet current (each owner stores them in its iteration t, so
//   they land), merge them in a fixed order (the k-way pairwise update
//   around workgroup 0's mean, one wave), take P back off the counter and
//   announce the sample's mean and rstd as two tagged fp64 words
//   (ln_tag.hpp), so one poll both finds and reads them;
//   then poll sample g's words until both carry this launch's tag and leave
//   its statistics in LDS before barrier t + 1.
// The counter only elects the merger; the tags, not the order of arrival,
// tell it which words are this launch's, so nothing on its path waits for
// a store to complete or for an atomic's round trip.  Counters are never
// reset: a sample's P arrivals see every residue mod P once, whatever count
// the counter held before (even one a launch that gave up left behind).  A
// workgroup issues its arrival at sample s + kRing in iteration s + kRing -
// AHEAD, after reading the statistics of sample s (kRing >= LAG + AHEAD),
// which exist only once all of sample s's arrivals were counted; the merger's
// subtraction lands before its own arrival at sample s + kRing (same
// address, same wave), so each count stays below 2P.  (When a workgroup
// is not resident, a sample's statistics can come from a waiter before all
// its arrivals; elections may then fall on other arrivals, including a
// late one, but every merge, elected or not, announces the same bits, no
// subtraction comes before a count of P, and a sample nobody merges is
// merged by its waiters.)  Measured per call at
// [16, 4M]: 140-144 us with the partials stored, drained and then counted
// and the counter reset, stored and drained before the announcement (the
// last arrival then kept merging every sample, each of its iterations ~7.7
// us against ~5.8 us for the data, and the whole grid ran at its pace);
// 133.9 us with the tagged words and the count issued right after them;
// 125-126 us with the count issued an iteration early; 108-109 us as an
// ordinary launch (the cooperative one cost ~17 us per call); 105-107 us
// with LLVM's AMDGPU atomic optimizer off for this file (build.py), which
// otherwise turns the single-lane arrival into a wave-wide atomic whose
// result is broadcast, and so waited for, right where it is issued; 98-100
// us with the control wave at raised priority; 98-99 us with arrivals
// counted LAG - 1 (two) iterations ahead.
// Merging sample t one iteration later, when every workgroup's words have
// surely landed, measured 128.5 us; a lag of 4 samples (with a ring of 8)
// 125.6 (both with the cooperative launch), and 113 us against 107 as an
// ordinary launch; issuing the merger's loads of the words first, 110 us.
// Every workgroup derives mean hi/lo and rstd from the same two words.  The
// last workgroup out advances the generation.
template <int F4PT, int DW, int LAG>
__device__ void ctl_wave_last_block(const double (*red)[3 * DW], const uint32_t* cnt, const double* cnt_inv,
                                    const float* wg_cnt, f4* s_stats, const float* x, int64_t outer, int64_t inner,
                                    int64_t P, int64_t P_cap, int64_t p, float eps, LnCtrl* ctrl, uint32_t* counters,
                                    double* lbd, double* lbdx, f4* stats, float* mean_out, float* rstd_out,
                                    bool may_recompute, uint32_t limit, bool silent, double* rc, uint32_t* rc_cnt,
                                    double* rc_inv)
{
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t target = dev_load(&ctrl->gen) + 1u;
    const uint32_t tag = ln_tag_of(target);
    const double inv_mine = inv_count_f64((uint32_t)wg_cnt[p]);
    const int64_t steps = outer + LAG;
    const int64_t nv = inner / 4;
    // polls before a wait gives up: with recompute allowed, then compute
    // what is missing; without (a cooperative launch, every workgroup
    // resident), set the error word and go on
    const uint32_t wait = may_recompute ? limit : kSpinLimit;
    // (mean hi, mean lo, rstd) from the tagged words
    auto unpack = [](double tm, double tr) {
        const double m = ln_untag(tm);
        const float hi = (float)m;
        return f4{hi, (float)(m - (double)hi), (float)ln_untag(tr), 0.0f};
    };
    // Arrivals are counted AHEAD iterations early.  A merge lengthens the
    // merger's iteration, and the arrival it issues next (at sample t +
    // AHEAD) then comes late, so its workgroup is elected again AHEAD + 1
    // samples on: the merges rotate over AHEAD + 1 workgroups.  With a lag
    // of 3 (the wide tile) two ahead measured faster per call at [16, 4M]
    // (98.1-98.7 against 99.9-100.3 us), [32, 4M] and [4, 4M]; with a lag of
    // 2 (the 8 x 8 tile) it measured slower ([64, 256K] 373 against 348-353
    // us: the workgroup elected two iterations back has often caught up and
    // waits for the laggard's words), so one ahead there.
    constexpr int AHEAD = LAG - 1;
    static_assert(AHEAD >= 1, "arrivals are counted at least an iteration ahead");
    static_assert(kRing >= LAG + AHEAD, "an arrival is counted before the statistics kRing samples back are read");
    // (returns this arrival's count in lane 0; its round trip is waited for
    // only where the count is used, an iteration later, as long as the
    // compiler's atomic optimizer is off for this file)
    auto arrive = [&](int64_t s) {
        return __hip_atomic_fetch_add(counters + (s % kRing) * kCounterStride, 1u, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
    };
    // Merge sample s from every workgroup's tagged words (lane l: workgroups
    // l, l + 64, ...; the k-way pairwise update around workgroup 0's mean)
    // and announce its mean and rstd; returns the two announced words
    // (uniform).  A word still missing after `wait` polls belongs to a
    // workgroup that is not resident: with recompute allowed it is computed
    // here from x with the same bits and stored in the owner's slot (the
    // owner, once it runs, stores the same bits there); x of sample s is
    // intact, since this path never runs in place.
    auto merge_sample = [&](int64_t s, double& wm, double& wr) {
        const double* xs = lbdx + s * 2 * P_cap;  // P_cap tagged means, then P_cap tagged M2s
        double c = 0.0, A = 0.0, B = 0.0;
        for (int64_t j0 = 0; j0 < P; j0 += 4 * kWave) {
            double a[4], b2[4];
            auto load_block = [&]() __attribute__((always_inline)) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int64_t j = j0 + lane + (int64_t)u * kWave;
                    const int64_t jj = j < P ? j : 0;
                    a[u] = dev_load(xs + jj);
                    b2[u] = dev_load(xs + P_cap + jj);
                }
            };
            auto present = [&](int u) __attribute__((always_inline)) {
                return j0 + lane + (int64_t)u * kWave >= P || (ln_has_tag(a[u], tag) && ln_has_tag(b2[u], tag));
            };
            auto block_ok = [&]() __attribute__((always_inline)) {
                bool ok = true;
#pragma unroll
                for (int u = 0; u < 4; ++u) ok = ok && present(u);
                return __all(ok);
            };
            load_block();
            bool late = false;
            for (uint32_t it = 0; !block_ok(); ++it) {
                if (it == wait) {
                    late = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
                load_block();
            }
            if (late && !may_recompute) {
                if (lane == 0) dev_store(&ctrl->error, 1u);
            } else if (late) {
                const f4* xg = reinterpret_cast<const f4*>(x + s * inner);
                uint32_t n_done = 0;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    uint64_t todo = __ballot(!present(u));
                    while (todo) {
                        const int l = __builtin_ctzll(todo);
                        todo &= todo - 1;
                        const uint32_t jj = (uint32_t)(j0 + l + u * kWave);
                        double mean, m2;
                        ctl_recompute<F4PT, DW>(xg, jj, (uint32_t)P, nv, rc, rc_cnt, rc_inv, mean, m2);
                        const double tm = ln_tag_word(mean, tag), tv = ln_tag_word(m2, tag);
                        if (lane == l) {
                            a[u] = tm;
                            b2[u] = tv;
                        }
                        if (lane == 0) {
                            dev_store(lbdx + s * 2 * P_cap + jj, tm);
                            dev_store(lbdx + s * 2 * P_cap + P_cap + jj, tv);
                        }
                        ++n_done;
                    }
                }
                if (lane == 0)
                    __hip_atomic_fetch_add(&ctrl->recomputed, n_done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            if (j0 == 0) c = ln_untag(lane_f64(a[0], 0));  // workgroup 0's mean
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t j = j0 + lane + (int64_t)u * kWave;
                if (j < P) {
                    const double nj = (double)wg_cnt[j];
                    const double d = ln_untag(a[u]) - c;
                    A += nj * d;
                    B += ln_untag(b2[u]) + nj * (d * d);
                }
            }
        }
        A = wave_total(A);
        B = wave_total(B);
        const double n = (double)inner;
        const double md = A / n;
        const double m = c + md, m2s = fmax(B - A * md, 0.0);
        const double var = m2s / n;
        wm = ln_tag_word(m, tag);
        wr = ln_tag_word(1.0 / sqrt(var + (double)eps), tag);
        if (lane == 0) {
            dev_store(lbd + 2 * s, wm);
            dev_store(lbd + 2 * s + 1, wr);
            const f4 st = unpack(wm, wr);
            stats[s] = st;
            if (mean_out) mean_out[s] = st.x;
            if (rstd_out) rstd_out[s] = st.z;
        }
    };
    // counts before this workgroup's arrivals at the next AHEAD samples
    // (lane 0; q[i]: sample t + i); a silent workgroup (test knob) neither
    // arrives nor stores its words
    uint32_t q[AHEAD];
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) q[i] = lane == 0 && !silent && i < outer ? arrive(i) : 0u;
    __syncthreads();  // prologue: w/b in LDS
    for (int64_t t = 0; t < steps; ++t) {
        __syncthreads();  // barrier t: the wave moments of sample t are in LDS
        const int64_t g = t - (LAG - 1);
        const bool gather = g >= 0 && g < outer;
        // sample t's arrival was counted AHEAD iterations ago; count sample t + AHEAD's now
        const uint32_t before = q[0];
#pragma unroll
        for (int i = 0; i + 1 < AHEAD; ++i) q[i] = q[i + 1];
        if (t + AHEAD < outer && lane == 0 && !silent) q[AHEAD - 1] = arrive(t + AHEAD);
        double tm = 0.0, tr = 0.0;
        if (gather && lane == 0) {
            tm = dev_load(lbd + 2 * g);
            tr = dev_load(lbd + 2 * g + 1);
        }
        if (t < outer) {
            // this workgroup's (mean, M2) of sample t, tagged, into its slot
            double mean, m2;
            merge_wave_moments<DW>(red[t & 1], cnt, cnt_inv, inv_mine, mean, m2);
            double* xs = lbdx + t * 2 * P_cap;
            if (lane == 0 && !silent) {
                dev_store(xs + p, ln_tag_word(mean, tag));
                dev_store(xs + P_cap + p, ln_tag_word(m2, tag));
            }
            if (__builtin_amdgcn_readfirstlane(lane == 0 && !silent && (before + 1u) % (uint32_t)P == 0u ? 1u : 0u)) {
                // the last arrival merges the sample and takes P back off the counter
                double wm, wr;
                merge_sample(t, wm, wr);
                if (lane == 0)
                    __hip_atomic_fetch_sub(counters + (t % kRing) * kCounterStride, (uint32_t)P, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        if (gather) {
            // sample g's statistics; if they do not come (no workgroup was
            // elected: one is not resident), merge the sample here
            bool ok = false;
            for (uint32_t it = 0;; ++it) {
                ok = __builtin_amdgcn_readfirstlane(lane == 0 && ln_has_tag(tm, tag) && ln_has_tag(tr, tag) ? 1u : 0u);
                if (ok || it == wait) break;
                __builtin_amdgcn_s_sleep(1);
                if (lane == 0) {
                    tm = dev_load(lbd + 2 * g);
                    tr = dev_load(lbd + 2 * g + 1);
                }
            }
            if (!ok && may_recompute) {
                double wm, wr;
                merge_sample(g, wm, wr);
                tm = wm;
                tr = wr;
            } else if (!ok && lane == 0) {
                dev_store(&ctrl->error, 1u);
            }
            if (lane == 0) s_stats[g & 1] = unpack(tm, tr);
        }
    }
    // completion: the last workgroup out advances the generation
    if (lane == 0) {
        vmem_drain();
        if (__hip_atomic_fetch_add(&ctrl->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(P - 1)) {
            dev_store(&ctrl->done, 0u);
            vmem_drain();
            dev_store(&ctrl->gen, target);
        }
    }
}

// Iterations of ln_single_ctl_kernel with compile-time tile indices:
// ctl_first_steps runs iterations 0 .. LAG-1 (moments only); ctl_steps runs
// t0 + U, t0 + U + 1, ... for U < NT (iteration t uses tile (t0 + U) % NT,
// t0 = LAG mod NT), stopping after the last of `steps` iterations, and
// returns false once that one has run.
template <int U, int LAG, typename F>
__device__ __forceinline__ void ctl_first_steps(F& f)
{
    if constexpr (U < LAG) {
        f((int64_t)U, std::integral_constant<int, U>{}, std::false_type{});
        ctl_first_steps<U + 1, LAG>(f);
    }
}
template <int U, int NT, int LAG, typename F>
__device__ __forceinline__ bool ctl_steps(int64_t t0, int64_t steps, F& f)
{
    if constexpr (U == NT) {
        return true;
    } else {
        f(t0 + U, std::integral_constant<int, (LAG + U) % NT>{}, std::true_type{});
        if (t0 + U + 1 >= steps) return false;
        return ctl_steps<U + 1, NT, LAG>(t0, steps, f);
    }
}

template <int F4PT, int DW, int LAG, int PROTO, bool ILV>
__global__ void __launch_bounds__((DW + 1) * kWave)
ln_single_ctl_kernel(const float* x_all, const float* w, const float* bias, float* y_all, int64_t outer_all,
                     int64_t inner, int64_t P_cap, float eps, LnCtrl* ctrl, f4* stats_all, double* xchg_all,
                     float* mean_all, float* rstd_all, int64_t groups, uint32_t spin_limit, uint32_t silent_mask,
                     uint32_t* counters, double* lbd, double* lbdx)
{
    constexpr int RW = DW * kWave;  // row width in float4 = data threads
    constexpr int NT = LAG + 2;     // register tiles per data thread
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    __shared__ double red[2][3 * DW];  // [sample parity][wave]: t1, t2, shift
    __shared__ f4 s_stats[2];          // [sample parity]: mean hi, mean lo, rstd
    __shared__ double rc[3 * DW];      // control wave: a recomputed workgroup's wave moments
    __shared__ uint32_t cnt[2][DW];    // control wave: element counts of this workgroup's / a recomputed one's waves
    __shared__ double cnt_inv[2][DW];  // ... and their reciprocals
    __shared__ float wg_cnt[1024];     // control wave: element count of every workgroup of a group (P <= 1024)
    f4* w_s = reinterpret_cast<f4*>(smem_raw);
    f4* b_s = w_s + (w ? F4PT * RW : 0);
    // `groups` groups of P workgroups; group gr takes samples gr, gr + groups,
    // ... as its own sequence (local sample i is sample gr + i * groups), so
    // a grid of groups x P workgroups fills the GPU when one sample spreads
    // over fewer.  Below, x, y, xchg, stats, mean_out, rstd_out and outer
    // are the group's view: local sample i at x + i * sstride, and so on.
    // Workgroup j's exchange words for a sample are its tagged mean and M2,
    // at the start of its slot of XS doubles.
    const int64_t P = gridDim.x / groups;
    const int64_t gr = blockIdx.x / P;
    const int64_t p = blockIdx.x - gr * P;
    const int64_t sstride = groups * inner;       // elements between the group's samples
    constexpr int64_t XS = NORMFWD_LN_XCHG_SLOT;  // doubles per workgroup slot (0: all means, then all M2s)
    const int64_t sw = XS ? XS * P_cap : 2 * P_cap;  // exchange words per sample
    const int64_t xstride = groups * sw;          // exchange words between the group's samples
    const int64_t xm2 = XS ? 1 : P_cap;           // M2 word relative to the mean word
    const int64_t xj = XS ? XS : 1;               // words between workgroups
    const float* x = x_all + gr * inner;
    float* y = y_all + gr * inner;
    double* xchg = xchg_all + gr * sw;
    f4* stats = stats_all + gr;
    float* mean_out = mean_all ? mean_all + gr : nullptr;
    float* rstd_out = rstd_all ? rstd_all + gr : nullptr;
    const int64_t outer = (outer_all - gr + groups - 1) / groups;  // >= 1: groups <= outer_all
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int64_t nv = inner / 4;
    const int64_t steps = outer + LAG;  // iterations = barriers after the prologue

    if (tid >= RW && PROTO == 1) {
        // ---- control wave, last workgroup merges (groups == 1)
        // (issued ahead of the data waves of its SIMD: see the control wave
        // below; priority 1 here measured ~1 us faster per call than 2 or 3
        // at [16, 4M]: 98.3-98.8 against 99.3-100.2 us, five alternations)
        __builtin_amdgcn_s_setprio(1);
        if (lane < DW) {
            const uint32_t n = ctl_wave_elems<F4PT, DW>((uint32_t)p, lane, (uint32_t)P, nv);
            cnt[0][lane] = n;
            cnt_inv[0][lane] = inv_count_f64(n);
        }
        for (int64_t j = lane; j < P; j += kWave) wg_cnt[j] = (float)ctl_wg_elems<F4PT, DW>((uint32_t)j, (uint32_t)P, nv);
        // Not in place, the launch is an ordinary one and a workgroup that
        // is not resident has its moments computed by the others (x stays
        // intact); in place it is cooperative, every workgroup resident.
        const bool may_recompute = x_all != y_all;
        const bool silent = may_recompute && ((uint32_t)p & silent_mask) == silent_mask;
        ctl_wave_last_block<F4PT, DW, LAG>(red, cnt[0], cnt_inv[0], wg_cnt, s_stats, x_all, outer, inner, P, P_cap, p,
                                           eps, ctrl, counters, lbd, lbdx, stats, mean_out, rstd_out, may_recompute,
                                           spin_limit, silent, rc, cnt[1], cnt_inv[1]);
        return;
    }
    if (tid >= RW) {
        // ---- control wave
        // Raised wave priority: the SIMD's arbiter issues this wave's
        // instructions ahead of the two data waves beside it, so the exchange
        // (its LDS reads, merges and publication) is not queued behind their
        // streaming.  Measured per call on MI355X, priority 2 against the
        // default: [16, 4M] 92.1-92.5 against 93.9-94.7 us, [8, 4M] 47.5-48.1
        // against 48.8-49.6, [4, 4M] 25.8-25.9 against 26.8-27.1 (priority
        // 3), [64, 4M] 353.0-353.1 against 350.8-351.6, [16, 3M] 75.4-75.5
        // against 74.3-75.2, the rest within 0.5 us; the last-workgroup-
        // merges kernel [16, 4M] 99.1-99.4 against 109.6-110.9 us, [64, 256K]
        // 345-350 against 386 (priorities 1, 2 and 3 within each other's
        // spread).  Outputs bitwise equal.
        __builtin_amdgcn_s_setprio(2);
        const uint32_t gen_target = ln_next_generation(dev_load(&ctrl->gen_ctl));
        const uint32_t tag = ln_tag_of(gen_target);
        uint32_t limit = spin_limit;
        // test knob: a silent workgroup does not publish at all, so every
        // reader (itself included) computes its moments from x
        const bool silent = ((uint32_t)p & silent_mask) == silent_mask;
        if (lane < DW) {
            const uint32_t n = ctl_wave_elems<F4PT, DW>((uint32_t)p, lane, (uint32_t)P, nv);
            cnt[0][lane] = n;
            cnt_inv[0][lane] = inv_count_f64(n);
        }
        for (int64_t j = lane; j < P; j += kWave) wg_cnt[j] = (float)ctl_wg_elems<F4PT, DW>((uint32_t)j, (uint32_t)P, nv);
        const double inv_mine = inv_count_f64(ctl_wg_elems<F4PT, DW>((uint32_t)p, (uint32_t)P, nv));
        const double inv_N = 1.0 / (double)inner;
        __syncthreads();  // prologue: w/b in LDS
        for (int64_t t = 0; t < steps; ++t) {
            __syncthreads();  // barrier t: the wave moments of sample t are in LDS
            const int64_t g = t - (LAG - 1);  // the sample gathered now, normalized after barrier g + LAG
            const bool gather = g >= 0 && g < outer;
            // gather every workgroup's words for sample g (lane l: workgroups
            // l, l + 64, ...), retrying until every tag is current.  The first
            // loads are issued before this workgroup merges and publishes its
            // own moments of sample t, so that work overlaps their latency.
            const double* xb = xchg + (gather ? g : 0) * xstride;
            double a[4], b2[4];
            auto load_block = [&](int64_t j0) __attribute__((always_inline)) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int64_t j = j0 + lane + (int64_t)u * kWave;
                    const int64_t jj = j < P ? j : p;
                    a[u] = dev_load(xb + jj * xj);
                    b2[u] = dev_load(xb + jj * xj + xm2);
                }
            };
            auto block_ok = [&]() __attribute__((always_inline)) {
                bool ok = true;
#pragma unroll
                for (int u = 0; u < 4; ++u) ok = ok && ln_has_tag(a[u], tag) && ln_has_tag(b2[u], tag);
                return __all(ok);
            };
            if (gather) load_block(0);
            if (t < outer) {
                // this workgroup's (mean, M2) over its elements of sample t
                double mean, m2;
                merge_wave_moments<DW>(red[t & 1], cnt[0], cnt_inv[0], inv_mine, mean, m2);
                if (lane == 0 && !silent) {
                    double* xt = xchg + t * xstride;
                    dev_store(xt + p * xj, ln_tag_word(mean, tag));
                    dev_store(xt + p * xj + xm2, ln_tag_word(m2, tag));
                }
            }
            if (!gather) continue;
            // Words that have not arrived after `limit` polls (their workgroup
            // is not resident: an ordinary launch does not promise that every
            // workgroup runs at once) are computed here from x, with the same
            // bits, and published in the owner's slot for the other readers
            // (the owner, once it runs, stores the same bits there).  x of
            // sample g is still intact: the kernel does not run in place.
            double c = 0.0, A = 0.0, B = 0.0;  // shift, sum n_j (mean_j - c), sum M2_j + n_j (mean_j - c)^2
            for (int64_t j0 = 0; j0 < P; j0 += 4 * kWave) {
                if (j0 > 0) load_block(j0);
                uint32_t spins = 0;
                bool late = false;
                while (!block_ok()) {
                    __builtin_amdgcn_s_sleep(2);
                    if (++spins > limit) {
                        late = true;
                        break;
                    }
                    load_block(j0);
                }
                if (late) {
                    // from now on this workgroup waits only briefly
                    limit = std::min(limit, kSpinLimitAfterMiss);
                    const f4* xg = reinterpret_cast<const f4*>(x + g * sstride);
                    uint32_t n_done = 0;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int64_t j = j0 + lane + (int64_t)u * kWave;
                        uint64_t todo = __ballot(j < P && !(ln_has_tag(a[u], tag) && ln_has_tag(b2[u], tag)));
                        while (todo) {
                            const int l = __builtin_ctzll(todo);
                            todo &= todo - 1;
                            const uint32_t jj = (uint32_t)(j0 + l + u * kWave);
                            double mean, m2;
                            ctl_recompute<F4PT, DW>(xg, jj, (uint32_t)P, nv, rc, cnt[1], cnt_inv[1], mean, m2);
                            const double tm = ln_tag_word(mean, tag), tv = ln_tag_word(m2, tag);
                            if (lane == l) {
                                a[u] = tm;
                                b2[u] = tv;
                            }
                            if (lane == 0) {
                                double* xq = xchg + g * xstride;
                                dev_store(xq + jj * xj, tm);
                                dev_store(xq + jj * xj + xm2, tv);
                            }
                            ++n_done;
                        }
                    }
                    if (lane == 0)
                        __hip_atomic_fetch_add(&ctrl->recomputed, n_done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                if (j0 == 0) c = ln_untag(lane_f64(a[0], 0));  // workgroup 0's mean
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int64_t j = j0 + lane + (int64_t)u * kWave;
                    if (j < P) {
                        const double nj = (double)wg_cnt[j];
                        const double d = ln_untag(a[u]) - c;
                        A += nj * d;
                        B += ln_untag(b2[u]) + nj * (d * d);
                    }
                }
            }
            A = wave_total(A);
            B = wave_total(B);
            if (lane == 0) {
                const double md = A * inv_N;
                const f4 st = finish_stats((double)inner, c + md, fmax(B - A * md, 0.0), eps);
                s_stats[g & 1] = st;
                if (p == 0) {
                    stats[g * groups] = st;
                    if (mean_out) mean_out[g * groups] = st.x;
                    if (rstd_out) rstd_out[g * groups] = st.z;
                }
            }
        }
        // completion: the last workgroup out advances the generation
        if (lane == 0) {
            vmem_drain();
            if (__hip_atomic_fetch_add(&ctrl->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                gridDim.x - 1u) {
                dev_store(&ctrl->done, 0u);
                vmem_drain();
                dev_store(&ctrl->gen_ctl, gen_target);
            }
        }
        return;
    }

    // ---- data waves.  Element k of this thread is float4 index(k) of row
    // p + k P (< 2^32), present iff index(k) < nv.  Loads are issued
    // unconditionally, clamped to a valid address and masked where used: the
    // memory counter retires in issue order, so with a fixed number of loads
    // per iteration a wave can wait for one tile while the next is in flight.
    // A tile past the last sample reads one fixed address (no traffic).
    // the wave's index, in a scalar register (it is the same in every lane)
    const int wave_id = __builtin_amdgcn_readfirstlane(tid / kWave);
    const float inv_wave = inv_count_f32(ctl_wave_elems<F4PT, DW>((uint32_t)p, wave_id, (uint32_t)P, nv));
    uint32_t off0 = (uint32_t)p * RW + (uint32_t)tid;
    const uint32_t stride = (uint32_t)P * RW;
    auto index = [&](int k) -> uint32_t { return off0 + (uint32_t)k * stride; };
    auto valid = [&](int k) -> bool { return (int64_t)index(k) < nv; };
    const uint32_t last_unit = (uint32_t)(nv - 1);
    auto addr = [&](int k) -> uint32_t { return std::min(index(k), last_unit); };
    f4 T[NT][F4PT];  // register tiles; sample s lives in tile s % NT
    // Sample s's row and the mask applied to every index: past the last
    // sample every lane reads the last sample's first float4 (index masked to
    // 0): same instruction count, no traffic.
    struct Row {
        const f4* xs;
        uint32_t m;
    };
    auto row = [&](int64_t s) __attribute__((always_inline)) {
        const int64_t sb = s < outer ? s : outer - 1;
        return Row{reinterpret_cast<const f4*>(x + sb * sstride), s < outer ? 0xFFFFFFFFu : 0u};
    };
    // Streaming loads: x is read once here (measured ~1% faster).
    auto load = [&](int r, int64_t s) __attribute__((always_inline)) {
        const Row q = row(s);
#pragma unroll
        for (int k = 0; k < F4PT; ++k) T[r][k] = ld_nt(q.xs + (addr(k) & q.m));
    };
    // weight and bias rows -> LDS: both rows' loads in flight together (tiles
    // 0 and 1), then the LDS stores; one round trip instead of one per row.
    // Per call on MI355X against weight first, then bias: [16, 4M] 91.9-92.3
    // against 92.6-93.1 us, [1, 4M] 14.8-15.0 against 15.4-15.7, [16, 1M]
    // 26.4-27.2 against 27.4-28.1, variant 2 [16, 4M] 98.1-98.3 against
    // 98.9-99.4; [4, 4M] and [64, 4M] even, [256, 16K] 11.9-12.0 against
    // 11.7-11.8.
    static_assert(NT >= 2, "two register tiles hold weight and bias");
    if (w) {
#pragma unroll
        for (int k = 0; k < F4PT; ++k) T[0][k] = reinterpret_cast<const f4*>(w)[addr(k)];
    }
    if (bias) {
#pragma unroll
        for (int k = 0; k < F4PT; ++k) T[1][k] = reinterpret_cast<const f4*>(bias)[addr(k)];
    }
    if (w) {
#pragma unroll
        for (int k = 0; k < F4PT; ++k) w_s[k * RW + tid] = T[0][k];
    }
    if (bias) {
#pragma unroll
        for (int k = 0; k < F4PT; ++k) b_s[k * RW + tid] = T[1][k];
    }
#pragma unroll
    for (int r = 0; r < NT - LAG; ++r) load(r, r);
    __syncthreads();  // prologue: w/b in LDS

    // One iteration with its register tiles fixed at compile time: the loop
    // below unrolls NT of them, so no tile is ever copied (a copy would wait
    // for the loads that fill it).
    auto step = [&](int64_t t, auto U, auto NORM) __attribute__((always_inline)) {
        constexpr int u = decltype(U)::value;     // tile of sample t
        constexpr int r = (u + NT - LAG) % NT;    // tile of sample t - LAG
        constexpr bool norm = decltype(NORM)::value;  // t >= LAG
        // the per-row offsets are recomputed in every iteration instead of
        // being kept live across the loop (registers hold NT x tiles)
        asm volatile("" : "+v"(off0));
        if (t < outer) {
            // two passes over the tile (see WaveMoments; ctl_recompute repeats them)
            f4 s = f4(0.0f);
#pragma unroll
            for (int k = 0; k < F4PT; ++k) s += valid(k) ? T[u][k] : f4(0.0f);
            const float m = wave_shift(s, inv_wave);
            f4 a1 = f4(0.0f), a2 = f4(0.0f);
#pragma unroll
            for (int k = 0; k < F4PT; ++k) shifted_acc(a1, a2, valid(k) ? T[u][k] - m : f4(0.0f));
            double t1, t2;
            wave_moments(a1, a2, t1, t2);
            if (lane == 0) {
                double* rd = red[t & 1] + 3 * wave_id;
                rd[0] = t1;
                rd[1] = t2;
                rd[2] = (double)m;
            }
        }
        __syncthreads();  // barrier t: sample t-LAG's statistics are in LDS
        // tile r then receives sample t-LAG+NT (in the first LAG iterations it
        // is still empty); the loads are unconditional so that every iteration
        // issues the same memory operations
        if constexpr (norm) {
            const int64_t s = t - LAG;
            const f4 st = s_stats[s & 1];
            f4* y4 = reinterpret_cast<f4*>(y + s * sstride);
            // ILV: each element's store is followed at once by its register's
            // refill, so loads enter the queue while the stores drain; else
            // all stores, then all loads
            const Row q = row(t - LAG + NT);
#pragma unroll
            for (int k = 0; k < F4PT; ++k) {
                if (valid(k)) {
                    const f4 tt = ((T[r][k] - st.x) - st.y) * st.z;
                    const f4 wv = w ? w_s[k * RW + tid] : f4(1.0f);
                    const f4 bv = bias ? b_s[k * RW + tid] : f4(0.0f);
                    st_nt(tt * wv + bv, y4 + index(k));
                }
                if constexpr (ILV) T[r][k] = ld_nt(q.xs + (addr(k) & q.m));
            }
            if constexpr (!ILV) load(r, t - LAG + NT);
        } else {
            load(r, t - LAG + NT);
        }
    };
    // the first LAG iterations have nothing to normalize yet; from then on
    // every iteration does (t < steps = outer + LAG, and outer >= 1)
    ctl_first_steps<0, LAG>(step);
    for (int64_t t0 = LAG; ctl_steps<0, NT, LAG>(t0, steps, step); t0 += NT) {
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
    uint32_t* counters =
        outer * lay.P < NORMFWD_LN_FUSE_BELOW ? reinterpret_cast<uint32_t*>(base + lay.off_split_counter) : nullptr;
    const bool vec4 = (inner % 4 == 0) && is_aligned16(x);
    const int64_t per = samples_per_launch(lay.P * kLnThreads);
    for (int64_t b0 = 0; b0 < outer; b0 += per) {
        const int64_t nb = std::min(per, outer - b0);
        const float* xb = x + b0 * inner;
        Partial* pb = parts + b0 * lay.P_cap;
        uint32_t* cb = counters ? counters + b0 * kCounterStride : nullptr;
        float* mb = mean_out ? mean_out + b0 : nullptr;
        float* rb = rstd_out ? rstd_out + b0 : nullptr;
        const dim3 grid((unsigned)(nb * lay.P));
        hipError_t e = vec4 ? launch_kernel(ln_partial_kernel<4>, grid, dim3(kLnThreads), 0, st, xb, inner, lay.P,
                                            lay.P_cap, pb, cb, eps, stats + b0, mb, rb)
                            : launch_kernel(ln_partial_kernel<1>, grid, dim3(kLnThreads), 0, st, xb, inner, lay.P,
                                            lay.P_cap, pb, cb, eps, stats + b0, mb, rb);
        if (e != hipSuccess) return e;
        if (!counters) {
            e = launch_kernel(ln_merge_kernel, dim3((unsigned)nb), dim3(kWave), 0, st, pb, lay.P, lay.P_cap, eps,
                              stats + b0, mb, rb);
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

hipError_t launch_ln_apply(const float* x, const float* w, const float* b, float* y, int64_t outer,
                           int64_t inner, const void* ws, const LnLayout& lay, hipStream_t st)
{
    const f4* stats = reinterpret_cast<const f4*>(static_cast<const char*>(ws) + lay.off_stats);
    const bool vec4 = (inner % 4 == 0) && is_aligned16(x) && is_aligned16(y) && is_aligned16(w) && is_aligned16(b);
    const int64_t nu = vec4 ? inner / 4 : inner;
    int64_t bps = ceil_div(nu, (int64_t)kLnThreads * NORMFWD_LN_NORM_ROWS);
    // The XCD mapping needs a multiple of 8 rows per sample and pays off
    // only when weight/bias are read for several samples.
    int xcd_map = 0;
    if (NORMFWD_LN_XCD_MAP && outer > 1 && bps >= 8 && (w || b)) {
        bps = ceil_div(bps, 8) * 8;
        xcd_map = 1;
    }
    // The sample loop needs enough rows per sample to fill the GPU (each of
    // its workgroups walks all `outer` samples); short samples use one row
    // per workgroup.
    const int64_t rows = ceil_div(nu, (int64_t)kLnThreads);
    if (NORMFWD_LN_NORM_MODE == 1 && rows >= 1024 && rows * kLnThreads <= max_grid_items()) {
        const dim3 g((unsigned)rows);
        return vec4 ? launch_kernel(ln_normalize_rows_kernel<4>, g, dim3(kLnThreads), 0, st, x, w, b, y, outer,
                                    inner, stats)
                    : launch_kernel(ln_normalize_rows_kernel<1>, g, dim3(kLnThreads), 0, st, x, w, b, y, outer,
                                    inner, stats);
    }
    const int64_t per = samples_per_launch(bps * kLnThreads);
    for (int64_t b0 = 0; b0 < outer; b0 += per) {
        const int64_t nb = std::min(per, outer - b0);
        const float* xb = x + b0 * inner;
        float* yb = y + b0 * inner;
        const int xm = nb > 1 ? xcd_map : 0;
        const dim3 grid((unsigned)(nb * bps));
        const hipError_t e = vec4 ? launch_kernel(ln_normalize_kernel<4>, grid, dim3(kLnThreads), 0, st, xb, w, b, yb,
                                                  nb, inner, bps, xm, stats + b0)
                                  : launch_kernel(ln_normalize_kernel<1>, grid, dim3(kLnThreads), 0, st, xb, w, b, yb,
                                                  nb, inner, bps, xm, stats + b0);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

bool launch_ln_rows(const float* x, const float* w, const float* b, float* y, int64_t outer, int64_t inner, float eps,
                    float* mean_out, float* rstd_out, hipStream_t st, hipError_t& err)
{
    const bool vec4 = (inner % 4 == 0) && is_aligned16(x) && is_aligned16(y) && is_aligned16(w) && is_aligned16(b);
    const int64_t nu = vec4 ? inner / 4 : inner;
    const int64_t per = samples_per_launch(kLnThreads);
#define NORMFWD_ROWS(VEC, U)                                                                                     \
    if (nu <= (int64_t)kLnThreads * (U)) {                                                                       \
        for (int64_t b0 = 0; b0 < outer; b0 += per) {                                                            \
            const int64_t nb = std::min(per, outer - b0);                                                        \
            err = launch_kernel((ln_row_kernel<VEC, U>), dim3((unsigned)nb), dim3(kLnThreads), 0, st,            \
                                x + b0 * inner, w, b, y + b0 * inner, inner, eps,                                \
                                mean_out ? mean_out + b0 : nullptr, rstd_out ? rstd_out + b0 : nullptr);         \
            if (err != hipSuccess) break;                                                                        \
        }                                                                                                        \
        return true;                                                                                             \
    }
    if (vec4) {
        NORMFWD_ROWS(4, 1)
        NORMFWD_ROWS(4, 2)
        NORMFWD_ROWS(4, 4)
        NORMFWD_ROWS(4, 8)
    } else {
        NORMFWD_ROWS(1, 1)
        NORMFWD_ROWS(1, 2)
        NORMFWD_ROWS(1, 4)
        NORMFWD_ROWS(1, 8)
    }
#undef NORMFWD_ROWS
    return false;
}

struct DeviceInfo {
    int cus = 0;
    int max_lds_per_block = 0;
};

static bool device_info(DeviceInfo& out)
{
    static std::mutex mu;
    static DeviceInfo info[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
    std::lock_guard<std::mutex> lock(mu);
    DeviceInfo& d = info[dev];
    if (d.cus == 0) {
        if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
        if (hipDeviceGetAttribute(&d.max_lds_per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
            hipSuccess)
            return false;
    }
    out = d;
    return true;
}

// Co-resident workgroups of `fn` with `lds` bytes of dynamic LDS on this
// device (queried once per device, kernel and LDS size).  A workgroup whose
// wave count is not a multiple of the CU's 4 SIMDs is counted once per CU
// whatever the occupancy query says: the query assumes its waves can be
// spread over the SIMDs freely, and a tuning run of such a kernel at two
// workgroups per CU (5 waves of 168 VGPRs each) did not finish.
static int coresident(const void* fn, size_t lds, int threads)
{
    struct Entry {
        int dev;
        const void* fn;
        size_t lds;
        int threads;
        int cap;
    };
    static std::mutex mu;
    static Entry cache[64];
    static int n_cache = 0;
    DeviceInfo d;
    if (!device_info(d)) return 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < n_cache; ++i)
        if (cache[i].dev == dev && cache[i].fn == fn && cache[i].lds == lds && cache[i].threads == threads)
            return cache[i].cap;
    int cap = 0;
    if (lds == 0 || hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) == hipSuccess) {
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds) == hipSuccess) {
            if ((threads / kWave) % 4 != 0) per_cu = std::min(per_cu, 1);
            cap = d.cus * per_cu;
        }
    }
    (void)hipGetLastError();
    if (n_cache < 64) cache[n_cache++] = Entry{dev, fn, lds, threads, cap};
    return cap;
}

// Launches ln_single_ctl_kernel<F4PT, DW, LAG, PROTO, ILV> when a co-resident grid
// of one workgroup per F4PT rows of DW * 64 float4 holds every sample's rows
// (false: it cannot, nothing launched).  PROTO 0, the tagged exchange: an
// ordinary launch; PROTO 1, the last workgroup merging: an ordinary one,
// and a cooperative one in place.
template <int F4PT, int DW, int LAG, int PROTO, bool ILV>
static bool try_launch_single(const float* x, const float* w, const float* b, float* y, int64_t outer,
                              int64_t inner, float eps, LnCtrl* ctrl, uint32_t* counters, double* lbd, f4* stats,
                              double* lbdx, double* xchg, int64_t P_cap, float* mean_out, float* rstd_out,
                              hipStream_t st, hipError_t& err)
{
    DeviceInfo d;
    if (!device_info(d)) return false;
    const int64_t rw = DW * kWave;
    const int64_t rows = ceil_div(inner / 4, rw);
    const int64_t P = ceil_div(rows, (int64_t)F4PT);
    if (P > P_cap) return false;
    const size_t lds = (size_t)((w ? 1 : 0) + (b ? 1 : 0)) * F4PT * rw * sizeof(f4);
    // Whether a tile fits is decided as if both weight and bias were given,
    // so a shape always runs the same tile (the tagged exchange relies on
    // every launch on a workspace writing the same slots).
    const size_t lds_max = (size_t)2 * F4PT * rw * sizeof(f4);
    if (lds_max + 8 * 1024 > (size_t)d.max_lds_per_block) return false;
    const void* fn = reinterpret_cast<const void*>(&ln_single_ctl_kernel<F4PT, DW, LAG, PROTO, ILV>);
    const int threads = (DW + 1) * kWave;
    const int cap = coresident(fn, lds_max, threads);
    if (cap < P) return false;
    int64_t pcap = P_cap;
    if constexpr (PROTO == 0) {
        // An ordinary launch (a cooperative one costs ~17 us more per call on
        // MI355X).  The grid fits the device, so normally every workgroup is
        // resident at once; when one is not (another kernel holds its CU), the
        // others compute its moments themselves after a bounded wait, so the
        // launch completes with the same result either way.  That needs x
        // intact until the end, so in place (y == x) never comes here.  Test
        // knob: force that path for every k-th workgroup: workgroup j is
        // forced (publishes nothing) iff (j & mask) == mask; all ones forces
        // none (P <= 1024).  The wait for a forced workgroup is cut short (8
        // polls) in that mode.
        if (x == y) return false;
        const uint32_t k = ln_force_recompute();
        const uint32_t force = k ? k - 1u : 0xFFFFFFFFu;
        // as many groups of P workgroups (each taking every groups-th
        // sample) as stay co-resident, at most one per sample
        const int64_t groups = std::max<int64_t>(1, std::min<int64_t>(outer, cap / P));
        err = launch_kernel(ln_single_ctl_kernel<F4PT, DW, LAG, 0, ILV>, dim3((unsigned)(groups * P)),
                            dim3(threads), (uint32_t)lds, st, x, w, b, y, outer, inner, pcap, eps, ctrl, stats, xchg,
                            mean_out, rstd_out, groups, k ? 8u : kCtlSpinLimit, force, counters, lbd, lbdx);
        return true;
    } else if (x != y) {
        // One group of P workgroups, an ordinary launch (the cooperative one
        // measured ~17 us more per call): a sample whose statistics do not
        // come (a workgroup that is not resident never arrives, so no merger
        // is elected) is merged by whoever waited for it, computing missing
        // moments from x with the same bits.  Test knob as for PROTO 0.
        const uint32_t k = ln_force_recompute();
        const uint32_t force = k ? k - 1u : 0xFFFFFFFFu;
        err = launch_kernel(ln_single_ctl_kernel<F4PT, DW, LAG, 1, ILV>, dim3((unsigned)P), dim3(threads),
                            (uint32_t)lds, st, x, w, b, y, outer, inner, pcap, eps, ctrl, stats, xchg, mean_out,
                            rstd_out, (int64_t)1, k ? 8u : kCtlSpinLimit, force, counters, lbd, lbdx);
        return true;
    } else {
        // In place: one group of P workgroups, a cooperative launch (a merge
        // from x could read rows their owner has already overwritten)
        int64_t groups = 1;
        uint32_t spin = kSpinLimit, force = 0xFFFFFFFFu;
        void* args[] = {(void*)&x,        (void*)&w,        (void*)&b,        (void*)&y,      (void*)&outer,
                        (void*)&inner,    (void*)&pcap,     (void*)&eps,      (void*)&ctrl,   (void*)&stats,
                        (void*)&xchg,     (void*)&mean_out, (void*)&rstd_out, (void*)&groups, (void*)&spin,
                        (void*)&force,    (void*)&counters, (void*)&lbd,      (void*)&lbdx};
        // a cooperative launch cannot carry events: armed ones bracket it as markers
        const LaunchEvents ev = take_launch_events();
        if (ev.start) (void)hipEventRecord(ev.start, st);
        err = hipLaunchCooperativeKernel(fn, dim3((unsigned)P), dim3(threads), args, lds, st);
        // a refused launch is reported through err; taking it off the runtime's
        // pending error keeps it from surfacing in the caller's next HIP call
        if (err == hipSuccess)
            err = hipGetLastError();
        else
            (void)hipGetLastError();
        if (err == hipSuccess && ev.stop) err = hipEventRecord(ev.stop, st);
        return true;
    }
}

bool ln_single_supported(int64_t inner, const float* x, const float* w, const float* b, const float* y)
{
    return (inner % 4 == 0) && is_aligned16(x) && is_aligned16(y) && is_aligned16(w) && is_aligned16(b);
}

// Workgroups per sample and co-resident workgroups of ln_single_ctl_kernel
// with the tile <F4PT, DW>.
template <int F4PT, int DW, int LAG>
static void single_grid(int64_t inner, int64_t& P, int& cap)
{
    P = ceil_div(ceil_div(inner / 4, (int64_t)DW * kWave), (int64_t)F4PT);
    const size_t lds = (size_t)2 * F4PT * DW * kWave * sizeof(f4);
    DeviceInfo d;
    cap = 0;
    if (!device_info(d) || lds + 8 * 1024 > (size_t)d.max_lds_per_block) return;
    cap = coresident(reinterpret_cast<const void*>(&ln_single_ctl_kernel<F4PT, DW, LAG, 0, true>), lds,
                     (DW + 1) * kWave);
}

// The wide tile where it measured faster, or where the other cannot hold
// a sample (see kLnWideWaves).
static bool ln_wide_tile(int64_t outer, int64_t inner)
{
    int64_t Pw = 0, Pn = 0;
    int capw = 0, capn = 0;
    single_grid<kLnWideF4, kLnWideWaves, kLnWideLag>(inner, Pw, capw);
    single_grid<kLnTileF4, kLnTileWaves, kLnTileLag>(inner, Pn, capn);
    if (capn < Pn) return true;
    return outer >= 4 && Pw <= capw && Pw * 10 >= (int64_t)capw * 9;
}

// Whether the 8 x 8 tile interleaves its stores with the next sample's loads
// (the wide tile always does: it runs where a sample takes at least 90% of
// the co-resident grid).  Measured per call on MI355X (median of 40
// launches, compared builds writing one shared output buffer), interleaved
// against all stores, then all loads, by workgroups per sample P out of 256
// co-resident: P = 256 [4, 4M] 27.7 vs 30.3 us; 192 [16, 3M] 74.4 vs 77.0;
// 128 [64, 2M] 176.9 vs 180.7, [32, 2M] 92.1 vs 94.3, [4, 2M] 16.4 vs 18.7;
// 112 [16, 1.75M] 44.8 vs 45.0; 96 [16, 1.5M] 40.3 vs 40.0, [8, 1.5M] 23.3
// vs 21.5; 80 [16, 1.25M] 34.2 vs 33.7; 64 [16, 1M] 27.3 vs 26.8, [32, 1M]
// 49.6 vs 49.6, [8, 1M] 16.4 vs 17.3; 16 [64, 256K] 29.3 vs 27.7; 4 [128,
// 64K] 16.1 vs 16.4; 1 [256, 16K] 12.1 vs 11.9.  So: where a sample spans at
// least half the grid.
static bool ln_tile_interleave(int64_t inner)
{
    int64_t P = 0;
    int cap = 0;
    single_grid<kLnTileF4, kLnTileWaves, kLnTileLag>(inner, P, cap);
    return 2 * P >= cap;
}

// Measured on MI355X (split against the single-read kernel with the tile
// ln_wide_tile picks and sample groups, per call, one call, 200 ms settle per
// shape): [16, 4M] 137.1 vs 97.2 us, [4, 4M] 42.6 vs 30.9, [32, 2M] 135.3 vs
// 94.2, [16, 2M] 72.0 vs 50.7, [4, 2M] 23.8 vs 19.2, [2, 2M] 14.3 vs 13.3,
// [32, 1M] 69.5 vs 49.7, [16, 1M] 40.7 vs 27.1, [8, 1M] 22.1 vs 17.7,
// [4, 1M] 12.8 vs 12.6, [2, 1M] 11.0 vs 10.5, [64, 256K] 35.0 vs 28.5,
// [16, 256K] 12.4 vs 11.9, [4, 256K] 10.2 vs 9.1, [128, 64K] 23.1 vs 17.1,
// [32, 64K] 11.9 vs 10.1, [256, 16K] 15.8 vs 11.9.  With as many groups of
// workgroups as stay co-resident, the single-read kernel fills the GPU
// whatever the sample size and saves one read of x, so it is taken
// wherever it can run.
int ln_auto_variant(const float* x, const float* w, const float* b, const float* y, int64_t outer, int64_t inner)
{
    // in place the control-wave kernel does not run (a reader may need x
    // after its owner has overwritten it): the split schedule does
    if (!ln_single_supported(inner, x, w, b, y) || x == y) return 0;
    int64_t P = 0;
    int cap = 0;
    if (ln_wide_tile(outer, inner))
        single_grid<kLnWideF4, kLnWideWaves, kLnWideLag>(inner, P, cap);
    else
        single_grid<kLnTileF4, kLnTileWaves, kLnTileLag>(inner, P, cap);
    return cap >= P ? 1 : 0;
}

hipError_t launch_ln_single(const float* x, const float* w, const float* b, float* y, int64_t outer,
                            int64_t inner, float eps, void* ws, const LnLayout& lay, float* mean_out,
                            float* rstd_out, int protocol, hipStream_t st)
{
    char* base = static_cast<char*>(ws);
    LnCtrl* ctrl = reinterpret_cast<LnCtrl*>(base + lay.off_ctrl);
    uint32_t* counters = reinterpret_cast<uint32_t*>(base + lay.off_counter);
    f4* stats = reinterpret_cast<f4*>(base + lay.off_stats);
    double* lbdx = reinterpret_cast<double*>(base + lay.off_lbdx);
    double* xchg = reinterpret_cast<double*>(base + lay.off_xchg);
    double* lbd = reinterpret_cast<double*>(base + lay.off_lbd);

    // The single-read kernel, when a co-resident grid can hold every
    // sample's rows (on MI355X: samples of up to 256 x 4224 float4, about
    // 4.3M elements, with the wide tile).  Smaller tiles fit more workgroups
    // per CU but need as many more, so none would hold a larger sample.
    // (in place the tagged exchange does not run and variant 1 takes the split)
    if (ln_single_supported(inner, x, w, b, y) && !(protocol == 1 && x == y)) {
        hipError_t err = hipSuccess;
#define NORMFWD_TRY_SINGLE(F, DW, LG, PR, IL)                                                                 \
    try_launch_single<F, DW, LG, PR, IL>(x, w, b, y, outer, inner, eps, ctrl, counters, lbd, stats, lbdx, xchg,   \
                                         lay.P_cap, mean_out, rstd_out, st, err)
        const bool wide = ln_wide_tile(outer, inner);
        const bool launched =
            wide ? (protocol == 1 ? NORMFWD_TRY_SINGLE(kLnWideF4, kLnWideWaves, kLnWideLag, 0, true)
                                  : NORMFWD_TRY_SINGLE(kLnWideF4, kLnWideWaves, kLnWideLag, 1, true))
            : ln_tile_interleave(inner)
                ? (protocol == 1 ? NORMFWD_TRY_SINGLE(kLnTileF4, kLnTileWaves, kLnTileLag, 0, true)
                                 : NORMFWD_TRY_SINGLE(kLnTileF4, kLnTileWaves, kLnTileLag, 1, true))
                : (protocol == 1 ? NORMFWD_TRY_SINGLE(kLnTileF4, kLnTileWaves, kLnTileLag, 0, false)
                                 : NORMFWD_TRY_SINGLE(kLnTileF4, kLnTileWaves, kLnTileLag, 1, false));
#undef NORMFWD_TRY_SINGLE
        if (launched) return err;
    }
    // Shapes no single-read kernel can hold run the split schedule.
    hipError_t e = launch_ln_stats(x, outer, inner, eps, ws, lay, mean_out, rstd_out, st);
    if (e != hipSuccess) return e;
    return launch_ln_apply(x, w, b, y, outer, inner, ws, lay, st);
}

}  // namespace normfwd
