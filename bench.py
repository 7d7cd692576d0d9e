#!/usr/bin/env python3
"""Benchmark: achieved HBM GB/s and % of MI355X peak per norm kernel (one GPU).

Headline step: LayerNorm forward on x [16, 64, 256, 256] fp32 ~ N(0,1),
normalized over (64, 256, 256), elementwise weight/bias (LN page "Kimi-K2.6
l1_p40" problem).  One step = the whole LN path (moments, merge, normalize)
over one batch, with inputs resident in HBM; `value` = the bytes the step's
schedule has to move through HBM / wall time per step.  The headline
schedule is the fastest measured, the single-read kernel (--variant 1):
x read once + y written + weight and bias read once = 570,425,344 B, the
floor for any schedule.  The split schedule (--variant 0) reads x twice
(moments pass, then normalize pass): 838,860,800 B, so its GB/s is priced on
those bytes; `ms_per_step` compares schedules directly.  The split schedule
and the last-block-done kernel (--variant 2) are also timed in the `kernels`
object.

Also measured (the `kernels` object): GroupNorm+LeakyReLU+x2 [1024, 8192],
RMSNorm over dim 1 [112, 64, 512, 512], the LN N(100, 0.01) stress input,
both LN schedules, fc+GN [1024 x 8192 x 8192] (TFLOP/s), and, as references
for the HBM fractions, the library's plain copies of the same bytes (dense
256 MiB as for LN, dense 32 MiB over 32 rotating sets as for GN, the RMS
kernel's own access pattern) and torch's device copy of 256 MiB; each
norm kernel's `frac_of_copy` is its rate over its copy's.

Timing: an untimed settle phase (--settle-ms, default 200 ms of the same
work: on MI355X kernel durations settle only after ~100 ms of sustained load;
the LN step measured 104 us after 10 warm-up steps and 99 us after 100 ms), then
W untimed warm-up steps, then K timed steps bracketed by
torch.cuda.synchronize(); average launch durations from a pair of HIP events
recorded around the K launches on the stream the library launches on
(torch's current stream).  Kernel durations (the roofline's dominant kernel,
and `kernel_ms` in the per-kernel table) come from a second, identical loop
in which each timed launch stamps its own start and end into a pair of HIP
events (normfwd_time_next_kernel -> hipExtLaunchKernel), so no marker packet
sits between kernels.  Calls are validated and marshalled once before the
timed region (normalization_ln_forward_amd.prepare), so the host enqueues
faster than the GPU drains and the GPU never waits for Python.
Inputs rotate over several buffer sets (>= 2 GiB working set) so the 256 MB
Infinity Cache cannot hold a step's inputs from the previous step.
"""
import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E peak
PEAK_FP32_MATRIX_TFLOPS = 157.3  # MI355X dense fp32 MFMA peak
METRIC = "achieved HBM GB/s and % of MI355X peak per norm kernel (1 GPU)"

LN_SHAPE = (16, 64, 256, 256)
LN_BYTES = 4 * (2 * 16 * 4194304 + 2 * 4194304 + 16 * 4194304)       # 838,860,800: x twice (split)
LN_NORMALIZE_BYTES = 4 * (16 * 4194304 + 2 * 4194304 + 16 * 4194304)  # 570,425,344: x once


def ln_step_bytes(variant):
    """HBM bytes one LN step has to move under a schedule: the split reads x twice, the single-read
    kernels once."""
    return LN_BYTES if variant == 0 else LN_NORMALIZE_BYTES
GN_BYTES = 4 * (2 * 1024 * 8192 + 2 * 8192)                           # 67,174,400
RMS_BYTES = 4 * 2 * 112 * 64 * 512 * 512                              # 15,032,385,536
FC_FLOPS = 2 * 1024 * 8192 * 8192                                     # 137,438,953,472
FC_GN_BYTES = 4 * (1024 * 8192 + 8192 * 8192 + 8192 + 1024 * 8192)    # x, W, b, h write (GEMM part)

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_bench_workloads.json")


def traffic_for(kernel):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary (FETCH_SIZE + WRITE_SIZE, scaled by
    a plain copy of known size), or None if the summary is missing or the kernel's source changed since."""
    from normalization_ln_forward_amd import profiling

    try:
        with open(TRAFFIC_FILE) as f:
            entries = json.load(f)
    except (OSError, ValueError):
        return None
    e = entries.get(kernel)
    if not e or e.get("source_sha") != profiling.source_sha(profiling.KERNEL_SOURCES[kernel]):
        return None
    return e.get("hbm_bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--variant", type=int, default=1, choices=[0, 1, 2],
                    help="LN schedule for the headline: 1 = single kernel, control wave and tagged exchange "
                         "(default, fastest measured), 0 = split, 2 = single kernel, last workgroup merges")
    ap.add_argument("--rotate", type=int, default=4, help="LN buffer sets rotated through (>=1)")
    ap.add_argument("--no-kernels", action="store_true", help="skip the per-kernel table")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed run of each measured workload before its warm-up steps, in ms of wall time "
                         "(lets kernel durations reach their steady state; 0 = none)")
    ap.add_argument("--copy-ref", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of MIB MiB a few times (reference kernel for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes)")
    return ap.parse_args()


def main():
    args = parse()
    global SETTLE_MS
    SETTLE_MS = args.settle_ms
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the library has no multi-GPU path", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch

    import normalization_ln_forward_amd as nf
    from normalization_ln_forward_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nf.lib()
    variant = args.variant

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    # ------------------------------------------------------------ headline: LN
    log(f"[bench] LN {LN_SHAPE} variant={variant} rotate={args.rotate}")
    R = max(1, args.rotate)
    base = synth.make("ln_16x64x256x256", device=dev)
    xs = [base["x"]] + [synth.make("ln_16x64x256x256", device=dev, seed=2000 + i)["x"] for i in range(1, R)]
    ys = [torch.empty_like(base["x"]) for _ in range(R)]
    w, b = base["weight"], base["bias"]
    outer, inner = 16, 4194304
    _, ws = nf.alloc_workspace(nf.ln_forward_workspace_size(outer, inner), dev)
    nf.ln_forward_workspace_init(ws)
    stream = torch.cuda.current_stream(dev)
    # argument checking and marshalling happen once per buffer set, outside the timed region
    if variant != 0:
        steps = [nf.prepare(nf.ln_forward, xs[r], w, b, variant=variant, out=ys[r], workspace=ws) for r in range(R)]
        t = time_launches(torch, stream, lambda i: steps[i % R](), args.steps, args.warmup, nf=nf)
        ms_per_step = t["wall_ms"]
        # The single-read kernel moves x once, so its roofline is priced on the bytes it must move
        # (x + y + weight + bias).  Variant 1 is an ordinary launch that stamps the armed events itself
        # (kernel start to end); variant 2's cooperative launch cannot, so there the events bracket each
        # launch and its duration includes the cooperative launch's own cost.
        # (variant 2 runs ln_single_ctl_kernel with its last-workgroup-merges control wave at this shape)
        dom_kernel = "ln_single_ctl_kernel"
        dom_bytes, avg_ms, med_ms = LN_NORMALIZE_BYTES, t["kernel_ms"], t["kernel_ms_median"]
    else:
        # the step is the two halves of the split schedule
        stats = [nf.prepare(nf.ln_forward_stats, xs[r], workspace=ws) for r in range(R)]
        applies = [nf.prepare(nf.ln_forward_apply, xs[r], w, b, ws, out=ys[r]) for r in range(R)]
        evs, arms = kernel_events(torch, nf, stream, args.steps)

        def step(i):
            stats[i % R]()
            arms[i]()  # the normalize kernel stamps its own start and end into evs[i]
            applies[i % R]()

        def plain_step(i):
            stats[i % R]()
            applies[i % R]()

        # the timed steps carry no events at all; a second, identical loop times the normalize
        # kernel inside each step with events stamped by its own launch
        t = time_launches(torch, stream, plain_step, args.steps, args.warmup)
        ms_per_step = t["wall_ms"]
        time_launches(torch, stream, step, args.steps, 0, settle_ms=0)
        dom_kernel, dom_bytes = "ln_normalize_rows_kernel", LN_NORMALIZE_BYTES
        durs = sorted(a.elapsed_time(b_) for a, b_ in evs)
        avg_ms = sum(durs) / len(durs)
        med_ms = durs[len(durs) // 2]
    value = ln_step_bytes(variant) / (ms_per_step / 1e3) / 1e9
    achieved = dom_bytes / (avg_ms / 1e3) / 1e9
    roofline = {"bound": "hbm", "kernel": dom_kernel, "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": traffic_for(dom_kernel),
                "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_ms": round(avg_ms, 5),
                "median_launch_ms": round(med_ms, 5)}
    log(f"[bench] LN: {ms_per_step:.4f} ms/step wall, {value:.1f} GB/s; {dom_kernel} {avg_ms:.4f} ms, "
        f"{achieved:.1f} GB/s")
    del xs, ys
    torch.cuda.empty_cache()

    if args.copy_ref > 0:
        n = args.copy_ref * (1 << 20) // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy reference: 3 x {args.copy_ref} MiB")
        del src, dst
        torch.cuda.empty_cache()

    kernels = {}
    if not args.no_kernels:
        kernels = per_kernel_table(torch, nf, synth, dev, stream, args, log)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(base, args.cpu_seconds, log, ln_step_bytes(variant))

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "frac_of_peak": round(value / PEAK_HBM_GBS, 4),
        "config": {"workload": "ln_16x64x256x256", "shape": list(LN_SHAPE), "normalized_shape": [64, 256, 256],
                   "variant": ["split", "single", "single_last_block"][variant], "rotate_buffer_sets": R,
                   "algorithmic_bytes": ln_step_bytes(variant), "parallelism": "single-gpu"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "device": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(line), flush=True)
    # orderly teardown: every launch done, the library's cached workspaces released before the process
    # ends (device memory is not left to be freed during interpreter exit)
    torch.cuda.synchronize()
    nf.release_cached_workspaces()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def kernel_events(torch, nf, stream, n):
    """n pairs of timing events (each recorded once, so the HIP events exist) and, per pair, a prepared
    call that arms it for the library's next kernel launch (normfwd_time_next_kernel)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    return evs, [nf.prepare(nf.time_next_kernel, a, b) for a, b in evs]


SETTLE_MS = 200.0  # set from --settle-ms in main()


def settle(torch, fn, ms):
    """Run fn untimed, in growing batches, for `ms` milliseconds of wall time.  MI355X needs ~100 ms of
    sustained work before a kernel's duration settles (measured: the LN step at 104 us after 10 warm-up
    steps, 99 us after 100 ms), so every timed loop starts from that steady state."""
    if ms <= 0:
        return
    t0, n, i = time.perf_counter(), 1, 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(n):
            fn(i)
            i += 1
        torch.cuda.synchronize()
        n = min(2 * n, 4096)


def time_launches(torch, stream, fn, steps, warmup, nf=None, settle_ms=None):
    """Settle (see settle()), run fn(i) for i < warmup untimed, then `steps` times between two HIP
    events on `stream`, bracketed by synchronize() for the wall clock.
    Returns the average per launch from the events and from the wall clock;
    with nf, a second loop of `steps` launches, each stamping its kernel's
    own start and end into events, adds the average and the median kernel
    duration."""
    settle(torch, fn, SETTLE_MS if settle_ms is None else settle_ms)
    for i in range(warmup):
        fn(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    res = {"avg_ms": e0.elapsed_time(e1) / steps, "wall_ms": 1e3 * wall}
    if nf is not None:
        evs, arms = kernel_events(torch, nf, stream, steps)
        for i in range(steps):
            arms[i]()
            fn(i)
        torch.cuda.synchronize()
        durs = sorted(a.elapsed_time(b) for a, b in evs)
        res["kernel_ms"] = sum(durs) / steps
        res["kernel_ms_median"] = durs[steps // 2] if steps % 2 else 0.5 * (durs[steps // 2 - 1] + durs[steps // 2])
    return res


def _entry(t, nbytes=None, flops=None):
    """Throughput from the kernel's own duration where measured (kernel_ms), else launch to launch."""
    e = {k: round(v, 5) for k, v in t.items()}
    ms = t.get("kernel_ms", t["avg_ms"])
    if nbytes:
        gbs = nbytes / (ms / 1e3) / 1e9
        e.update({"algorithmic_bytes": nbytes, "GB/s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)})
    if flops:
        tf = flops / (ms / 1e3) / 1e12
        e.update({"flops": flops, "TFLOP/s": round(tf, 2), "frac_of_fp32_matrix_peak":
                  round(tf / PEAK_FP32_MATRIX_TFLOPS, 4)})
    return e


def per_kernel_table(torch, nf, synth, dev, stream, args, log):
    steps, warm = max(10, args.steps // 2), max(3, args.warmup // 2)
    out = {}

    # GroupNorm + LeakyReLU + x2: 64 MiB per set, rotate 32 sets (2 GiB)
    log("[bench] GN [1024, 8192]")
    g = synth.make("gn_lrelu_x2_1024x8192", device=dev)
    R = 32
    xs = [g["x"]] + [synth.make("gn_lrelu_x2_1024x8192", device=dev, seed=3000 + i)["x"] for i in range(1, R)]
    ys = [torch.empty_like(g["x"]) for _ in range(R)]
    calls = [nf.prepare(nf.gn_lrelu_x2_forward, xs[r], g["gamma"], g["beta"], 512, out=ys[r]) for r in range(R)]
    t = time_launches(torch, stream, lambda i: calls[i % R](), max(steps, 64), warm, nf)
    out["gn_lrelu_x2_1024x8192"] = _entry(t, GN_BYTES)
    del xs, ys
    torch.cuda.empty_cache()

    # LN, both schedules, N(0,1) and the N(100, 0.01) stress input
    # All schedules share the binding's workspace for this shape (as callers' calls do); after each timed
    # loop the last output is compared bit for bit with the same schedule run on a freshly zeroed
    # workspace (`bitwise_vs_fresh_workspace`).
    for name in ("ln_16x64x256x256", "ln_stress_16x64x256x256"):
        d = synth.make(name, device=dev)
        y = torch.empty_like(d["x"])
        x2 = synth.make(name, device=dev, seed=4000)["x"]
        y2 = torch.empty_like(d["x"])
        _, fresh_ws = nf.alloc_workspace(nf.ln_forward_workspace_size(16, 4194304), dev)
        for variant in (0, 1, 2):
            log(f"[bench] {name} variant={variant}")
            calls = [nf.prepare(nf.ln_forward, xx, d["weight"], d["bias"], variant=variant, out=yy)
                     for xx, yy in ((d["x"], y), (x2, y2))]
            t = time_launches(torch, stream, lambda i: calls[i % 2](), steps, warm)
            same = True
            for xx, yy in ((d["x"], y), (x2, y2)):  # both outputs were last written by this schedule
                nf.ln_forward_workspace_init(fresh_ws)
                again = nf.ln_forward(xx, d["weight"], d["bias"], variant=variant, workspace=fresh_ws)
                same = same and bool(torch.equal(again, yy))
                del again
            e = _entry(t, ln_step_bytes(variant))
            e["bitwise_vs_fresh_workspace"] = same
            out[f"{name}/{['split', 'single', 'single_last_block'][variant]}"] = e
        del d, y, x2, y2, fresh_ws
        torch.cuda.empty_cache()

    # Copy references (the library's hand-written copies, normfwd_copy_reference): what a plain copy of
    # each workload's bytes reaches in this run, set beside the kernels as frac_of_copy.
    #   256 MiB -> 256 MiB, 4 rotating pairs (2 GiB), as the LN input: the LN reference
    #   32 MiB -> 32 MiB, 32 rotating pairs (2 GiB), as the GN input: the GN reference
    # and torch's own device copy of 256 MiB for comparison.
    for mib, sets, name in ((256, 4, "copy_dense_256MiB"), (32, 32, "copy_dense_32MiB")):
        log(f"[bench] copy reference: {mib} MiB, {sets} sets")
        n = (mib << 20) // 4
        srcs = [torch.randn(n, device=dev) for _ in range(sets)]
        dsts = [torch.empty_like(t) for t in srcs]
        calls = [nf.prepare(nf.copy_reference, srcs[r], dsts[r]) for r in range(sets)]
        t = time_launches(torch, stream, lambda i: calls[i % sets](), max(steps, 64) if mib == 32 else steps, warm,
                          nf)
        out[name] = _entry(t, 2 * 4 * n)
        if mib == 256:
            t = time_launches(torch, stream, lambda i: dsts[i % 4].copy_(srcs[i % 4]), steps, warm)
            out["copy_reference_torch_256MiB"] = _entry(t, 2 * 4 * n)
        del srcs, dsts, calls
        torch.cuda.empty_cache()

    # RMSNorm over dim 1: 7.5 GB in, 7.5 GB out (far beyond any cache)
    log("[bench] RMS [112, 64, 512, 512]")
    r = synth.make("rms_ch_112x64x512x512", device=dev)
    y = torch.empty_like(r["x"])
    call = nf.prepare(nf.rmsnorm_ch_forward, r["x"], out=y)
    t = time_launches(torch, stream, lambda i: call(), max(5, steps // 4), 2, nf)
    out["rms_ch_112x64x512x512"] = _entry(t, RMS_BYTES)
    # the same access pattern as a plain copy (the RMS reference)
    log("[bench] copy reference: RMS access pattern")
    call = nf.prepare(nf.copy_reference, r["x"], y, pattern=1)
    t = time_launches(torch, stream, lambda i: call(), max(5, steps // 4), 2, nf)
    out["copy_rms_pattern_112x64x512x512"] = _entry(t, RMS_BYTES)
    del r, y, call
    torch.cuda.empty_cache()

    # fc + GN
    log("[bench] fc+GN [1024 x 8192 x 8192]")
    f = synth.make("fc_gn_1024x8192x8192", device=dev)
    y = torch.empty(1024, 8192, device=dev)
    call = nf.prepare(nf.fc_gn_forward, f["x"], f["W"], f["b"], f["gamma"], f["beta"], 512, out=y)
    t = time_launches(torch, stream, lambda i: call(), max(5, steps // 4), 2, nf)
    out["fc_gn_1024x8192x8192"] = _entry(t, flops=FC_FLOPS)
    del f, y
    torch.cuda.empty_cache()
    # each kernel's GB/s as a fraction of the copy of its own bytes in this run
    for k, ref in (("gn_lrelu_x2_1024x8192", "copy_dense_32MiB"), ("ln_16x64x256x256/single", "copy_dense_256MiB"),
                   ("ln_stress_16x64x256x256/single", "copy_dense_256MiB"),
                   ("rms_ch_112x64x512x512", "copy_rms_pattern_112x64x512x512")):
        if k in out and ref in out:
            out[k]["frac_of_copy"] = round(out[k]["GB/s"] / out[ref]["GB/s"], 4)
    return out


def cpu_baseline(base, seconds, log, nbytes):
    """The fp64 oracle on the host cores, on the same LN workload, repeated for ~`seconds`.  Only the
    oracle's computation is timed: the inputs are promoted to fp64 and the output allocated once, before
    the timed loop."""
    import numpy as np

    import oracle

    x = np.ascontiguousarray(base["x"].cpu().numpy(), dtype=np.float64)
    w = np.ascontiguousarray(base["weight"].cpu().numpy(), dtype=np.float64)
    b = np.ascontiguousarray(base["bias"].cpu().numpy(), dtype=np.float64)
    y = np.empty_like(x)
    oracle.ln(x, w, b, eps=1e-5, out=y)  # first call: loads the library and touches y's pages
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.ln(x, w, b, eps=1e-5, out=y)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 2000:
            break
    per = el / reps
    log(f"[bench] oracle LN: {per:.3f} s per full workload ({reps} reps, {oracle.num_threads()} threads)")
    # priced on the same bytes as the headline value, so the two rates compare as times
    return {"value": round(nbytes / per / 1e9, 3), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds_per_step": round(per, 4),
            "sample": f"full ln_16x64x256x256 workload (16 samples x 4,194,304), {reps} repetitions, fp64 two-pass, "
                      "computation only (inputs promoted and output allocated before timing)",
            "host_cpu": platform.processor() or platform.machine(), "host_logical_cpus": os.cpu_count()}


if __name__ == "__main__":
    main()
