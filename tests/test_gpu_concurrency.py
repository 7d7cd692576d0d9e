"""The single-read LayerNorm kernel (an ordinary launch whose workgroups exchange moments: variant 1, every
workgroup merging every sample, and variant 2, the last to arrive merging it) next to other work on a
second stream: every result equals its solo result bit for bit, and a short kernel alongside does not
stall it (its waits are bounded; a missing workgroup's moments are computed by the readers).
Durations are medians of several repetitions, each taken with events on the LayerNorm's own stream."""
import sys

import pytest
import torch

from normalization_ln_forward_amd import _lib, synth
import normalization_ln_forward_amd as nf

pytestmark = pytest.mark.gpu

SHAPE = (16, 1 << 22)
REPS = 8
VARIANTS = (1, 2)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.lib()
    dev = torch.device("cuda:0")
    d = synth.make("ln_16x64x256x256", device=dev, shape=SHAPE, normalized_ndim=1)
    ws = []
    for _ in range(2):
        _, w = nf.alloc_workspace(nf.ln_forward_workspace_size(*SHAPE), dev)
        nf.ln_forward_workspace_init(w)
        ws.append(w)
    refs = {v: nf.ln_forward(d["x"], d["weight"], d["bias"], variant=v) for v in VARIANTS}
    torch.cuda.synchronize()
    yield dev, d, ws, refs
    torch.cuda.synchronize()


def _timed(fn, stream):
    a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        a.record(stream)
        fn()
        e.record(stream)
    return a, e


def _median(xs):
    return sorted(xs)[len(xs) // 2]


def _solo_ms(fn, stream):
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(REPS):
        a, e = _timed(fn, stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(e))
    return _median(ts)


def _concurrent(other, ln, s_other, s_ln, check):
    """`other` enqueued on s_other, then `ln` at once on s_ln; per repetition the LN duration (from its
    enqueue on its stream to its end) and the other's; `check()` after each repetition (it refills the
    outputs on the current stream, so the device is synchronized before the next repetition)."""
    tl, to = [], []
    for _ in range(REPS):
        b0, b1 = _timed(other, s_other)
        a0, a1 = _timed(ln, s_ln)
        torch.cuda.synchronize()
        tl.append(a0.elapsed_time(a1))
        to.append(b0.elapsed_time(b1))
        check()
        torch.cuda.synchronize()
    return _median(tl), _median(to)


@pytest.mark.parametrize("variant", VARIANTS)
def test_ln_beside_a_short_kernel(setup, variant):
    """GroupNorm [1024, 8192] (~12 us) on one stream, the LayerNorm [16, 4M] right after on another: both
    results bitwise equal to their solo results; the LayerNorm takes under 2x its solo time."""
    dev, d, ws, refs = setup
    ref = refs[variant]
    g = synth.make("gn_lrelu_x2_1024x8192", device=dev)
    g_ref = nf.gn_lrelu_x2_forward(g["x"], g["gamma"], g["beta"], 512)
    gy, y = torch.empty_like(g_ref), torch.empty_like(ref)
    s_ln, s_other = torch.cuda.Stream(), torch.cuda.Stream()
    ln = lambda: nf.ln_forward(d["x"], d["weight"], d["bias"], variant=variant, out=y, workspace=ws[0])  # noqa: E731
    other = lambda: nf.gn_lrelu_x2_forward(g["x"], g["gamma"], g["beta"], 512, out=gy)  # noqa: E731
    solo = _solo_ms(ln, s_ln)

    def check():
        assert torch.equal(y, ref), "LayerNorm beside GroupNorm differs from its solo result"
        assert torch.equal(gy, g_ref)
        y.fill_(float("nan"))

    t_ln, t_other = _concurrent(other, ln, s_other, s_ln, check)
    _say(f"v{variant}: solo LN {solo * 1e3:.1f} us; beside GN: LN {t_ln * 1e3:.1f} us, "
         f"GN {t_other * 1e3:.1f} us")
    assert t_ln < 2.0 * solo, (t_ln, solo)


@pytest.mark.parametrize("variant", VARIANTS)
def test_ln_beside_a_streaming_kernel(setup, variant):
    """RMSNorm [4, 64, 512, 512] (~100 us, HBM-bound like the LayerNorm) alongside: both bitwise equal to
    their solo results; the two share HBM, so the LayerNorm takes at most about the time of both."""
    dev, d, ws, refs = setup
    ref = refs[variant]
    r = synth.make("rms_ch_112x64x512x512", device=dev, shape=(4, 64, 512, 512))
    r_ref = nf.rmsnorm_ch_forward(r["x"])
    ry, y = torch.empty_like(r_ref), torch.empty_like(ref)
    s_ln, s_other = torch.cuda.Stream(), torch.cuda.Stream()
    ln = lambda: nf.ln_forward(d["x"], d["weight"], d["bias"], variant=variant, out=y, workspace=ws[0])  # noqa: E731
    other = lambda: nf.rmsnorm_ch_forward(r["x"], out=ry)  # noqa: E731
    solo_ln, solo_other = _solo_ms(ln, s_ln), _solo_ms(other, s_other)

    def check():
        assert torch.equal(y, ref), "LayerNorm beside RMSNorm differs from its solo result"
        assert torch.equal(ry, r_ref)
        y.fill_(float("nan"))

    t_ln, t_other = _concurrent(other, ln, s_other, s_ln, check)
    _say(f"v{variant}: solo LN {solo_ln * 1e3:.1f} us, RMS {solo_other * 1e3:.1f} us; "
         f"together: LN {t_ln * 1e3:.1f} us, RMS {t_other * 1e3:.1f} us")
    assert t_ln < 1.5 * (solo_ln + solo_other), (t_ln, solo_ln, solo_other)


@pytest.mark.parametrize("variant", VARIANTS)
def test_two_ln_calls_on_two_streams(setup, variant):
    """Two single-read LayerNorm calls on two streams (separate workspaces) at once: both equal the solo
    result bit for bit and finish within twice the time of the two run one after the other."""
    dev, d, ws, refs = setup
    ref = refs[variant]
    x2 = d["x"].clone()
    y1, y2 = torch.empty_like(ref), torch.empty_like(ref)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    a = lambda: nf.ln_forward(d["x"], d["weight"], d["bias"], variant=variant, out=y1, workspace=ws[0])  # noqa: E731
    b = lambda: nf.ln_forward(x2, d["weight"], d["bias"], variant=variant, out=y2, workspace=ws[1])  # noqa: E731
    solo = _solo_ms(a, s1)

    def check():
        assert torch.equal(y1, ref) and torch.equal(y2, ref), "concurrent LayerNorm calls differ from solo"
        y1.fill_(float("nan"))
        y2.fill_(float("nan"))

    t1, t2 = _concurrent(b, a, s2, s1, check)
    _say(f"v{variant}: solo LN {solo * 1e3:.1f} us; two at once: {t1 * 1e3:.1f} / {t2 * 1e3:.1f} us")
    assert max(t1, t2) < 4.0 * solo, (t1, t2, solo)
