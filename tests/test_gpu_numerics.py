"""Numerics edge cases of the GPU path against the fp64 oracle, through the C ABI.

* LayerNorm on N(100, 0.01) data whose first element (and the first element of other workgroups' and
  waves' shares) is an outlier: the statistics must not depend on which element a kernel happens to read
  first (LN page "Kimi-K2.6 l1_p40", turn 2 warns of catastrophic cancellation in one-pass moments).
* GroupNorm and fc + GroupNorm on groups far from 0 (N(100, 0.01), N(10, 0.01), a large fc bias; GN page
  "Kimi-K2.6 l2_p62", turn 1 discusses the one-pass variance and its clamp).
* The single-read LayerNorm kernel's exchange: words the other schedules leave in the shared slots are
  never taken for this launch's (planted from the host under every generation value), and schedules that
  alternate on one workspace past the tag cycle keep their results bit for bit.

Pass rule as everywhere: |g - o| <= 1e-4 + 1e-4 |o| (rtol 2e-3 for fc), g finite.
"""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
from normalization_ln_forward_amd import _lib, synth
import normalization_ln_forward_amd as nf

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _np(t):
    return t.detach().cpu().numpy()


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.lib()
    yield
    torch.cuda.synchronize()


def _close(got, ref, rtol=1e-4, what=""):
    rep = oracle.allclose_report(got, ref, 1e-4, rtol)
    assert rep["ok"], f"{what}: {rep}"
    return rep


# ---------------------------------------------------------------- LayerNorm, outlier first elements

def _plant_outliers(x, value):
    """x [outer, inner] on N(100, 0.01): set the first element of every sample, of several 2048-element
    blocks (a single-read workgroup's first row), of 256-element blocks (a wave's first float4 row) and
    of 1024-element blocks (a split-schedule row) to `value`."""
    inner = x.shape[1]
    pos = {0, 256, 1024, 2048, 2048 + 256 * 3, 7 * 2048, 100 * 2048 + 256 * 5, 1024 * 37, inner - 1}
    for p in sorted(q for q in pos if q < inner):
        x[:, p] = value
    return x


LN_OUTLIER_SHAPES = [(16, 4194304), (3, 300000), (1, 1 << 22), (64, 4096), (33, 2047)]


@pytest.mark.parametrize("value", [0.0, 90.0])
@pytest.mark.parametrize("shape", LN_OUTLIER_SHAPES)
@pytest.mark.parametrize("variant", [0, 1, 2, 3])
def test_ln_outlier_first_elements(variant, shape, value):
    """Every schedule (split, single-read control wave, last workgroup merges, automatic; samples of up to
    8192 elements take the one-workgroup kernel under every variant) on N(100, 0.01) samples whose first
    element, and the first elements of other workgroups' and waves' shares, are outliers."""
    _say(f"ln outliers variant={variant} shape={shape} value={value}")
    outer, inner = shape
    d = synth.make("ln_stress_16x64x256x256", device="cuda", shape=shape, normalized_ndim=1, seed=outer + inner)
    x = _plant_outliers(d["x"], value)
    mean = torch.empty(outer, device="cuda")
    rstd = torch.empty(outer, device="cuda")
    y = nf.ln_forward(x, d["weight"], d["bias"], variant=variant, mean_out=mean, rstd_out=rstd)
    ref, om, ov = oracle.ln(_np(x), _np(d["weight"]), _np(d["bias"]), return_stats=True)
    rep = _close(_np(y), ref, what=f"ln outliers {shape} v{variant} {value}")
    _say(f"  max_abs={rep['max_abs']:.3e}")
    np.testing.assert_allclose(_np(mean), om, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(_np(rstd), 1.0 / np.sqrt(ov + np.float32(1e-5)), rtol=1e-5)
    del d, x, y
    torch.cuda.empty_cache()


def test_ln_in_place_default_variant_on_outliers():
    """In place, the default variant runs the split schedule (the single-read kernel keeps x intact until
    its end and does not run in place); the result still follows the oracle and equals variant 0's."""
    _say("ln in place, outliers")
    d = synth.make("ln_stress_16x64x256x256", device="cuda", shape=(4, 1 << 20), normalized_ndim=1, seed=5)
    x = _plant_outliers(d["x"], 0.0)
    ref = oracle.ln(_np(x), _np(d["weight"]), _np(d["bias"]))
    split = nf.ln_forward(x, d["weight"], d["bias"], variant=0)
    for variant in (3, 1):
        xi = x.clone()
        nf.ln_forward(xi, d["weight"], d["bias"], variant=variant, out=xi)
        assert torch.equal(xi, split), variant
    _close(_np(split), ref, what="ln in place")


# ---------------------------------------------------------------- GroupNorm away from 0

GN_SHIFT_CASES = [
    # (N, C, G, misalign): the fast kernel with 1, 2, 4, 32 lanes per group, the lane and wave kernels
    (64, 8192, 512, False),   # M = 16 (the GN page's problem)
    (16, 4096, 1024, False),  # M = 4
    (16, 4096, 512, False),   # M = 8
    (16, 8192, 64, False),    # M = 128
    (16, 35, 7, False),       # M = 5: lane kernel
    (8, 3000, 30, False),     # M = 100: wave kernel
    (4, 8192, 16, False),     # M = 512: wave kernel
    (8, 4096, 256, True),     # misaligned: lane kernel with M = 16
]


@pytest.mark.parametrize("mean,std", [(100.0, 0.01), (10.0, 0.01)])
@pytest.mark.parametrize("N,C,G,misalign", GN_SHIFT_CASES)
def test_gn_groups_far_from_zero(N, C, G, misalign, mean, std):
    _say(f"gn shifted N={N} C={C} G={G} misalign={misalign} N({mean}, {std})")
    d = synth.make("gn_lrelu_x2_1024x8192", device="cuda", shape=(N, C), seed=N + C + G,
                   x_dist=("normal", mean, std))
    x = d["x"]
    x[:, ::37] += 0.5  # a few channels off the group's bulk, some of them a group's first
    if misalign:
        buf = torch.empty(N * C + 1, device="cuda")
        buf[1:].copy_(x.reshape(-1))
        x = buf[1:].view(N, C)
    y = nf.gn_lrelu_x2_forward(x, d["gamma"], d["beta"], G)
    ref = oracle.gn_lrelu_x2(_np(x), _np(d["gamma"]), _np(d["beta"]), G)
    rep = _close(_np(y), ref, what="gn shifted")
    _say(f"  max_abs={rep['max_abs']:.3e}")


FC_BIAS_CASES = [
    # (N, K, C, G, w_scale): fused epilogues (4, 8, 16, 32, 64 channels per group; both GEMM kernels) with
    # a bias of ~100 and weights scaled so the groups spread ~0.006 around it; unfused group sizes (the
    # GEMM writes h in fp32, whose rounding at 100 is inherent) with the unscaled spread of ~0.6
    (64, 256, 512, 32, 0.01),   # M = 16, direct-to-LDS GEMM
    (64, 256, 512, 128, 0.01),  # M = 4
    (64, 256, 512, 64, 0.01),   # M = 8
    (64, 256, 512, 16, 0.01),   # M = 32
    (64, 256, 512, 8, 0.01),    # M = 64
    (70, 70, 256, 16, 0.01),    # M = 16, staged GEMM (K % 4 != 0)
    (50, 64, 100, 5, 1.0),      # M = 20: h, then the GroupNorm kernel
]


@pytest.mark.parametrize("N,K,C,G,w_scale", FC_BIAS_CASES)
def test_fc_gn_large_bias(N, K, C, G, w_scale):
    _say(f"fc large bias N={N} K={K} C={C} G={G} w_scale={w_scale}")
    d = synth.make("fc_gn_1024x8192x8192", device="cuda", shape=(N, K), hidden=C, seed=N + K + C + G)
    W = d["W"] * w_scale
    b = d["b"] + 100.0
    y = nf.fc_gn_forward(d["x"], W, b, d["gamma"], d["beta"], G)
    ref = oracle.fc_gn_lrelu_x2(_np(d["x"]), _np(W), _np(b), _np(d["gamma"]), _np(d["beta"]), G)
    rep = _close(_np(y), ref, rtol=2e-3, what="fc large bias")
    _say(f"  max_abs={rep['max_abs']:.3e}")


# ---------------------------------------------------------------- single-read LayerNorm exchange slots

def _ctrl(ws):
    """(gen, done, error, recomputed, gen_ctl) words of an LN workspace's control block."""
    return ws[:20].view(torch.int32).cpu().tolist()


def test_ln_planted_partials_are_never_taken():
    """A child process with NORMFWD_LN_FORCE_RECOMPUTE=4 (every 4th workgroup of the single-read kernel
    publishes nothing) plants split-schedule partials in every exchange slot (a variant-0 call on the same
    workspace), sets the control-wave generation to values across its range (and beyond, as an unzeroed
    workspace could hold), then runs variant 1: the silent workgroups' slots hold only the planted words,
    which no generation accepts, so the readers compute those moments from x and every output equals this
    process's normal variant-1 output bit for bit."""
    path = os.path.join(os.environ.get("TMPDIR", "/tmp"), f"planted_{os.getpid()}.npz")
    env = dict(os.environ, NORMFWD_LN_FORCE_RECOMPUTE="4")
    _say("planted partials: child")
    r = subprocess.run([sys.executable, os.path.join(HERE, "planted_child.py"), path], capture_output=True,
                       text=True, timeout=300, env=env)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    got = np.load(path)
    os.remove(path)
    sys.path.insert(0, HERE)
    import planted_child

    d = planted_child.inputs()
    normal = nf.ln_forward(d["x"], d["weight"], d["bias"], variant=1)
    ref = oracle.ln(_np(d["x"]), _np(d["weight"]), _np(d["bias"]))
    normal_np = _np(normal)
    for g in planted_child.GENERATIONS:
        y = got[f"y_{g}"]
        assert np.array_equal(y.view(np.uint32), normal_np.view(np.uint32)), f"generation {g}: differs"
    assert int(got["recomputed"]) > 0
    _close(normal_np, ref, what="planted")


def test_ln_variants_alternating_on_one_workspace_past_the_tag_cycle():
    """600 calls on one workspace alternating the split (which overwrites the exchange slots with its own
    partials) and the single-read kernel, with a last-workgroup-merges call every fifth: each schedule's
    output stays bitwise equal to its first, nothing is recomputed, and the control-wave generation
    counts the single-read launches mod 255."""
    _say("ln alternating variants")
    shape = (4, 1 << 19)
    d = synth.make("ln_stress_16x64x256x256", device="cuda", shape=shape, normalized_ndim=1, seed=17)
    x = _plant_outliers(d["x"], 90.0)
    _, ws = nf.alloc_workspace(nf.ln_forward_workspace_size(*shape), "cuda")
    nf.ln_forward_workspace_init(ws)
    first = {}
    n1 = 0
    for i in range(600):
        v = 2 if i % 5 == 4 else (1 if i % 2 else 0)
        y = nf.ln_forward(x, d["weight"], d["bias"], variant=v, workspace=ws)
        n1 += v == 1
        if v not in first:
            first[v] = y
        elif not torch.equal(y, first[v]):
            pytest.fail(f"call {i} (variant {v}) differs from that variant's first result")
    torch.cuda.synchronize()
    gen, done, err, recomputed, gen_ctl = _ctrl(ws)
    assert done == 0 and err == 0 and recomputed == 0, (gen, done, err, recomputed, gen_ctl)
    assert gen_ctl == n1 % 255, (gen_ctl, n1)
    ref = oracle.ln(_np(x), _np(d["weight"]), _np(d["bias"]))
    for v, y in first.items():
        _close(_np(y), ref, what=f"variant {v}")


# the last-workgroup-merges kernel's arrival counters: int32 index of the first (right after the 256-byte
# control block) and words between them (one per 128-byte line, eight of them)
COUNTER_RING_WORD = 64
COUNTER_STRIDE_WORDS = 32
COUNTER_RING = 8


@pytest.mark.parametrize("shape", [(12, 1 << 19), (16, 4000000)])
def test_ln_last_block_election_survives_leftover_counts(shape):
    """Variant 2 elects as a sample's merger the arrival that finds P - 1 modulo P before it, and the merger
    takes P back off the counter, so counts left in the ring (a launch that gave up on a wait stops counting
    halfway) move no election: with counts planted from the host the output stays bitwise equal to a clean
    run's and no wait gives up.  Shapes: 32 workgroups per sample with the 8 x 8 tile (arrivals counted one
    sample ahead), and 237 with the wide tile (two ahead), whose 16 samples take each counter twice."""
    _say(f"ln last-block election with planted counts shape={shape}")
    d = synth.make("ln_16x64x256x256", device="cuda", shape=shape, normalized_ndim=1, seed=29)
    _, ws = nf.alloc_workspace(nf.ln_forward_workspace_size(*shape), "cuda")
    nf.ln_forward_workspace_init(ws)
    clean = nf.ln_forward(d["x"], d["weight"], d["bias"], variant=2, workspace=ws)
    words = ws.view(torch.int32)
    for planted in ([1, 31, 5, 100, 2, 63, 17, 4], [(1 << 20) + 3, 7, 0, 236, 1, 235, 64, 3], [9] * COUNTER_RING):
        for k, v in enumerate(planted):
            words[COUNTER_RING_WORD + k * COUNTER_STRIDE_WORDS] = v
        y = nf.ln_forward(d["x"], d["weight"], d["bias"], variant=2, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y, clean), planted
        left = [int(words[COUNTER_RING_WORD + k * COUNTER_STRIDE_WORDS]) for k in range(COUNTER_RING)]
        assert left == planted, (planted, left)  # every sample's arrivals and its merger's subtraction cancel
        nf.ln_forward_workspace_check(ws)
    ref = oracle.ln(_np(d["x"]), _np(d["weight"]), _np(d["bias"]))
    _close(_np(clean), ref, what=f"variant 2 {shape}")


def test_ln_last_block_past_the_tag_cycle():
    """300 consecutive variant-2 calls on one workspace, past the 255-launch cycle of the generation tags
    that its partials and statistics words carry: every output equals the first bit for bit, no wait
    gives up, and the completion counter is back at zero."""
    _say("ln last-block 300 calls")
    shape = (6, 1 << 19)
    d = synth.make("ln_stress_16x64x256x256", device="cuda", shape=shape, normalized_ndim=1, seed=31)
    _, ws = nf.alloc_workspace(nf.ln_forward_workspace_size(*shape), "cuda")
    nf.ln_forward_workspace_init(ws)
    first = nf.ln_forward(d["x"], d["weight"], d["bias"], variant=2, workspace=ws)
    for i in range(1, 300):
        y = nf.ln_forward(d["x"], d["weight"], d["bias"], variant=2, workspace=ws)
        if not torch.equal(y, first):
            pytest.fail(f"call {i} differs from the first")
    torch.cuda.synchronize()
    gen, done, err, recomputed, gen_ctl = _ctrl(ws)
    assert done == 0 and err == 0 and gen == 300, (gen, done, err)
    _close(_np(first), oracle.ln(_np(d["x"]), _np(d["weight"]), _np(d["bias"])), what="variant 2, 300 calls")
