"""GPU parity: the HIP library (through its C ABI) against the fp64 CPU oracle.

Pass rule, elementwise: |g - o| <= atol + rtol*|o| with g finite, where o is
the oracle's unrounded fp64 value.  atol = rtol = 1e-4 for the three norms,
rtol = 2e-3 for the fc path (fp32 accumulation over K = 8192 products).
Inputs come from the shared seeded generators (normalization_ln_forward_amd.synth)
with the workloads' distributions; small cases span several tiles and ragged
tails, full-size cases use the workloads' own shapes.
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from normalization_ln_forward_amd import _lib, synth
import normalization_ln_forward_amd as nf

pytestmark = pytest.mark.gpu

ATOL = 1e-4
RTOL = 1e-4
RTOL_FC = 2e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.lib()  # fail loudly if the library is missing
    yield
    torch.cuda.synchronize()


def _assert_close(got, ref, atol=ATOL, rtol=RTOL, what=""):
    rep = oracle.allclose_report(got, ref, atol, rtol)
    assert rep["ok"], f"{what}: {rep}"
    return rep


def _np(t):
    return t.detach().cpu().numpy()


# ---------------------------------------------------------------- GroupNorm + LeakyReLU + x2

GN_CASES = [
    # (N, C, G, affine, misalign)  -> path
    (5, 8192, 512, True, False),     # fast path, M=16, several tiles per row
    (3, 1000, 125, True, False),     # fast, M=8, ragged last tile (C/4 = 250)
    (7, 48, 3, True, False),         # fast, M=16, tile shorter than a wave
    (4, 256, 64, True, False),       # fast, M=4 (one lane per group)
    (2, 1024, 4, True, False),       # fast, M=256 (64 lanes per group)
    (3, 8192, 16, True, False),      # generic wave kernel, M=512
    (6, 35, 7, True, False),         # generic lane kernel, M=5
    (2, 300, 3, True, False),        # generic wave kernel, M=100
    (4, 24, 24, True, False),        # M=1: output is 2*lrelu(beta)
    (5, 8192, 512, False, False),    # no affine
    (5, 4096, 256, True, True),      # misaligned base pointer -> generic path
]


@pytest.mark.parametrize("N,C,G,affine,misalign", GN_CASES)
def test_gn_parity(N, C, G, affine, misalign):
    _say(f"gn N={N} C={C} G={G} affine={affine} misalign={misalign}")
    d = synth.make("gn_lrelu_x2_1024x8192", device="cuda", shape=(N, C), seed=7 + N + C)
    x = d["x"]
    if misalign:
        buf = torch.empty(N * C + 1, device="cuda")
        buf[1:].copy_(x.reshape(-1))
        x = buf[1:].view(N, C)
    gamma = d["gamma"] if affine else None
    beta = d["beta"] if affine else None
    y = nf.gn_lrelu_x2_forward(x, gamma, beta, G, eps=1e-5, negative_slope=0.01)
    ref = oracle.gn_lrelu_x2(_np(x), None if gamma is None else _np(gamma), None if beta is None else _np(beta),
                             G, eps=1e-5, negative_slope=0.01)
    _assert_close(_np(y), ref, what="gn")


def test_gn_full_size_and_determinism():
    _say("gn full 1024x8192 G=512")
    d = synth.make("gn_lrelu_x2_1024x8192", device="cuda")
    y1 = nf.gn_lrelu_x2_forward(d["x"], d["gamma"], d["beta"], 512)
    y2 = nf.gn_lrelu_x2_forward(d["x"], d["gamma"], d["beta"], 512)
    ref = oracle.gn_lrelu_x2(_np(d["x"]), _np(d["gamma"]), _np(d["beta"]), 512)
    rep = _assert_close(_np(y1), ref, what="gn full")
    _say(f"  max_abs={rep['max_abs']:.3e} max_rel={rep['max_rel']:.3e}")
    assert torch.equal(y1, y2)


def test_gn_in_place():
    _say("gn in place")
    d = synth.make("gn_lrelu_x2_1024x8192", device="cuda", shape=(64, 8192), seed=11)
    ref = oracle.gn_lrelu_x2(_np(d["x"]), _np(d["gamma"]), _np(d["beta"]), 512)
    x = d["x"].clone()
    nf.gn_lrelu_x2_forward(x, d["gamma"], d["beta"], 512, out=x)
    _assert_close(_np(x), ref, what="gn in place")


# ---------------------------------------------------------------- RMSNorm over dim 1

RMS_CASES = [
    # shape, misalign
    ((3, 64, 1000), False),          # 128-bit path, ragged tile
    ((3, 64, 1001), False),          # scalar path (S % 4 != 0)
    ((2, 1, 512), False),            # C = 1
    ((2, 3, 256), False),            # C < channels per wave
    ((2, 100, 260), False),          # 7 waves, last one partial
    ((2, 300, 64), False),           # 32 channels per wave
    ((2, 600, 64), False),           # streaming kernel (C > 512)
    ((4, 64, 32, 32), False),        # 4-D input
    ((2, 64, 1024), True),           # misaligned -> scalar path
]


@pytest.mark.parametrize("shape,misalign", RMS_CASES)
def test_rms_parity(shape, misalign):
    _say(f"rms shape={shape} misalign={misalign}")
    d = synth.make("rms_ch_112x64x512x512", device="cuda", shape=shape, seed=sum(shape))
    x = d["x"]
    if misalign:
        buf = torch.empty(x.numel() + 1, device="cuda")
        buf[1:].copy_(x.reshape(-1))
        x = buf[1:].view(shape)
    y = nf.rmsnorm_ch_forward(x, eps=1e-5)
    ref = oracle.rms_ch(_np(x), eps=1e-5)
    _assert_close(_np(y), ref, what="rms")


def test_rms_in_place():
    _say("rms in place")
    d = synth.make("rms_ch_112x64x512x512", device="cuda", shape=(2, 64, 4096), seed=5)
    ref = oracle.rms_ch(_np(d["x"]))
    x = d["x"].clone()
    nf.rmsnorm_ch_forward(x, out=x)
    _assert_close(_np(x), ref, what="rms in place")


# ---------------------------------------------------------------- LayerNorm

LN_CASES = [
    # (outer, inner, affine, variant)
    (3, 5000, True, 0),
    (3, 5000, True, 1),
    (2, 40000, True, 0),             # 3 chunks, ragged last
    (2, 40000, True, 1),
    (4, 40001, True, 0),             # scalar path (inner % 4 != 0)
    (4, 40001, True, 1),
    (5, 1, True, 0),                 # one element per sample: y = bias
    (5, 1, True, 1),
    (3, 300000, False, 0),           # no affine
    (3, 300000, False, 1),
    (1, 1 << 20, True, 1),           # one sample, many workgroups
    (2, 40000, True, 2),             # single kernel, last workgroup merges
    (4, 40001, True, 2),
    (3, 300000, False, 2),
    (1, 1 << 20, True, 2),
    # the wide single-read tile (11 data waves x 6 float4): 8 samples that fill 237 workgroups (ragged
    # last row), and a sample of 1,081,344 float4 that only the wide tile's 256 workgroups hold
    (8, 4000000, True, 1),
    (8, 4000000, True, 2),
    (2, 4325376, True, 1),
    (2, 4325376, True, 2),
    # variant 2 on the wide tile counts arrivals two samples ahead: one sample (no second arrival) and three
    (1, 4325376, True, 2),
    (3, 4325376, False, 2),
    # the wide tile from 4 samples on: 5 samples of 975,000 float4 (222 workgroups, ragged last row),
    # no affine
    (5, 3900000, False, 1),
    (5, 3900000, False, 2),
    # the 8 x 8 tile with its stores interleaved with the next sample's loads (a sample spans at least half
    # the grid): 153 workgroups per sample, the last with 5 rows, the last row with 360 of 512 float4
    (3, 2500000, True, 1),
    (3, 2500000, True, 2),
]


@pytest.mark.parametrize("outer,inner,affine,variant", LN_CASES)
def test_ln_parity(outer, inner, affine, variant):
    _say(f"ln outer={outer} inner={inner} affine={affine} variant={variant}")
    d = synth.make("ln_16x64x256x256", device="cuda", shape=(outer, inner), seed=outer * 7 + inner,
                   normalized_ndim=1)
    w = d["weight"] if affine else None
    b = d["bias"] if affine else None
    mean = torch.empty(outer, device="cuda")
    rstd = torch.empty(outer, device="cuda")
    y = nf.ln_forward(d["x"], w, b, eps=1e-5, variant=variant, mean_out=mean, rstd_out=rstd)
    ref, om, ov = oracle.ln(_np(d["x"]), None if w is None else _np(w), None if b is None else _np(b), eps=1e-5,
                            return_stats=True)
    _assert_close(_np(y), ref, what="ln")
    np.testing.assert_allclose(_np(mean), om, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(_np(rstd), 1.0 / np.sqrt(ov + np.float32(1e-5)), rtol=1e-5)


LN_ROW_CASES = [
    # (outer, inner, dist)  one workgroup per sample (inner <= 8192 vectorized, <= 2048 scalar)
    (64, 4096, "n01"),
    (1000, 768, "n01"),
    (33, 2047, "n01"),          # scalar path
    (7, 8192, "n01"),           # largest vectorized row
    (9, 8196, "n01"),           # just above: split schedule, one row per normalize workgroup
    (300, 20000, "n01"),        # split, many samples of a few rows each
    (64, 4096, "stress"),       # N(100, 0.01) in the row kernel
    (16, 1000, "stress"),
]


@pytest.mark.parametrize("outer,inner,dist", LN_ROW_CASES)
def test_ln_many_short_samples(outer, inner, dist):
    _say(f"ln rows outer={outer} inner={inner} dist={dist}")
    name = "ln_stress_16x64x256x256" if dist == "stress" else "ln_16x64x256x256"
    d = synth.make(name, device="cuda", shape=(outer, inner), seed=outer + inner, normalized_ndim=1)
    mean = torch.empty(outer, device="cuda")
    rstd = torch.empty(outer, device="cuda")
    y = nf.ln_forward(d["x"], d["weight"], d["bias"], eps=1e-5, mean_out=mean, rstd_out=rstd)
    ref, om, ov = oracle.ln(_np(d["x"]), _np(d["weight"]), _np(d["bias"]), eps=1e-5, return_stats=True)
    _assert_close(_np(y), ref, what="ln rows")
    np.testing.assert_allclose(_np(mean), om, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(_np(rstd), 1.0 / np.sqrt(ov + np.float32(1e-5)), rtol=1e-5)
    x = d["x"].clone()
    nf.ln_forward(x, d["weight"], d["bias"], out=x)  # in place: the split schedule (or the row kernel)
    assert torch.equal(x, nf.ln_forward(d["x"], d["weight"], d["bias"], variant=0))


@pytest.mark.parametrize("name", ["ln_16x64x256x256", "ln_stress_16x64x256x256"])
@pytest.mark.parametrize("variant", [0, 1, 2])
def test_ln_full_size(name, variant):
    """Full [16, 64, 256, 256] workloads, N(0,1) and the N(100, 0.01) cancellation stress."""
    _say(f"ln full {name} variant={variant}")
    d = synth.make(name, device="cuda")
    y = nf.ln_forward(d["x"], d["weight"], d["bias"], eps=1e-5, variant=variant)
    ref = oracle.ln(_np(d["x"]), _np(d["weight"]), _np(d["bias"]), eps=1e-5)
    rep = _assert_close(_np(y), ref, what=name)
    _say(f"  max_abs={rep['max_abs']:.3e} max_rel={rep['max_rel']:.3e}")
    y2 = nf.ln_forward(d["x"], d["weight"], d["bias"], eps=1e-5, variant=variant)
    assert torch.equal(y, y2), "not bitwise deterministic"


def test_ln_split_with_the_merge_kernel():
    """The split schedule with at least 16384 moments workgroups in all, where ln_merge_kernel merges the
    partials (below that the last workgroup of each sample does): [16384, 8196], one ragged workgroup per
    sample; y, means and rstds of sampled rows against the oracle, bitwise deterministic."""
    shape = (16384, 8196)
    _say(f"ln split, merge kernel {shape}")
    d = synth.make("ln_16x64x256x256", device="cuda", shape=shape, normalized_ndim=1, seed=77)
    mean = torch.empty(shape[0], device="cuda")
    rstd = torch.empty(shape[0], device="cuda")
    y = nf.ln_forward(d["x"], d["weight"], d["bias"], variant=0, mean_out=mean, rstd_out=rstd)
    rows = [0, 1, 255, 4096, 8191, 8192, 12345, 16382, 16383]
    ref, om, ov = oracle.ln(_np(d["x"][rows]), _np(d["weight"]), _np(d["bias"]), eps=1e-5, return_stats=True)
    _assert_close(_np(y[rows]), ref, what="ln split merge kernel")
    np.testing.assert_allclose(_np(mean[rows]), om, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(_np(rstd[rows]), 1.0 / np.sqrt(ov + np.float32(1e-5)), rtol=1e-5)
    assert torch.equal(y, nf.ln_forward(d["x"], d["weight"], d["bias"], variant=0)), "not bitwise deterministic"
    del d, y
    torch.cuda.empty_cache()


def test_ln_auto_variant_picks_the_measured_fastest():
    """variant 3 runs the single-read kernel wherever it can run (float4 rows, 16-byte aligned tensors,
    a co-resident grid) and the split schedule elsewhere: its output is bitwise that of the variant it
    picks (with groups of workgroups for samples that spread over fewer than all CUs)."""
    for shape, pick in (((16, 4194304), 1), ((4, 4194304), 1), ((8, 2097152), 1), ((1, 4194304), 1),
                        ((16, 1048576), 1), ((64, 262144), 1), ((100, 20000), 1), ((4, 1000001), 0)):
        _say(f"ln auto {shape}")
        d = synth.make("ln_16x64x256x256", device="cuda", shape=shape, normalized_ndim=1, seed=shape[0])
        auto = nf.ln_forward(d["x"], d["weight"], d["bias"], variant=3)
        assert torch.equal(auto, nf.ln_forward(d["x"], d["weight"], d["bias"], variant=pick)), shape
        del d, auto
        torch.cuda.empty_cache()


@pytest.mark.parametrize("shape", [(64, 262144), (32, 1048576), (256, 16384)])
def test_ln_sample_groups_against_the_oracle(shape):
    """Samples that span fewer than all CUs: the default variant runs the single-read kernel with several
    groups of workgroups (16, 4 and 256 groups here); y, the means and the rstds match the oracle."""
    _say(f"ln sample groups {shape}")
    outer, inner = shape
    d = synth.make("ln_16x64x256x256", device="cuda", shape=shape, normalized_ndim=1, seed=outer + 11)
    mean = torch.empty(outer, device="cuda")
    rstd = torch.empty(outer, device="cuda")
    y = nf.ln_forward(d["x"], d["weight"], d["bias"], mean_out=mean, rstd_out=rstd)
    assert torch.equal(y, nf.ln_forward(d["x"], d["weight"], d["bias"], variant=1))
    ref, om, ov = oracle.ln(_np(d["x"]), _np(d["weight"]), _np(d["bias"]), eps=1e-5, return_stats=True)
    _assert_close(_np(y), ref, what=f"ln {shape}")
    np.testing.assert_allclose(_np(mean), om, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(_np(rstd), 1.0 / np.sqrt(ov + np.float32(1e-5)), rtol=1e-5)
    del d, y
    torch.cuda.empty_cache()


@pytest.mark.parametrize("variant", [1, 2])
def test_ln_single_kernel_repeated_and_split_halves(variant):
    """Many back-to-back single-kernel launches on one workspace stay bitwise equal and
    leave the control block clean; stats + apply equals the split variant."""
    _say(f"ln single repeated variant={variant}")
    d = synth.make("ln_16x64x256x256", device="cuda", shape=(4, 1 << 19), normalized_ndim=1, seed=3)
    outer, inner = 4, 1 << 19
    nbytes = nf.ln_forward_workspace_size(outer, inner)
    _, ws = nf.alloc_workspace(nbytes, "cuda")
    nf.ln_forward_workspace_init(ws)
    first = nf.ln_forward(d["x"], d["weight"], d["bias"], variant=variant, workspace=ws)
    for _ in range(300):  # the control-wave kernel's tags cycle every 255 launches
        again = nf.ln_forward(d["x"], d["weight"], d["bias"], variant=variant, workspace=ws)
        assert torch.equal(first, again)
    torch.cuda.synchronize()
    ctrl = ws[:20].view(torch.int32).cpu().tolist()  # gen, done, error, recomputed, gen_ctl
    assert ctrl[1] == 0 and ctrl[2] == 0, ctrl
    if variant == 1:
        assert ctrl[4] == 301 % 255 and ctrl[0] == 0, ctrl
    else:
        assert ctrl[0] == 301 and ctrl[4] == 0, ctrl
    assert ctrl[3] == 0, f"every workgroup was resident, none had its sums recomputed: {ctrl}"
    ws0 = nf.ln_forward_stats(d["x"])
    halves = nf.ln_forward_apply(d["x"], d["weight"], d["bias"], ws0)
    split = nf.ln_forward(d["x"], d["weight"], d["bias"], variant=0)
    assert torch.equal(halves, split)
    ref = oracle.ln(_np(d["x"]), _np(d["weight"]), _np(d["bias"]))
    _assert_close(_np(first), ref, what="ln single")


@pytest.mark.parametrize("variant", [0, 1, 2])
def test_ln_in_place(variant):
    _say(f"ln in place variant={variant}")
    d = synth.make("ln_16x64x256x256", device="cuda", shape=(3, 100000), normalized_ndim=1, seed=9)
    ref = oracle.ln(_np(d["x"]), _np(d["weight"]), _np(d["bias"]))
    x = d["x"].clone()
    nf.ln_forward(x, d["weight"], d["bias"], variant=variant, out=x)
    _assert_close(_np(x), ref, what="ln in place")


# ---------------------------------------------------------------- fc -> GroupNorm epilogue

FC_CASES = [
    # (N, K, C, G)   groups of 4-64 channels use the fused GEMM epilogue, other sizes the GN kernel on h;
    # K % 32 == 0 with 16-byte rows runs the direct-to-LDS GEMM (256-row tiles), else the staged one
    (100, 96, 384, 24),     # M = 16 fused; ragged row tile (100 < 256), 3 column tiles
    (130, 70, 256, 16),     # M = 16 fused; K % 4 != 0 -> staged GEMM, scalar tile loader
    (64, 512, 160, 10),     # M = 16 fused; ragged column tile
    (96, 128, 256, 8),      # M = 32 fused
    (70, 64, 256, 32),      # M = 8 fused
    (300, 32, 200, 25),     # M = 8 fused; two row tiles, the second ragged; ragged column tile
    (40, 36, 512, 8),       # M = 64 fused, staged GEMM
    (90, 64, 320, 5),       # M = 64 fused, direct-to-LDS GEMM; 320 = 2.5 column tiles
    (100, 40, 96, 24),      # M = 4 fused, staged GEMM
    (66, 30, 12, 3),        # M = 4 fused; K % 4 != 0; one narrow column tile
    (50, 64, 100, 5),       # M = 20: GEMM writes h, then the GroupNorm kernel
    (40, 32, 96, 48),       # M = 2: GEMM writes h, then the GroupNorm kernel
    (513, 256, 128, 8),     # M = 16 fused; three row tiles, one row in the last
]


@pytest.mark.parametrize("N,K,C,G", FC_CASES)
def test_fc_gn_parity(N, K, C, G):
    _say(f"fc N={N} K={K} C={C} G={G}")
    d = synth.make("fc_gn_1024x8192x8192", device="cuda", shape=(N, K), hidden=C, seed=N + K + C)
    y = nf.fc_gn_forward(d["x"], d["W"], d["b"], d["gamma"], d["beta"], G)
    ref = oracle.fc_gn_lrelu_x2(_np(d["x"]), _np(d["W"]), _np(d["b"]), _np(d["gamma"]), _np(d["beta"]), G)
    _assert_close(_np(y), ref, rtol=RTOL_FC, what="fc_gn")


def test_fc_gn_full_size_sampled_rows():
    """Full 1024 x 8192 x 8192 problem; the oracle recomputes rows from every 256-row GEMM tile (the first
    and last row of each, and rows inside)."""
    _say("fc full 1024x8192x8192 (sampled rows)")
    d = synth.make("fc_gn_1024x8192x8192", device="cuda")
    y = nf.fc_gn_forward(d["x"], d["W"], d["b"], d["gamma"], d["beta"], 512)
    rows = [0, 1, 127, 255, 256, 300, 511, 512, 600, 767, 768, 900, 1023]
    ref = oracle.fc_gn_lrelu_x2(_np(d["x"][rows]), _np(d["W"]), _np(d["b"]), _np(d["gamma"]), _np(d["beta"]), 512)
    rep = _assert_close(_np(y[rows]), ref, rtol=RTOL_FC, what="fc full")
    _say(f"  max_abs={rep['max_abs']:.3e} max_rel={rep['max_rel']:.3e}")


def test_prepared_calls_match_direct_calls():
    """nf.prepare re-issues exactly the marshalled C call (used by the benchmark's launch loops)."""
    _say("prepared calls")
    d = synth.make("gn_lrelu_x2_1024x8192", device="cuda", shape=(32, 8192), seed=21)
    y1 = nf.gn_lrelu_x2_forward(d["x"], d["gamma"], d["beta"], 512)
    y2 = torch.empty_like(y1)
    call = nf.prepare(nf.gn_lrelu_x2_forward, d["x"], d["gamma"], d["beta"], 512, out=y2)
    call()
    assert torch.equal(y1, y2)
    l = synth.make("ln_16x64x256x256", device="cuda", shape=(2, 64, 64, 64), seed=22)
    for variant in (0, 1, 2):
        z1 = nf.ln_forward(l["x"], l["weight"], l["bias"], variant=variant)
        z2 = torch.zeros_like(z1)
        run = nf.prepare(nf.ln_forward, l["x"], l["weight"], l["bias"], variant=variant, out=z2)
        run()
        run()
        assert torch.equal(z1, z2)


def test_captured_graph_replays_match_eager():
    """The split LayerNorm, the single-read LayerNorm (an ordinary launch), GN, RMS and fc+GN calls
    captured in one HIP graph (via torch's graph API on the capturing stream) replay correctly several
    times, with eager work and synchronizations in between."""
    _say("graph capture")
    l = synth.make("ln_16x64x256x256", device="cuda", shape=(4, 70000), normalized_ndim=1, seed=31)
    s1 = synth.make("ln_16x64x256x256", device="cuda", shape=(3, 1 << 20), normalized_ndim=1, seed=35)
    single_eager = nf.ln_forward(s1["x"], s1["weight"], s1["bias"], variant=1)
    single_out = torch.empty_like(single_eager)
    _, ws1 = nf.alloc_workspace(nf.ln_forward_workspace_size(3, 1 << 20), "cuda")
    nf.ln_forward_workspace_init(ws1)
    g = synth.make("gn_lrelu_x2_1024x8192", device="cuda", shape=(64, 8192), seed=32)
    r = synth.make("rms_ch_112x64x512x512", device="cuda", shape=(2, 64, 4096), seed=33)
    f = synth.make("fc_gn_1024x8192x8192", device="cuda", shape=(128, 256), hidden=512, seed=34)
    ln_eager = nf.ln_forward(l["x"], l["weight"], l["bias"])
    gn_eager = nf.gn_lrelu_x2_forward(g["x"], g["gamma"], g["beta"], 512)
    rms_eager = nf.rmsnorm_ch_forward(r["x"])
    fc_eager = nf.fc_gn_forward(f["x"], f["W"], f["b"], f["gamma"], f["beta"], 32)
    outs = [torch.empty_like(t) for t in (ln_eager, gn_eager, rms_eager, fc_eager)]
    _, ws = nf.alloc_workspace(nf.ln_forward_workspace_size(4, 70000), "cuda")
    nf.ln_forward_workspace_init(ws)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            nf.ln_forward(l["x"], l["weight"], l["bias"], out=outs[0], workspace=ws)
            nf.gn_lrelu_x2_forward(g["x"], g["gamma"], g["beta"], 512, out=outs[1])
            nf.rmsnorm_ch_forward(r["x"], out=outs[2])
            nf.fc_gn_forward(f["x"], f["W"], f["b"], f["gamma"], f["beta"], 32, out=outs[3])
            nf.ln_forward(s1["x"], s1["weight"], s1["bias"], variant=1, out=single_out, workspace=ws1)
    torch.cuda.synchronize()
    outs.append(single_out)
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))          # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, e, name in zip(outs, (ln_eager, gn_eager, rms_eager, fc_eager, single_eager),
                              ("ln", "gn", "rms", "fc", "ln single-read")):
            assert torch.equal(o, e), f"replay {rep}: {name} differs from eager"
    ctrl = ws1[:20].view(torch.int32).cpu().tolist()  # gen, done, error, recomputed, gen_ctl
    assert ctrl[4] == 4 and ctrl[1] == 0 and ctrl[3] == 0, ctrl


def test_modules_match_the_functions():
    """The nn.Module front ends (the pages' constructor arguments) call the same kernels."""
    _say("modules")
    from normalization_ln_forward_amd import modules

    x = synth.make("ln_16x64x256x256", device="cuda", shape=(2, 8, 16, 16), seed=41)["x"]
    ln = modules.LayerNorm((8, 16, 16), eps=1e-5, device="cuda")
    with torch.no_grad():
        ln.weight.normal_(1.0, 0.1)
        ln.bias.normal_(0.0, 0.1)
    assert torch.equal(ln(x), nf.ln_forward(x, ln.weight.detach(), ln.bias.detach()))
    _assert_close(_np(ln(x)), oracle.ln(_np(x), _np(ln.weight), _np(ln.bias)), what="module ln")
    rms = modules.RMSNormChannel(8)
    _assert_close(_np(rms(x)), oracle.rms_ch(_np(x)), what="module rms")
    g = synth.make("gn_lrelu_x2_1024x8192", device="cuda", shape=(4, 256), seed=42)["x"]
    gn = modules.GroupNormLeakyReLUx2(256, 16, device="cuda")
    _assert_close(_np(gn(g)), oracle.gn_lrelu_x2(_np(g), None, None, 16), what="module gn")
    fc = modules.FcGroupNormLeakyReLUx2(64, 128, 8, device="cuda")
    xf = synth.make("fc_gn_1024x8192x8192", device="cuda", shape=(16, 64), hidden=128, seed=43)["x"]
    ref = oracle.fc_gn_lrelu_x2(_np(xf), _np(fc.fc_weight), _np(fc.fc_bias), None, None, 8)
    _assert_close(_np(fc(xf)), ref, rtol=RTOL_FC, what="module fc_gn")


def test_ln_alternating_shapes_and_workspace_reinit():
    """Calls of different shapes in turn (the binding keeps one workspace per shape) stay correct, and a
    caller's workspace re-zeroed between shapes serves each of them."""
    _say("ln alternating shapes")
    shapes = [(6, 4097), (2, 40001), (16, 20000), (6, 4097), (3, 70000), (16, 20000), (2, 40001)]
    data = {s: synth.make("ln_16x64x256x256", device="cuda", shape=s, normalized_ndim=1, seed=s[0] + s[1])
            for s in set(shapes)}
    refs = {s: oracle.ln(_np(d["x"]), _np(d["weight"]), _np(d["bias"])) for s, d in data.items()}
    for variant in (0, 1, 2):
        for s in shapes:
            d = data[s]
            _assert_close(_np(nf.ln_forward(d["x"], d["weight"], d["bias"], variant=variant)), refs[s],
                          what=f"ln {s} variant {variant}")
    big = max(nf.ln_forward_workspace_size(*s) for s in shapes)
    _, ws = nf.alloc_workspace(big, "cuda")
    for variant in (0, 1, 2):
        for s in shapes:
            d = data[s]
            nf.ln_forward_workspace_init(ws)
            for _ in range(2):
                y = nf.ln_forward(d["x"], d["weight"], d["bias"], variant=variant, workspace=ws)
                _assert_close(_np(y), refs[s], what=f"ln {s} variant {variant}, own workspace")


def test_workspace_check_reports_and_clears_a_failed_wait():
    """ln_forward_workspace_check: OK after healthy single-kernel calls; a recorded give-up (planted from
    the host in the workspace's error word, as a kernel whose wait ran out would leave it) is reported as
    NORMFWD_ERR_INCOMPLETE once and then cleared."""
    _say("ln workspace check")
    s = (6, 40000)
    d = synth.make("ln_16x64x256x256", device="cuda", shape=s, normalized_ndim=1, seed=77)
    ref = oracle.ln(_np(d["x"]), _np(d["weight"]), _np(d["bias"]))
    _, ws = nf.alloc_workspace(nf.ln_forward_workspace_size(*s), "cuda")
    nf.ln_forward_workspace_init(ws)
    for variant in (1, 2, 0):
        y = nf.ln_forward(d["x"], d["weight"], d["bias"], variant=variant, workspace=ws)
        nf.ln_forward_workspace_check(ws)
        _assert_close(_np(y), ref, what=f"ln {s} variant {variant} before the check")
    word = ws.view(torch.int32)[2:3]
    word.fill_(1)
    with pytest.raises(nf.NormFwdError) as e:
        nf.ln_forward_workspace_check(ws)
    assert e.value.status == 5
    assert int(word.item()) == 0
    nf.ln_forward_workspace_check(ws)


def test_time_next_kernel_stamps_one_launch():
    """normfwd_time_next_kernel: the next launch (ordinary or cooperative) stamps the armed events, later
    launches leave them alone, and the results are unchanged."""
    _say("time_next_kernel")
    g = synth.make("gn_lrelu_x2_1024x8192", device="cuda", shape=(256, 8192), seed=51)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    b.record()
    torch.cuda.synchronize()
    nf.time_next_kernel(a, b)
    y = nf.gn_lrelu_x2_forward(g["x"], g["gamma"], g["beta"], 512)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    assert 0.0 < ms < 100.0, ms
    y2 = nf.gn_lrelu_x2_forward(g["x"], g["gamma"], g["beta"], 512)
    torch.cuda.synchronize()
    assert a.elapsed_time(b) == ms, "a later launch re-stamped the events"
    assert torch.equal(y, y2)
    d = synth.make("ln_16x64x256x256", device="cuda", shape=(4, 1 << 18), normalized_ndim=1, seed=52)
    for variant in (0, 1, 2):
        nf.time_next_kernel(a, b)
        out = nf.ln_forward(d["x"], d["weight"], d["bias"], variant=variant)
        torch.cuda.synchronize()
        assert 0.0 < a.elapsed_time(b) < 100.0
        _assert_close(_np(out), oracle.ln(_np(d["x"]), _np(d["weight"]), _np(d["bias"])), what=f"ln {variant}")


def test_empty_inputs_and_k_zero():
    """Empty batches return empty outputs (the library launches nothing); fc with K = 0 gives
    GroupNorm of the bias."""
    _say("empty inputs")
    e = torch.empty(0, 64, 8, 8, device="cuda")
    assert nf.ln_forward(e).shape == e.shape
    for variant in (1, 2):
        assert nf.ln_forward(e, variant=variant).shape == e.shape
    assert nf.gn_lrelu_x2_forward(torch.empty(0, 256, device="cuda"), None, None, 16).shape == (0, 256)
    assert nf.rmsnorm_ch_forward(torch.empty(0, 64, 16, device="cuda")).shape == (0, 64, 16)
    assert nf.rmsnorm_ch_forward(torch.empty(3, 64, 0, device="cuda")).shape == (3, 64, 0)
    f = synth.make("fc_gn_1024x8192x8192", device="cuda", shape=(5, 64), hidden=128, seed=61)
    y0 = nf.fc_gn_forward(f["x"][:0], f["W"], f["b"], f["gamma"], f["beta"], 8)
    assert y0.shape == (0, 128)
    x0 = torch.empty(5, 0, device="cuda")
    w0 = torch.empty(128, 0, device="cuda")
    y = nf.fc_gn_forward(x0, w0, f["b"], f["gamma"], f["beta"], 8)
    ref = oracle.fc_gn_lrelu_x2(np.zeros((5, 0), np.float32), np.zeros((128, 0), np.float32), _np(f["b"]),
                                _np(f["gamma"]), _np(f["beta"]), 8)
    _assert_close(_np(y), ref, rtol=RTOL_FC, what="fc K=0")
