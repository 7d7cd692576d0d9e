"""Strided RMSNorm views and the statistics outputs of GroupNorm and RMSNorm, against the fp64 oracle,
through the C ABI.

* rmsnorm_ch_forward_strided (RMS page "Kimi-K2.6 l1_p36", turn 2 weighs the layout and the wrapper's
  contiguity handling): channel slices, batch-strided views, strided outputs (elements outside the view
  untouched) and in place, on the 128-bit, scalar and streaming kernels; rstd_out per position.
* gn_lrelu_x2_forward / fc_gn_forward mean_out and rstd_out per (row, group) (GN page "Kimi-K2.6 l2_p62",
  turn 1: the framework layer keeps them for backward), on every kernel that computes them.
Outputs: |g - o| <= 1e-4 + 1e-4 |o| (rtol 2e-3 for fc); statistics as stated per test.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from normalization_ln_forward_amd import _lib, synth
import normalization_ln_forward_amd as nf

pytestmark = pytest.mark.gpu

EPS = np.float32(1e-5)


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


# ---------------------------------------------------------------- strided RMSNorm

RMS_VIEW_CASES = [
    # (full x shape, x view (dim 0 slice, dim 1 slice), full out shape or None, out dim-1 slice)
    ((3, 96, 32, 32), (slice(None), slice(16, 80)), None, None),              # channel slice, 128-bit path
    ((6, 64, 32, 32), (slice(None, None, 2), slice(None)), None, None),       # batch stride
    ((6, 96, 16, 16), (slice(1, None, 2), slice(8, 72)), (3, 80, 16, 16), slice(8, 72)),  # both, strided out
    ((4, 70, 5, 7), (slice(None), slice(3, 67)), None, None),                 # S = 35: scalar path
    ((2, 700, 64), (slice(None), slice(50, 650)), None, None),                # C = 600: streaming kernel
    ((3, 130, 48), (slice(None), slice(1, 101)), (3, 101, 48), slice(0, 100)),  # C = 100: 16-channel waves
]


@pytest.mark.parametrize("full,view,out_full,out_view", RMS_VIEW_CASES)
def test_rms_strided_views(full, view, out_full, out_view):
    _say(f"rms view full={full} view={view} out_full={out_full}")
    d = synth.make("rms_ch_112x64x512x512", device="cuda", shape=full, seed=sum(full))
    x = d["x"][view]
    B, C = x.shape[0], x.shape[1]
    S = x.numel() // (B * C)
    if out_full is not None:
        ybuf = torch.full(out_full, float("nan"), device="cuda")
        y = ybuf[:, out_view]
    else:
        ybuf, y = None, None
    rstd = torch.empty((B,) + tuple(x.shape[2:]), device="cuda")
    y = nf.rmsnorm_ch_forward(x, out=y, rstd_out=rstd)
    ref, ms = oracle.rms_ch(_np(x.contiguous()), return_ms=True)
    _close(_np(y.contiguous()), ref, what="rms view")
    np.testing.assert_allclose(_np(rstd).reshape(B, S), 1.0 / np.sqrt(ms + EPS), rtol=1e-5)
    if ybuf is not None:  # nothing outside the view was written
        mask = torch.ones(out_full, dtype=torch.bool, device="cuda")
        mask[:, out_view] = False
        assert torch.isnan(ybuf[mask]).all()


def test_rms_strided_in_place_and_equal_to_contiguous():
    """In place on a channel slice of a larger tensor equals the contiguous call on a copy of the slice,
    bit for bit, and leaves the other channels alone."""
    _say("rms strided in place")
    d = synth.make("rms_ch_112x64x512x512", device="cuda", shape=(4, 80, 64, 64), seed=3)
    buf = d["x"].clone()
    ref = nf.rmsnorm_ch_forward(buf[:, 8:72].contiguous())
    before = buf.clone()
    view = buf[:, 8:72]
    nf.rmsnorm_ch_forward(view, out=view)
    assert torch.equal(buf[:, 8:72], ref)
    assert torch.equal(buf[:, :8], before[:, :8]) and torch.equal(buf[:, 72:], before[:, 72:])


def test_rms_full_size_every_sample():
    """The full [112, 64, 512, 512] workload in the benchmark's launch, every sample against the oracle
    (streamed from the GPU eight samples at a time), with rstd_out through the strided entry point."""
    _say("rms full 112x64x512x512, every sample")
    d = synth.make("rms_ch_112x64x512x512", device="cuda")
    x = d["x"]
    y = nf.rmsnorm_ch_forward(x, eps=1e-5)
    torch.cuda.synchronize()
    worst = 0.0
    for b0 in range(0, 112, 8):
        xs = _np(x[b0:b0 + 8])
        ref = oracle.rms_ch(xs)
        rep = _close(_np(y[b0:b0 + 8]), ref, what=f"rms full samples {b0}..{b0 + 7}")
        worst = max(worst, rep["max_abs"])
        del xs, ref
    _say(f"  max_abs over all samples {worst:.3e}")
    rstd = torch.empty((112, 512, 512), device="cuda")
    y2 = nf.rmsnorm_ch_forward(x, rstd_out=rstd)
    assert torch.equal(y, y2), "the strided entry point differs from the contiguous one"
    _, ms = oracle.rms_ch(_np(x[:2]), return_ms=True)
    np.testing.assert_allclose(_np(rstd[:2]).reshape(2, -1), 1.0 / np.sqrt(ms + EPS), rtol=1e-5)
    del x, y, y2, rstd, d
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- GroupNorm statistics

GN_STATS_CASES = [
    (64, 8192, 512, False),   # fast kernel, M = 16
    (16, 4096, 1024, False),  # fast, M = 4 (one lane per group)
    (16, 8192, 64, False),    # fast, M = 128 (32 lanes per group)
    (16, 35, 7, False),       # lane kernel, M = 5
    (8, 3000, 30, False),     # wave kernel, M = 100
    (8, 4096, 256, True),     # misaligned: lane kernel, M = 16
]


@pytest.mark.parametrize("N,C,G,misalign", GN_STATS_CASES)
def test_gn_statistics(N, C, G, misalign):
    _say(f"gn stats N={N} C={C} G={G} misalign={misalign}")
    d = synth.make("gn_lrelu_x2_1024x8192", device="cuda", shape=(N, C), seed=N * C + G)
    x = d["x"]
    x[:, ::11] += 3.0
    if misalign:
        buf = torch.empty(N * C + 1, device="cuda")
        buf[1:].copy_(x.reshape(-1))
        x = buf[1:].view(N, C)
    mean = torch.empty(N, G, device="cuda")
    rstd = torch.empty(N, G, device="cuda")
    y = nf.gn_lrelu_x2_forward(x, d["gamma"], d["beta"], G, mean_out=mean, rstd_out=rstd)
    ref, om, ov = oracle.gn_lrelu_x2(_np(x), _np(d["gamma"]), _np(d["beta"]), G, return_stats=True)
    _close(_np(y), ref, what="gn with stats")
    np.testing.assert_allclose(_np(mean), om, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(_np(rstd), 1.0 / np.sqrt(ov + EPS), rtol=1e-5)
    # asking for the statistics changes nothing else
    assert torch.equal(y, nf.gn_lrelu_x2_forward(x, d["gamma"], d["beta"], G))


FC_STATS_CASES = [
    (100, 96, 384, 24),     # fused, 16 channels per group, direct-to-LDS GEMM
    (96, 128, 512, 8),      # fused, 64 channels per group
    (100, 40, 96, 24),      # fused, 4 channels per group, staged GEMM
    (130, 70, 256, 8),      # fused, 32 channels per group, staged GEMM (K % 4 != 0)
    (50, 64, 100, 5),       # 20 channels per group: h, then the GroupNorm kernel
]


@pytest.mark.parametrize("N,K,C,G", FC_STATS_CASES)
def test_fc_gn_statistics(N, K, C, G):
    _say(f"fc stats N={N} K={K} C={C} G={G}")
    d = synth.make("fc_gn_1024x8192x8192", device="cuda", shape=(N, K), hidden=C, seed=N + K + C + G)
    b = d["b"] + 2.0
    mean = torch.empty(N, G, device="cuda")
    rstd = torch.empty(N, G, device="cuda")
    y = nf.fc_gn_forward(d["x"], d["W"], b, d["gamma"], d["beta"], G, mean_out=mean, rstd_out=rstd)
    h = oracle.fc(_np(d["x"]), _np(d["W"]), _np(b))
    ref, om, ov = oracle.gn_lrelu_x2(h, _np(d["gamma"]), _np(d["beta"]), G, return_stats=True)
    _close(_np(y), ref, rtol=2e-3, what="fc with stats")
    np.testing.assert_allclose(_np(mean), om, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(_np(rstd), 1.0 / np.sqrt(ov + EPS), rtol=2e-3)
    assert torch.equal(y, nf.fc_gn_forward(d["x"], d["W"], b, d["gamma"], d["beta"], G))
