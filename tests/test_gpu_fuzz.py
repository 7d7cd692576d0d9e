"""GPU parity on seeded random shapes (every dispatch path, ragged sizes), against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import normalization_ln_forward_amd as nf
from normalization_ln_forward_amd import _lib, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.lib()
    yield
    torch.cuda.synchronize()


def _np(t):
    return t.detach().cpu().numpy()


def _check(got, ref, rtol=1e-4, what=""):
    rep = oracle.allclose_report(_np(got), ref, 1e-4, rtol)
    assert rep["ok"], f"{what}: {rep}"


RNG = np.random.default_rng(20261202)
LN_SHAPES = [(int(RNG.integers(1, 7)), int(n)) for n in
             [1, 3, 17, 1000, 4097, 8191, 9000, 70000, 300001] + list(RNG.integers(2, 200000, 6))]
GN_SHAPES = []
for _ in range(14):
    M = int(RNG.choice([1, 2, 3, 4, 5, 8, 12, 16, 20, 32, 64, 128, 256, 300]))
    G = int(RNG.integers(1, 20))
    GN_SHAPES.append((int(RNG.integers(1, 10)), M * G, G))
RMS_SHAPES = [(int(RNG.integers(1, 4)), int(RNG.integers(1, 700)), int(RNG.integers(1, 5000))) for _ in range(12)]
FC_SHAPES = []
for _ in range(8):
    M = int(RNG.choice([5, 8, 16, 32]))
    G = int(RNG.integers(1, 12))
    FC_SHAPES.append((int(RNG.integers(1, 200)), int(RNG.integers(1, 300)), M * G, G))


@pytest.mark.parametrize("outer,inner", LN_SHAPES)
@pytest.mark.parametrize("variant", [0, 1, 2])
def test_ln_random_shapes(outer, inner, variant):
    print(f"ln fuzz outer={outer} inner={inner} variant={variant}", flush=True)
    d = synth.make("ln_16x64x256x256", device="cuda", shape=(outer, inner), seed=outer + 3 * inner,
                   normalized_ndim=1)
    y = nf.ln_forward(d["x"], d["weight"], d["bias"], variant=variant)
    _check(y, oracle.ln(_np(d["x"]), _np(d["weight"]), _np(d["bias"])), what="ln")


@pytest.mark.parametrize("N,C,G", GN_SHAPES)
def test_gn_random_shapes(N, C, G):
    print(f"gn fuzz N={N} C={C} G={G}", flush=True)
    d = synth.make("gn_lrelu_x2_1024x8192", device="cuda", shape=(N, C), seed=N + C + G)
    y = nf.gn_lrelu_x2_forward(d["x"], d["gamma"], d["beta"], G)
    _check(y, oracle.gn_lrelu_x2(_np(d["x"]), _np(d["gamma"]), _np(d["beta"]), G), what="gn")


@pytest.mark.parametrize("B,C,S", RMS_SHAPES)
def test_rms_random_shapes(B, C, S):
    print(f"rms fuzz B={B} C={C} S={S}", flush=True)
    d = synth.make("rms_ch_112x64x512x512", device="cuda", shape=(B, C, S), seed=B + C + S)
    _check(nf.rmsnorm_ch_forward(d["x"]), oracle.rms_ch(_np(d["x"])), what="rms")


@pytest.mark.parametrize("N,K,C,G", FC_SHAPES)
def test_fc_gn_random_shapes(N, K, C, G):
    print(f"fc fuzz N={N} K={K} C={C} G={G}", flush=True)
    d = synth.make("fc_gn_1024x8192x8192", device="cuda", shape=(N, K), hidden=C, seed=N + K + C)
    y = nf.fc_gn_forward(d["x"], d["W"], d["b"], d["gamma"], d["beta"], G)
    ref = oracle.fc_gn_lrelu_x2(_np(d["x"]), _np(d["W"]), _np(d["b"]), _np(d["gamma"]), _np(d["beta"]), G)
    _check(y, ref, rtol=2e-3, what="fc_gn")
