"""ln_forward_noalloc (the LayerNorm entry point that allocates nothing: its workspace is the library's
static per-GPU scratch) against ln_forward on a caller workspace, through the C ABI."""
import sys

import numpy as np
import pytest
import torch

import oracle
from normalization_ln_forward_amd import _lib, synth
import normalization_ln_forward_amd as nf

pytestmark = pytest.mark.gpu


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


def _pair(shape, name, seed, variant):
    """y and (mean, rstd) from ln_forward_noalloc and from ln_forward with its own zeroed workspace."""
    outer = shape[0]
    d = synth.make(name, device="cuda", shape=shape, normalized_ndim=1, seed=seed)
    m1, r1 = torch.empty(outer, device="cuda"), torch.empty(outer, device="cuda")
    y1 = nf.ln_forward_noalloc(d["x"], d["weight"], d["bias"], variant=variant, mean_out=m1, rstd_out=r1)
    _, ws = nf.alloc_workspace(nf.ln_forward_workspace_size(*shape), "cuda")
    nf.ln_forward_workspace_init(ws)
    m2, r2 = torch.empty(outer, device="cuda"), torch.empty(outer, device="cuda")
    y2 = nf.ln_forward(d["x"], d["weight"], d["bias"], variant=variant, workspace=ws, mean_out=m2, rstd_out=r2)
    torch.cuda.synchronize()
    return d, (y1, m1, r1), (y2, m2, r2)


@pytest.mark.parametrize("variant", [3, 0, 1, 2])
def test_noalloc_matches_ln_forward_two_calls_second_smaller(variant):
    """Two calls in a row, the second on a smaller input (so the scratch is re-laid out): each equals
    ln_forward bit for bit and the oracle within 1e-4."""
    for shape, name in (((16, 1 << 20), "ln_16x64x256x256"), ((3, 300000), "ln_stress_16x64x256x256")):
        _say(f"noalloc variant={variant} shape={shape} {name}")
        d, a, b = _pair(shape, name, 5 + shape[0], variant)
        for u, v in zip(a, b):
            assert torch.equal(u, v)
        ref = oracle.ln(_np(d["x"]), _np(d["weight"]), _np(d["bias"]))
        rep = oracle.allclose_report(_np(a[0]), ref, 1e-4, 1e-4)
        assert rep["ok"], rep
        del d, a, b
        torch.cuda.empty_cache()


def test_noalloc_repeated_same_shape_and_back():
    """Repeated calls of one shape reuse the scratch as it was left; returning to an earlier shape clears
    it again.  Every result equals ln_forward's."""
    shapes = [(4, 1 << 19), (4, 1 << 19), (2, 65536), (4, 1 << 19), (2, 65536), (2, 65536)]
    for i, s in enumerate(shapes):
        _say(f"noalloc sequence {i} shape={s}")
        _, a, b = _pair(s, "ln_16x64x256x256", 100 + i, 3)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])


def test_noalloc_refuses_shapes_beyond_its_scratch():
    """A shape whose workspace exceeds the 8 MiB scratch is refused before anything is enqueued."""
    big = (1024, 1 << 20)
    need = nf.ln_forward_workspace_size(*big)
    assert need > (8 << 20)
    x = torch.empty(8, device="cuda")
    st = _lib.lib().ln_forward_noalloc(_lib._ptr(x), None, None, _lib._ptr(x), big[0], big[1], 1e-5, None, None,
                                       3, None)
    assert st == 2, _lib.lib().normfwd_last_error()
    assert b"scratch" in _lib.lib().normfwd_last_error()
