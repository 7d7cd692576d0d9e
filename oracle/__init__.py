"""CPU oracle for the normalization forward passes — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the GPU library
(``normalization_ln_forward_amd``) and does not import it.

Each function promotes its fp32 (or any real) inputs exactly to float64,
calls the plain double-precision definition in ``oracle.c`` and returns the
unrounded float64 result.  ``eps`` and ``negative_slope`` are first rounded to
fp32 (the value the GPU library receives through its ``float`` arguments) and
then promoted, so both sides start from the same numbers.

Pages cited (POPCORNBENCH agent transcripts; a "turn" is one agent message):
  LN page  "Kimi-K2.6 l1_p40"  LayerNorm over (64, 256, 256) per sample
  GN page  "Kimi-K2.6 l2_p62"  fc -> GroupNorm(512) -> LeakyReLU -> x + x
  RMS page "Kimi-K2.6 l1_p36"  RMSNorm along dim 1 of NCHW
"""
import ctypes
import os

import numpy as np

from . import build as _build

_DP = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.c_int64


def _f64(a):
    """Exact promotion to a C-contiguous float64 array (None stays None)."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # a torch tensor on the CPU
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a), dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_DP)


def as_f32_scalar(v) -> float:
    """The fp32 value a C ``float`` argument holds, as a Python float."""
    return float(np.float32(v))


class Oracle:
    """The oracle functions bound to one build of ``oracle.c``."""

    def __init__(self, libpath: str):
        lib = ctypes.CDLL(libpath)
        lib.oracle_ln.argtypes = [_DP, _DP, _DP, _I64, _I64, ctypes.c_double, _DP, _DP, _DP]
        lib.oracle_gn_lrelu_x2.argtypes = [_DP, _DP, _DP, _I64, _I64, _I64, ctypes.c_double,
                                           ctypes.c_double, _DP, _DP, _DP]
        lib.oracle_rms_ch.argtypes = [_DP, _I64, _I64, _I64, ctypes.c_double, _DP, _DP]
        lib.oracle_fc.argtypes = [_DP, _DP, _DP, _I64, _I64, _I64, _DP]
        for f in (lib.oracle_ln, lib.oracle_gn_lrelu_x2, lib.oracle_rms_ch, lib.oracle_fc):
            f.restype = None
        lib.oracle_num_threads.restype = ctypes.c_int
        self.lib = lib

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def ln(self, x, weight=None, bias=None, eps=1e-5, normalized_ndim=None, return_stats=False, out=None):
        """LayerNorm over the trailing dims of each sample (LN page, turn 1).

        ``x`` has shape ``[outer, *normalized_shape]``; by default every dim
        but the first is normalized (the LN page normalizes (C, H, W) of
        NCHW).  ``weight``/``bias`` have ``normalized_shape`` or are None.
        Returns y (float64, x's shape) and optionally (mean[outer], var[outer]).
        Inputs that already are C-contiguous float64 arrays are used as they
        are (no copy), and ``out`` (a C-contiguous float64 array of x's shape)
        receives y if given, so a caller can time the computation alone.
        """
        xd = _f64(x)
        nd = xd.ndim - 1 if normalized_ndim is None else normalized_ndim
        inner = int(np.prod(xd.shape[xd.ndim - nd:], dtype=np.int64)) if nd > 0 else 1
        outer = xd.size // inner if inner else 0
        w, b = _f64(weight), _f64(bias)
        if w is not None:
            assert w.size == inner
        if b is not None:
            assert b.size == inner
        if out is not None:
            assert out.dtype == np.float64 and out.shape == xd.shape and out.flags.c_contiguous
            y = out
        else:
            y = np.empty_like(xd)
        mean = np.empty(outer, np.float64)
        var = np.empty(outer, np.float64)
        self.lib.oracle_ln(_ptr(xd), _ptr(w), _ptr(b), outer, inner, as_f32_scalar(eps),
                           _ptr(y), _ptr(mean), _ptr(var))
        return (y, mean, var) if return_stats else y

    def gn_lrelu_x2(self, x, gamma, beta, num_groups, eps=1e-5, negative_slope=0.01,
                    return_stats=False):
        """GroupNorm(num_groups) on [N, C] -> LeakyReLU -> x + x (GN page, turn 1)."""
        xd = _f64(x)
        assert xd.ndim == 2, "x must be [N, C]"
        N, C = xd.shape
        G = int(num_groups)
        assert G > 0 and C % G == 0, "C must be a multiple of num_groups"
        g, bt = _f64(gamma), _f64(beta)
        y = np.empty_like(xd)
        mean = np.empty((N, G), np.float64)
        var = np.empty((N, G), np.float64)
        self.lib.oracle_gn_lrelu_x2(_ptr(xd), _ptr(g), _ptr(bt), N, C, G, as_f32_scalar(eps),
                                    as_f32_scalar(negative_slope), _ptr(y), _ptr(mean),
                                    _ptr(var))
        return (y, mean, var) if return_stats else y

    def rms_ch(self, x, eps=1e-5, return_ms=False):
        """RMSNorm along dim 1 of a [B, C, *spatial] tensor (RMS page, turns 1-2)."""
        xd = _f64(x)
        assert xd.ndim >= 2
        B, C = xd.shape[0], xd.shape[1]
        S = int(np.prod(xd.shape[2:], dtype=np.int64)) if xd.ndim > 2 else 1
        y = np.empty_like(xd)
        ms = np.empty((B, S), np.float64)
        self.lib.oracle_rms_ch(_ptr(xd), B, C, S, as_f32_scalar(eps), _ptr(y), _ptr(ms))
        return (y, ms) if return_ms else y

    def fc(self, x, W, bias=None):
        """h = x W^T + bias with x [N, K], W [Cout, K] (GN page, turn 1)."""
        xd, Wd, bd = _f64(x), _f64(W), _f64(bias)
        N, K = xd.shape
        Cout, K2 = Wd.shape
        assert K == K2
        h = np.empty((N, Cout), np.float64)
        self.lib.oracle_fc(_ptr(xd), _ptr(Wd), _ptr(bd), N, K, Cout, _ptr(h))
        return h

    def fc_gn_lrelu_x2(self, x, W, bias, gamma, beta, num_groups, eps=1e-5,
                       negative_slope=0.01):
        """fc, then GroupNorm -> LeakyReLU -> x + x on the unrounded fc output."""
        return self.gn_lrelu_x2(self.fc(x, W, bias), gamma, beta, num_groups, eps,
                                negative_slope)


_DEFAULT = None


def default() -> Oracle:
    """The oracle built from ``oracle.c`` (compiled on first use if missing or stale)."""
    global _DEFAULT
    if _DEFAULT is None:
        if not os.path.exists(_build.LIB) or (
                os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
            _build.build()
        _DEFAULT = Oracle(_build.LIB)
    return _DEFAULT


def num_threads():
    return default().num_threads()


def ln(*a, **k):
    return default().ln(*a, **k)


def gn_lrelu_x2(*a, **k):
    return default().gn_lrelu_x2(*a, **k)


def rms_ch(*a, **k):
    return default().rms_ch(*a, **k)


def fc(*a, **k):
    return default().fc(*a, **k)


def fc_gn_lrelu_x2(*a, **k):
    return default().fc_gn_lrelu_x2(*a, **k)


def allclose_report(got, ref, atol, rtol):
    """Elementwise ``|g - o| <= atol + rtol*|o|`` with g finite.

    ``got`` is the GPU result (any float dtype), ``ref`` the oracle's
    unrounded float64.  Returns a dict with ok, max_abs, max_rel (over
    |o| > 1e-3), n_bad and the worst offending flat index.
    """
    g = np.asarray(got, dtype=np.float64).ravel()
    o = np.asarray(ref, dtype=np.float64).ravel()
    assert g.shape == o.shape, (g.shape, o.shape)
    err = np.abs(g - o)
    lim = atol + rtol * np.abs(o)
    finite = np.isfinite(g)
    bad = ~(finite & (err <= lim))
    big = np.abs(o) > 1e-3
    rel = err[big] / np.abs(o[big]) if big.any() else np.zeros(1)
    worst = int(np.argmax(np.where(finite, err - lim, np.inf))) if g.size else -1
    return {
        "ok": bool(not bad.any()),
        "n_bad": int(bad.sum()),
        "max_abs": float(err[finite].max()) if finite.any() else float("inf"),
        "max_rel": float(rel.max()) if rel.size else 0.0,
        "worst_index": worst,
        "n": int(g.size),
    }
