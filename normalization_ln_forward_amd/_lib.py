"""ctypes binding of libnormfwd.so (the C ABI in include/normfwd.h).

Argument marshalling only: shapes, dtypes, devices and contiguity are checked
here, outputs and workspaces are allocated with torch, and every call goes
straight to the HIP library on the caller's current stream.  Nothing is
computed in Python, and there is no fallback: if the library is not built the
functions raise.

torch is imported before the library is loaded so that the library binds to
the HIP runtime torch already loaded (one runtime per process, so torch's
stream handles and device pointers are valid inside the library).
"""
import ctypes
import os
import threading

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnormfwd.so")

NORMFWD_OK = 0
STATUS_NAMES = {0: "NORMFWD_OK", 1: "NORMFWD_ERR_INVALID", 2: "NORMFWD_ERR_UNSUPPORTED",
                3: "NORMFWD_ERR_WORKSPACE", 4: "NORMFWD_ERR_HIP", 5: "NORMFWD_ERR_INCOMPLETE"}

# Every symbol include/normfwd.h declares, with (restype, argtypes).
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t
_ST = ctypes.c_int
SIGNATURES = {
    "normfwd_status_string": (ctypes.c_char_p, [_ST]),
    "normfwd_last_error": (ctypes.c_char_p, []),
    "normfwd_time_next_kernel": (_ST, [_P, _P]),
    "ln_forward_workspace_size": (_SZ, [_I64, _I64]),
    "ln_forward_workspace_init": (_ST, [_P, _SZ, _P]),
    "ln_forward_workspace_check": (_ST, [_P, _SZ, _P]),
    "ln_forward": (_ST, [_P, _P, _P, _P, _I64, _I64, _F, _P, _SZ, _P, _P, ctypes.c_int, _P]),
    "ln_forward_noalloc": (_ST, [_P, _P, _P, _P, _I64, _I64, _F, _P, _P, ctypes.c_int, _P]),
    "ln_forward_stats": (_ST, [_P, _I64, _I64, _F, _P, _SZ, _P, _P, _P]),
    "ln_forward_apply": (_ST, [_P, _P, _P, _P, _I64, _I64, _P, _SZ, _P]),
    "gn_lrelu_x2_forward": (_ST, [_P, _P, _P, _P, _I64, _I64, _I64, _F, _F, _P, _P, _P]),
    "rmsnorm_ch_forward": (_ST, [_P, _P, _I64, _I64, _I64, _F, _P]),
    "rmsnorm_ch_forward_strided": (_ST, [_P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _I64, _F, _P, _P]),
    "normfwd_copy_reference": (_ST, [_P, _P, _I64, _I64, _I64, ctypes.c_int, _P]),
    "fc_gn_forward_workspace_size": (_SZ, [_I64, _I64, _I64]),
    "fc_gn_forward": (_ST, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _F, _F, _P, _SZ, _P, _P, _P]),
}

_LIB = None


class NormFwdError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")


def lib():
    """The loaded library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m normalization_ln_forward_amd.build` "
                               "(hipcc, gfx950)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def _check(status):
    if status != NORMFWD_OK:
        raise NormFwdError(status, lib().normfwd_last_error().decode())


_tls = threading.local()  # .capture: list of recorded calls while prepare() runs on this thread


def _invoke(name, *args):
    """Call C entry point `name`, or record the marshalled call while prepare() runs on this thread."""
    capture = getattr(_tls, "capture", None)
    if capture is not None:
        capture.append((name, args))
        return
    _check(getattr(lib(), name)(*args))


def prepare(fn, *args, **kwargs):
    """Validate and marshal one call of a binding function once; return a
    zero-argument callable that re-issues the same C call(s) (same tensors,
    same stream) with no Python-side checks.  For tight launch loops, where
    per-call argument checking would otherwise cost more host time than the
    kernels take on the GPU."""
    if getattr(_tls, "capture", None) is not None:
        raise RuntimeError("prepare() calls do not nest")
    _tls.capture = []
    try:
        out = fn(*args, **kwargs)
    finally:
        calls, _tls.capture = _tls.capture, None
    handle = lib()
    bound = [(getattr(handle, name), a) for name, a in calls]

    def run():
        for f, a in bound:
            st = f(*a)
            if st != NORMFWD_OK:
                _check(st)
        return out

    return run


def _event_handle(ev):
    if ev is None:
        return None
    h = int(getattr(ev, "cuda_event", 0) or 0)
    if h == 0:
        raise ValueError("event has no HIP event yet: record it once (torch creates events lazily)")
    return ctypes.c_void_p(h)


def time_next_kernel(start, stop):
    """Arm two torch.cuda.Event objects (timing enabled, each recorded once so that it exists) for the next
    kernel the library launches from this thread; see normfwd_time_next_kernel in include/normfwd.h.
    Inside prepare() the arming is recorded like any other call, so the prepared closure re-arms it."""
    _invoke("normfwd_time_next_kernel", _event_handle(start), _event_handle(stop))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t, name, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _opt(t, name, numel, device):
    if t is None:
        return
    _need(t, name, device)
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


def alloc_workspace(nbytes, device):
    """A 256-byte aligned uint8 device buffer of at least nbytes (returned as (buffer, view))."""
    nbytes = max(int(nbytes), 256)
    buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf, buf[off:off + nbytes]


# ---------------------------------------------------------------- LayerNorm

_LN_WS = {}


def release_cached_workspaces():
    """Drop the workspaces the binding keeps per shape (LayerNorm) and per device (fc + GroupNorm).  For an
    orderly end of a process that used them: call it once the device is idle (prepared calls that captured
    a released workspace must not run afterwards; later ordinary calls allocate new ones)."""
    _LN_WS.clear()
    _FC_WS.clear()


def ln_forward_workspace_size(outer, inner):
    return int(lib().ln_forward_workspace_size(outer, inner))


def ln_forward_workspace_init(workspace):
    _check(lib().ln_forward_workspace_init(_ptr(workspace), workspace.numel(), _stream(workspace.device)))


def ln_forward_workspace_check(workspace):
    """Raise NormFwdError (NORMFWD_ERR_INCOMPLETE) if a single-kernel call that used ``workspace``
    since the last check gave up waiting; waits for the current stream, then clears the record."""
    _check(lib().ln_forward_workspace_check(_ptr(workspace), workspace.numel(), _stream(workspace.device)))


def _ln_shape(x, normalized_ndim):
    nd = x.dim() - 1 if normalized_ndim is None else int(normalized_ndim)
    if not 0 <= nd <= x.dim():
        raise ValueError("normalized_ndim out of range")
    inner = 1
    for s in x.shape[x.dim() - nd:]:
        inner *= s
    outer = x.numel() // inner if inner else 0
    return outer, inner


def _ln_workspace(device, outer, inner):
    """A cached workspace per (device, outer, inner), zeroed once by ln_forward_workspace_init.

    A workspace is left ready for the next call of the same shape only (its
    counters sit at offsets that depend on the shape), so shapes do not share
    one; the cache keeps every workspace alive for the life of the process,
    which prepared calls that captured its address rely on."""
    key = (device, int(outer), int(inner))
    hit = _LN_WS.get(key)
    if hit is None:
        buf, view = alloc_workspace(ln_forward_workspace_size(outer, inner), device)
        ln_forward_workspace_init(view)
        hit = (buf, view)
        _LN_WS[key] = hit
    return hit[1]


def ln_forward(x, weight=None, bias=None, eps=1e-5, normalized_ndim=None, variant=3, out=None,
               workspace=None, mean_out=None, rstd_out=None):
    """LayerNorm over the trailing ``normalized_ndim`` dims (default: all but dim 0).

    ``variant`` 0 = split (moments kernel + normalize kernel), 1 = single
    kernel (control wave, tagged exchange; x read once), 2 = single cooperative
    kernel in which the last workgroup of each sample merges it, 3 (default) =
    the library's choice (1 wherever it can run: float4 rows, aligned tensors; else 0).  A caller-provided ``workspace`` must have been passed
    through ``ln_forward_workspace_init`` once.  Returns ``out`` (allocated if
    None).
    """
    _need(x, "x")
    dev = x.device
    outer, inner = _ln_shape(x, normalized_ndim)
    _opt(weight, "weight", inner, dev)
    _opt(bias, "bias", inner, dev)
    _opt(mean_out, "mean_out", outer, dev)
    _opt(rstd_out, "rstd_out", outer, dev)
    y = torch.empty_like(x) if out is None else out
    _need(y, "out", dev)
    if y.shape != x.shape:
        raise ValueError("out must have x's shape")
    ws = _ln_workspace(dev, outer, inner) if workspace is None else workspace
    _invoke("ln_forward", _ptr(x), _ptr(weight), _ptr(bias), _ptr(y), outer, inner, float(eps), _ptr(ws),
                            ws.numel() * ws.element_size(), _ptr(mean_out), _ptr(rstd_out), int(variant),
                            _stream(dev))
    return y


def ln_forward_noalloc(x, weight=None, bias=None, eps=1e-5, normalized_ndim=None, variant=3, out=None,
                       mean_out=None, rstd_out=None):
    """ln_forward on the library's own static scratch instead of a workspace (no device allocation in the
    library; ``out`` is still allocated here when None).  Calls that may overlap on one GPU race on that
    scratch; shapes whose workspace exceeds it raise NORMFWD_ERR_UNSUPPORTED."""
    _need(x, "x")
    dev = x.device
    outer, inner = _ln_shape(x, normalized_ndim)
    _opt(weight, "weight", inner, dev)
    _opt(bias, "bias", inner, dev)
    _opt(mean_out, "mean_out", outer, dev)
    _opt(rstd_out, "rstd_out", outer, dev)
    y = torch.empty_like(x) if out is None else out
    _need(y, "out", dev)
    if y.shape != x.shape:
        raise ValueError("out must have x's shape")
    _invoke("ln_forward_noalloc", _ptr(x), _ptr(weight), _ptr(bias), _ptr(y), outer, inner, float(eps),
            _ptr(mean_out), _ptr(rstd_out), int(variant), _stream(dev))
    return y


def ln_forward_stats(x, eps=1e-5, normalized_ndim=None, workspace=None, mean_out=None, rstd_out=None):
    """Partial-moment and merge kernels only; returns the workspace holding the statistics."""
    _need(x, "x")
    dev = x.device
    outer, inner = _ln_shape(x, normalized_ndim)
    _opt(mean_out, "mean_out", outer, dev)
    _opt(rstd_out, "rstd_out", outer, dev)
    ws = _ln_workspace(dev, outer, inner) if workspace is None else workspace
    _invoke("ln_forward_stats", _ptr(x), outer, inner, float(eps), _ptr(ws), ws.numel() * ws.element_size(),
                                  _ptr(mean_out), _ptr(rstd_out), _stream(dev))
    return ws


def ln_forward_apply(x, weight, bias, workspace, normalized_ndim=None, out=None):
    """Normalize kernel only, from statistics left in ``workspace`` by ln_forward_stats."""
    _need(x, "x")
    dev = x.device
    outer, inner = _ln_shape(x, normalized_ndim)
    _opt(weight, "weight", inner, dev)
    _opt(bias, "bias", inner, dev)
    y = torch.empty_like(x) if out is None else out
    _need(y, "out", dev)
    _invoke("ln_forward_apply", _ptr(x), _ptr(weight), _ptr(bias), _ptr(y), outer, inner, _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(dev))
    return y


# ---------------------------------------------------------------- GroupNorm + LeakyReLU + x2

def _gn_stats(mean_out, rstd_out, N, G, dev):
    if (mean_out is None) != (rstd_out is None):
        raise ValueError("give both mean_out and rstd_out, or neither")
    _opt(mean_out, "mean_out", N * G, dev)
    _opt(rstd_out, "rstd_out", N * G, dev)


def gn_lrelu_x2_forward(x, gamma, beta, num_groups, eps=1e-5, negative_slope=0.01, out=None, mean_out=None,
                        rstd_out=None):
    """GroupNorm(num_groups) on [N, C], then LeakyReLU(negative_slope), then x + x.  ``mean_out`` and
    ``rstd_out`` ([N, num_groups], both or neither) receive each (row, group)'s statistics."""
    _need(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be [N, C]")
    N, C = x.shape
    dev = x.device
    _opt(gamma, "gamma", C, dev)
    _opt(beta, "beta", C, dev)
    _gn_stats(mean_out, rstd_out, N, int(num_groups), dev)
    y = torch.empty_like(x) if out is None else out
    _need(y, "out", dev)
    _invoke("gn_lrelu_x2_forward", _ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), N, C, int(num_groups),
                                     float(eps), float(negative_slope), _ptr(mean_out), _ptr(rstd_out), _stream(dev))
    return y


# ---------------------------------------------------------------- RMSNorm over dim 1

def _rms_strides(t, name):
    """(batch stride, channel stride) of a [B, C, *spatial] view whose spatial block is contiguous."""
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    expect = 1
    for d in range(t.dim() - 1, 1, -1):
        if t.shape[d] != 1 and t.stride(d) != expect:
            raise ValueError(f"{name}: the dims after dim 1 must be contiguous (a batch or channel stride is fine)")
        expect *= t.shape[d]
    return t.stride(0), t.stride(1)


def rmsnorm_ch_forward(x, eps=1e-5, out=None, rstd_out=None):
    """y = x / sqrt(mean over dim 1 of x^2 + eps) for x of shape [B, C, *spatial].

    x (and ``out``) may be strided in dims 0 and 1 (a channel slice, a batch-strided view) as long as the
    trailing dims are contiguous; ``rstd_out`` ([B, *spatial], contiguous) receives 1 / rms per position.
    Contiguous tensors without ``rstd_out`` go through rmsnorm_ch_forward, the rest through
    rmsnorm_ch_forward_strided."""
    if not isinstance(x, torch.Tensor):
        raise TypeError("x must be a torch.Tensor")
    if x.dim() < 2:
        raise ValueError("x must have at least 2 dims")
    B, C = x.shape[0], x.shape[1]
    S = x.numel() // (B * C) if B * C else 0
    xsb, xsc = _rms_strides(x, "x")
    y = torch.empty_like(x, memory_format=torch.contiguous_format) if out is None else out
    if y.shape != x.shape:
        raise ValueError("out must have x's shape")
    if y.device != x.device:
        raise ValueError(f"out is on {y.device}, expected {x.device}")
    ysb, ysc = _rms_strides(y, "out")
    if rstd_out is not None:
        _need(rstd_out, "rstd_out", x.device)
        if rstd_out.numel() != B * S:
            raise ValueError(f"rstd_out has {rstd_out.numel()} elements, expected {B * S}")
    if x.is_contiguous() and y.is_contiguous() and rstd_out is None:
        _invoke("rmsnorm_ch_forward", _ptr(x), _ptr(y), B, C, S, float(eps), _stream(x.device))
    else:
        _invoke("rmsnorm_ch_forward_strided", _ptr(x), _ptr(y), B, C, S, xsb, xsc, ysb, ysc, float(eps),
                _ptr(rstd_out), _stream(x.device))
    return y


# ---------------------------------------------------------------- fc + GroupNorm epilogue

_FC_WS = {}


def fc_gn_forward(x, W, b, gamma, beta, num_groups, eps=1e-5, negative_slope=0.01, out=None, workspace=None,
                  mean_out=None, rstd_out=None):
    """h = x W^T + b (fp32 on the matrix cores), then gn_lrelu_x2_forward on h (``mean_out`` and ``rstd_out``:
    h's (row, group) statistics, [N, num_groups], both or neither)."""
    _need(x, "x")
    _need(W, "W", x.device)
    if x.dim() != 2 or W.dim() != 2 or x.shape[1] != W.shape[1]:
        raise ValueError("x must be [N, K] and W [C, K]")
    N, K = x.shape
    C = W.shape[0]
    dev = x.device
    _opt(b, "b", C, dev)
    _opt(gamma, "gamma", C, dev)
    _opt(beta, "beta", C, dev)
    _gn_stats(mean_out, rstd_out, N, int(num_groups), dev)
    y = torch.empty((N, C), dtype=torch.float32, device=dev) if out is None else out
    _need(y, "out", dev)
    nbytes = int(lib().fc_gn_forward_workspace_size(N, K, C))
    if workspace is None:
        hit = _FC_WS.get(dev)
        if hit is None or hit[1].numel() < nbytes:
            hit = alloc_workspace(nbytes, dev)
            _FC_WS[dev] = hit
        workspace = hit[1]
    _invoke("fc_gn_forward", _ptr(x), _ptr(W), _ptr(b), _ptr(gamma), _ptr(beta), _ptr(y), N, K, C,
                               int(num_groups), float(eps), float(negative_slope), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _ptr(mean_out), _ptr(rstd_out),
                               _stream(dev))
    return y


# ---------------------------------------------------------------- measurement references

def copy_reference(src, out, pattern=0):
    """A plain copy src -> out with one of the library's access patterns (normfwd_copy_reference):
    0 = dense streaming copy, 1 = rmsnorm_ch_forward's pattern on src viewed as [B, C, *spatial]."""
    _need(src, "src")
    _need(out, "out", src.device)
    if out.shape != src.shape:
        raise ValueError("out must have src's shape")
    if pattern == 1:
        if src.dim() < 2:
            raise ValueError("pattern 1 needs [B, C, *spatial]")
        B, C = src.shape[0], src.shape[1]
        S = src.numel() // (B * C)
    else:
        B, C, S = 1, 1, src.numel()
    _invoke("normfwd_copy_reference", _ptr(src), _ptr(out), B, C, S, int(pattern), _stream(src.device))
    return out
