"""The C ABI library without a GPU: it loads, exports every declared symbol, and
rejects invalid arguments before touching the device."""
import ctypes
import os
import re

import pytest
import torch  # noqa: F401  (loads the HIP runtime the library binds to)

from normalization_ln_forward_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "normfwd.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libnormfwd.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


def test_header_and_binding_agree():
    assert declared_functions() == sorted(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = _lib.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    lib = _lib.lib()
    for code, name in _lib.STATUS_NAMES.items():
        assert lib.normfwd_status_string(code).decode().startswith(name)
    assert lib.normfwd_status_string(99).decode() == "unknown status"


FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: every call below fails validation first
FAKE_WS = ctypes.c_void_p(0x200000)  # 256-byte aligned


def _err(code):
    return code, _lib.lib().normfwd_last_error().decode()


def test_ln_validation():
    lib = _lib.lib()
    st, msg = _err(lib.ln_forward(None, None, None, FAKE, 2, 8, 1e-5, FAKE_WS, 1 << 20, None, None, 0, None))
    assert st == 1 and "NULL" in msg
    st, _ = _err(lib.ln_forward(FAKE, None, None, FAKE, 2, 0, 1e-5, FAKE_WS, 1 << 20, None, None, 0, None))
    assert st == 1  # normalizing over no elements
    st, _ = _err(lib.ln_forward(FAKE, None, None, FAKE, 2, -1, 1e-5, FAKE_WS, 1 << 20, None, None, 0, None))
    assert st == 1
    st, _ = _err(lib.ln_forward(FAKE, None, None, FAKE, 2, 8, 1e-5, FAKE_WS, 1 << 20, None, None, 7, None))
    assert st == 1
    st, _ = _err(lib.ln_forward(FAKE, None, None, FAKE, 2, 8, -1.0, FAKE_WS, 1 << 20, None, None, 0, None))
    assert st == 1
    need = lib.ln_forward_workspace_size(16, 4194304)
    assert need > 16 * 256 * 32
    st, msg = _err(lib.ln_forward(FAKE, None, None, FAKE, 16, 4194304, 1e-5, FAKE_WS, need - 1, None, None, 0,
                                  None))
    assert st == 3 and "needs" in msg
    st, _ = _err(lib.ln_forward(FAKE, None, None, FAKE, 16, 4194304, 1e-5, None, need, None, None, 0, None))
    assert st == 3
    st, _ = _err(lib.ln_forward(FAKE, None, None, FAKE, 16, 4194304, 1e-5, ctypes.c_void_p(0x200010), need,
                                None, None, 0, None))
    assert st == 3
    st, _ = _err(lib.ln_forward_stats(FAKE, 16, 4194304, 1e-5, FAKE_WS, 100, None, None, None))
    assert st == 3
    st, _ = _err(lib.ln_forward_apply(FAKE, None, None, None, 16, 4194304, FAKE_WS, need, None))
    assert st == 1
    assert lib.ln_forward_workspace_size(0, 5) == 0
    st, _ = _err(lib.ln_forward_workspace_init(None, 1024, None))
    assert st == 3
    st, _ = _err(lib.ln_forward_workspace_check(None, 1024, None))
    assert st == 3
    st, _ = _err(lib.ln_forward_workspace_check(ctypes.c_void_p(0x200010), 1024, None))
    assert st == 3
    st, _ = _err(lib.ln_forward_workspace_check(FAKE_WS, 255, None))
    assert st == 3


def test_ln_workspace_size_monotone():
    lib = _lib.lib()
    prev = 0
    for outer in (1, 2, 16, 100):
        s = lib.ln_forward_workspace_size(outer, 4194304)
        assert s > prev and s % 256 == 0
        prev = s


def test_gn_validation():
    lib = _lib.lib()
    st, msg = _err(lib.gn_lrelu_x2_forward(FAKE, None, None, FAKE, 4, 10, 3, 1e-5, 0.01, None, None, None))
    assert st == 1 and "multiple" in msg
    st, _ = _err(lib.gn_lrelu_x2_forward(None, None, None, FAKE, 4, 12, 3, 1e-5, 0.01, None, None, None))
    assert st == 1
    st, _ = _err(lib.gn_lrelu_x2_forward(FAKE, None, None, FAKE, -1, 12, 3, 1e-5, 0.01, None, None, None))
    assert st == 1
    st, _ = _err(lib.gn_lrelu_x2_forward(FAKE, None, None, FAKE, 4, 12, 0, 1e-5, 0.01, None, None, None))
    assert st == 1


def test_rms_validation():
    lib = _lib.lib()
    st, _ = _err(lib.rmsnorm_ch_forward(None, FAKE, 2, 3, 4, 1e-5, None))
    assert st == 1
    st, _ = _err(lib.rmsnorm_ch_forward(FAKE, FAKE, 2, 0, 4, 1e-5, None))
    assert st == 1
    st, _ = _err(lib.rmsnorm_ch_forward(FAKE, FAKE, 2, 3, 1 << 30, 1e-5, None))
    assert st == 2


def test_documented_size_limits_are_refused():
    """Each limit the header states is enforced before anything is launched (NORMFWD_ERR_UNSUPPORTED)."""
    lib = _lib.lib()
    big_ws = 1 << 62

    def ln(outer, inner):
        return _err(lib.ln_forward(FAKE, None, None, FAKE, outer, inner, 1e-5, FAKE_WS, big_ws, None, None, 0,
                                   None))[0]

    assert ln((1 << 22) + 1, 1) == 2          # samples
    assert ln(1, (1 << 31) + 4) == 2          # elements per sample
    assert ln(1 << 12, 1 << 29) == 2          # elements per tensor (2^41 > 2^40)

    def gn(N, C, G):
        return _err(lib.gn_lrelu_x2_forward(FAKE, None, None, FAKE, N, C, G, 1e-5, 0.01, None, None, None))[0]

    assert gn(1, 1 << 31, 1) == 2             # channels
    assert gn(1 << 12, 1 << 29, 1 << 20) == 2  # elements per tensor

    def rms(B, C, S):
        return _err(lib.rmsnorm_ch_forward(FAKE, FAKE, B, C, S, 1e-5, None))[0]

    assert rms(1, 1 << 31, 4) == 2            # channels
    assert rms(1, 3, (1 << 26) + 4) == 2      # positions per sample
    assert rms(1 << 12, 1 << 10, 1 << 20) == 2  # elements per tensor

    def fc(N, K, C, G):
        return _err(lib.fc_gn_forward(FAKE, FAKE, None, None, None, FAKE, N, K, C, G, 1e-5, 0.01, FAKE_WS, big_ws,
                                      None, None, None))[0]

    assert fc((1 << 23) + 1, 16, 64, 4) == 2  # rows
    assert fc(64, 16, (1 << 24) + 16, 16) == 2  # output channels


def test_fc_validation():
    lib = _lib.lib()
    need = lib.fc_gn_forward_workspace_size(1024, 8192, 8192)
    assert need == 1024 * 8192 * 4
    st, _ = _err(lib.fc_gn_forward(FAKE, FAKE, None, None, None, FAKE, 1024, 8192, 8192, 500, 1e-5, 0.01, FAKE_WS,
                                   need, None, None, None))
    assert st == 1
    st, _ = _err(lib.fc_gn_forward(FAKE, FAKE, None, None, None, FAKE, 1024, 8192, 8192, 512, 1e-5, 0.01, FAKE_WS,
                                   need - 4, None, None, None))
    assert st == 3
    st, _ = _err(lib.fc_gn_forward(FAKE, None, None, None, None, FAKE, 1024, 8192, 8192, 512, 1e-5, 0.01, FAKE_WS,
                                   need, None, None, None))
    assert st == 1
    # statistics: both outputs or neither
    st, msg = _err(lib.fc_gn_forward(FAKE, FAKE, None, None, None, FAKE, 1024, 8192, 8192, 512, 1e-5, 0.01,
                                     FAKE_WS, need, FAKE, None, None))
    assert st == 1 and "both" in msg
    st, msg = _err(lib.gn_lrelu_x2_forward(FAKE, None, None, FAKE, 4, 12, 3, 1e-5, 0.01, None, FAKE, None))
    assert st == 1 and "both" in msg


def test_empty_work_is_a_no_op_that_touches_nothing():
    """Empty batches return OK before any pointer is inspected or anything is launched (so this runs
    without a GPU): NULL everywhere, no workspace."""
    lib = _lib.lib()
    for variant in (0, 1, 2, 3):
        assert lib.ln_forward(None, None, None, None, 0, 4096, 1e-5, None, 0, None, None, variant, None) == 0
    assert lib.ln_forward(None, None, None, None, 0, 4096, 1e-5, None, 0, None, None, 4, None) != 0
    assert lib.ln_forward_stats(None, 0, 4096, 1e-5, None, 0, None, None, None) == 0
    assert lib.ln_forward_apply(None, None, None, None, 0, 4096, None, 0, None) == 0
    assert lib.gn_lrelu_x2_forward(None, None, None, None, 0, 8192, 512, 1e-5, 0.01, None, None, None) == 0
    assert lib.rmsnorm_ch_forward(None, None, 0, 64, 1024, 1e-5, None) == 0
    assert lib.rmsnorm_ch_forward(None, None, 3, 64, 0, 1e-5, None) == 0
    assert lib.fc_gn_forward(None, None, None, None, None, None, 0, 64, 128, 8, 1e-5, 0.01, None, 0, None, None, None) == 0
    # still invalid: a bad group count or a negative size
    assert lib.gn_lrelu_x2_forward(None, None, None, None, 0, 100, 7, 1e-5, 0.01, None, None, None) == 1
    assert lib.rmsnorm_ch_forward(None, None, -1, 64, 1024, 1e-5, None) == 1


def test_ln_noalloc_validation():
    """ln_forward_noalloc validates like ln_forward and refuses shapes whose workspace exceeds its static
    scratch, all before touching the device."""
    lib = _lib.lib()
    st, msg = _err(lib.ln_forward_noalloc(None, None, None, FAKE, 2, 8, 1e-5, None, None, 3, None))
    assert st == 1 and "NULL" in msg
    st, _ = _err(lib.ln_forward_noalloc(FAKE, None, None, FAKE, 2, 8, 1e-5, None, None, 4, None))
    assert st == 1
    st, _ = _err(lib.ln_forward_noalloc(FAKE, None, None, FAKE, 2, 8, -1.0, None, None, 3, None))
    assert st == 1
    assert lib.ln_forward_workspace_size(1024, 1 << 20) > (8 << 20)
    st, msg = _err(lib.ln_forward_noalloc(FAKE, None, None, FAKE, 1024, 1 << 20, 1e-5, None, None, 3, None))
    assert st == 2 and "scratch" in msg
    assert lib.ln_forward_noalloc(FAKE, None, None, FAKE, 0, 8, 1e-5, None, None, 3, None) == 0  # empty batch


def test_rms_strided_validation():
    """rmsnorm_ch_forward_strided refuses, before touching the device: negative strides, views that span
    2^40 elements, and y strides under which two of y's rows overlap."""
    lib = _lib.lib()
    f = lib.rmsnorm_ch_forward_strided
    st, _ = _err(f(None, FAKE, 2, 3, 4, 12, 4, 12, 4, 1e-5, None, None))
    assert st == 1
    st, _ = _err(f(FAKE, FAKE, 2, 3, 4, -12, 4, 12, 4, 1e-5, None, None))
    assert st == 2
    st, _ = _err(f(FAKE, FAKE, 2, 3, 4, 12, 4, 12, 3, 1e-5, None, None))  # y's channel rows overlap
    assert st == 1
    st, _ = _err(f(FAKE, FAKE, 2, 3, 4, 12, 4, 8, 4, 1e-5, None, None))   # y's samples overlap
    assert st == 1
    st, _ = _err(f(FAKE, FAKE, 2, 3, 4, 1 << 40, 4, 12, 4, 1e-5, None, None))  # x spans over 2^40
    assert st == 2
    st, _ = _err(f(FAKE, FAKE, 2, 3, 4, 12, 4, 12, 4, -1.0, None, None))
    assert st == 1
    assert f(None, None, 0, 3, 4, 12, 4, 12, 4, 1e-5, None, None) == 0  # no positions

