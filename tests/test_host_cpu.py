"""Host-side logic without a GPU: input generators, binding argument checks, oracle determinism."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import normalization_ln_forward_amd as nf
from normalization_ln_forward_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_synth_is_seeded_and_has_the_stated_distributions():
    a = synth.make("ln_16x64x256x256", shape=(4, 4096), normalized_ndim=1, seed=5)
    b = synth.make("ln_16x64x256x256", shape=(4, 4096), normalized_ndim=1, seed=5)
    c = synth.make("ln_16x64x256x256", shape=(4, 4096), normalized_ndim=1, seed=6)
    assert torch.equal(a["x"], b["x"]) and torch.equal(a["weight"], b["weight"])
    assert not torch.equal(a["x"], c["x"])
    x = a["x"].double()
    assert abs(x.mean().item()) < 0.05 and abs(x.std().item() - 1) < 0.05
    assert abs(a["weight"].double().mean().item() - 1) < 0.01
    assert abs(a["weight"].double().std().item() - 0.1) < 0.01
    s = synth.make("ln_stress_16x64x256x256", shape=(2, 65536), normalized_ndim=1)["x"].double()
    assert abs(s.mean().item() - 100) < 1e-3 and abs(s.std().item() - 0.01) < 1e-3
    f = synth.make("fc_gn_1024x8192x8192", shape=(8, 256), hidden=512)
    bound = 1 / np.sqrt(256)
    assert f["W"].shape == (512, 256) and float(f["W"].abs().max()) <= bound
    assert float(f["W"].double().std()) == pytest.approx(bound / np.sqrt(3), rel=0.05)
    g = synth.make("gn_lrelu_x2_1024x8192", shape=(2, 64))
    assert g["gamma"].shape == (64,) and g["num_groups"] == 512


def test_workloads_carry_the_problem_parameters():
    w = synth.WORKLOADS
    assert w["gn_lrelu_x2_1024x8192"].params == {"num_groups": 512, "eps": 1e-5, "negative_slope": 0.01}
    assert w["ln_16x64x256x256"].shape == (16, 64, 256, 256)
    assert w["rms_ch_112x64x512x512"].shape == (112, 64, 512, 512)
    assert w["ln_stress_16x64x256x256"].x_dist == ("normal", 100.0, 0.01)
    assert [synth.default_seed(n) for n in synth.ORDER] == [1000, 1001, 1002, 1003, 1004]


def test_binding_rejects_bad_tensors_before_calling_the_library():
    x = torch.zeros(4, 8)
    with pytest.raises(ValueError, match="GPU"):
        nf.ln_forward(x)
    with pytest.raises(TypeError, match="float32"):
        nf.rmsnorm_ch_forward(torch.zeros(2, 3, 4, dtype=torch.float64))
    with pytest.raises(TypeError):
        nf.gn_lrelu_x2_forward([1.0], None, None, 1)


def test_oracle_does_not_depend_on_the_thread_count():
    code = ("import sys; sys.path.insert(0, %r); import numpy as np, oracle; "
            "x = np.random.default_rng(0).standard_normal((6, 50000)).astype(np.float32); "
            "y = oracle.ln(x); g = oracle.gn_lrelu_x2(x[:, :4000], None, None, 250); "
            "r = oracle.rms_ch(x.reshape(6, 10, 5000)); "
            "sys.stdout.buffer.write(y.tobytes() + g.tobytes() + r.tobytes())" % ROOT)
    outs = []
    for threads in ("1", "4"):
        env = dict(os.environ, OMP_NUM_THREADS=threads)
        outs.append(subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, check=True).stdout)
    assert outs[0] == outs[1] and len(outs[0]) > 0


def test_prepare_records_only_its_own_thread_and_does_not_nest():
    """prepare() records the C calls its function makes on the calling thread (other threads' calls go
    straight to the library), re-issues them when run, and refuses to nest."""
    import threading

    from normalization_ln_forward_amd import _lib

    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("library not built")
    seen = []

    def fn():
        _lib._invoke("normfwd_time_next_kernel", None, None)
        t = threading.Thread(target=lambda: seen.append(getattr(_lib._tls, "capture", None)))
        t.start()
        t.join()
        return 7

    run = _lib.prepare(fn)
    assert seen == [None]
    assert run() == 7 and run() == 7
    with pytest.raises(RuntimeError):
        _lib.prepare(lambda: _lib.prepare(fn))
    assert getattr(_lib._tls, "capture", None) is None
