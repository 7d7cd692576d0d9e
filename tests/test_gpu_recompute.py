"""The control-wave LayerNorm kernel runs as an ordinary launch (ln_forward variant 1, and variant 2 when not
in place): when a workgroup's published sums do not arrive (it is not resident), the others compute them
from x with the same bits (variant 2: a sample no merger announces, since that workgroup never arrives, is
merged by whoever waited for it).  A child process forces that path for every k-th workgroup
(NORMFWD_LN_FORCE_RECOMPUTE=k, read once by the library: those workgroups publish and count nothing) and
the results must equal this process's normal results bit for bit, and the oracle."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
import normalization_ln_forward_amd as nf
from normalization_ln_forward_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
import recompute_child  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("k", [4, 1])
def test_forced_recompute_is_bitwise_equal(k, tmp_path):
    path = str(tmp_path / f"forced_{k}.npz")
    env = dict(os.environ, NORMFWD_LN_FORCE_RECOMPUTE=str(k))
    print(f"forced recompute k={k}: child", flush=True)
    r = subprocess.run([sys.executable, os.path.join(HERE, "recompute_child.py"), path], capture_output=True,
                       text=True, timeout=300, env=env)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    forced = np.load(path)
    normal = recompute_child.run_cases()  # this process: no knob, nothing recomputed
    # k = 4 forces workgroups 3, 7, ...: none in the 3-workgroup case
    n_cases = len(recompute_child.CASES)
    for v in recompute_child.VARIANTS:
        assert sum(int(forced[f"recomputed_v{v}_{o}x{i}"]) > 0 for o, i, _, _ in recompute_child.CASES) >= (
            n_cases if k == 1 else n_cases - 1), v
    for (outer, inner, seed, name), v in [(c, v) for c in recompute_child.CASES for v in recompute_child.VARIANTS]:
        tag = f"v{v}_{outer}x{inner}"
        assert int(normal[f"recomputed_{tag}"]) == 0, f"{tag}: a healthy launch recomputed sums"
        for key in ("y", "mean", "rstd"):
            a, b = forced[f"{key}_{tag}"], normal[f"{key}_{tag}"]
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{tag} {key}: forced != normal"
        if k == 4:
            d = synth.make(name, device="cuda", shape=(outer, inner), normalized_ndim=1, seed=seed)
            ref = oracle.ln(*(d[t].cpu().numpy() for t in ("x", "weight", "bias")))
            rep = oracle.allclose_report(forced[f"y_{tag}"], ref, 1e-4, 1e-4)
            assert rep["ok"], f"{tag}: {rep}"
        torch.cuda.empty_cache()
