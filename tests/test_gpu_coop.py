"""The runtime grants cooperative launches on a GPU to one process at a time: once this process has made
one (ln_forward variant 2 in place), a child process's cooperative launch is refused while this process
lives.  The library turns that refusal into NORMFWD_ERR_UNSUPPORTED with a message naming the cause,
launches nothing for it, and the child's other calls keep working (variant 2 not in place is an ordinary
launch)."""
import os
import subprocess
import sys

import pytest
import torch

import normalization_ln_forward_amd as nf
from normalization_ln_forward_amd import synth

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def test_refused_cooperative_launch_is_reported_clearly():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    d = synth.make("ln_16x64x256x256", device="cuda", shape=(4, 1 << 18), normalized_ndim=1, seed=9)
    xi = d["x"].clone()
    nf.ln_forward(xi, d["weight"], d["bias"], variant=2, out=xi)  # this process now holds cooperative launches
    torch.cuda.synchronize()
    print("coop child", flush=True)
    r = subprocess.run([sys.executable, os.path.join(HERE, "coop_child.py")], capture_output=True, text=True,
                       timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    lines = dict(l.split(": ", 1) for l in r.stdout.splitlines() if l.startswith("variant "))
    assert lines["variant 2 in place"].startswith("status 2") and "cooperative launch" in lines["variant 2 in place"], \
        lines
    assert lines["variant 2"] == "status 0", lines
    assert lines["variant 1"] == "status 0", lines
