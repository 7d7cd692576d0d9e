"""Launch batching: with NORMFWD_MAX_GRID_ITEMS lowered (read once by the library, hence a child process),
every launcher splits its grid into launches of whole samples/rows, and the results still match the
oracle.  At real sizes the same code splits grids that would exceed HIP's 32-bit work-item count."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.gpu
def test_batched_launches_match_the_oracle():
    env = dict(os.environ, NORMFWD_MAX_GRID_ITEMS="65536")
    r = subprocess.run([sys.executable, os.path.join(HERE, "batching_child.py")], capture_output=True, text=True,
                       timeout=300, env=env)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "batching: ok" in r.stdout
