import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library through its C ABI")


def pytest_collection_modifyitems(session, config, items):
    """Tests that drive the GPU from a child process (the plain-C program, a short bench.py run) run
    first.  The runtime grants cooperative launches on a GPU to one process at a time (after the test
    process has made one, a child's is refused until the test process exits; ln_forward variant 2 then
    returns NORMFWD_ERR_UNSUPPORTED), so running these children first lets the plain-C program exercise
    variant 2 too; it passes either way.  (The batching, recompute and planted children make no
    cooperative launch.)"""
    first = ("test_c_abi.py", "test_bench_contract.py")
    child = [it for it in items if any(f in it.nodeid for f in first)]
    rest = [it for it in items if not any(f in it.nodeid for f in first)]
    items[:] = child + rest
