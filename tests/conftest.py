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
    first.  The last-workgroup-merges LayerNorm kernel (variant 2) uses a cooperative launch; after the
    test process had made one, a child's cooperative launch on the same GPU was refused
    (hipErrorIllegalState) on MI355X, so these children run before any such launch here.  (The batching
    and recompute children make no cooperative launch.)"""
    first = ("test_c_abi.py", "test_bench_contract.py")
    child = [it for it in items if any(f in it.nodeid for f in first)]
    rest = [it for it in items if not any(f in it.nodeid for f in first)]
    items[:] = child + rest
