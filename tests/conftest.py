import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library through its C ABI")


def pytest_collection_modifyitems(session, config, items):
    """The plain-C program that drives the GPU from a child process runs first.  The last-workgroup-merges
    LayerNorm kernel (variant 2) uses a cooperative launch; after the test process had made one, the
    child's cooperative launch on the same GPU was refused (hipErrorIllegalState) on MI355X, so the child
    runs before any such launch here.  (The recompute child makes no cooperative launch.)"""
    child = [it for it in items if "test_c_abi.py" in it.nodeid]
    rest = [it for it in items if "test_c_abi.py" not in it.nodeid]
    items[:] = child + rest
