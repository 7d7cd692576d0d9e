"""The single-read LayerNorm kernel's exchange tags (csrc/ln_tag.hpp, host and device are the same code),
checked on the CPU by tests/c/ln_tag_test.hip: no generation's tag accepts a zeroed word or an element
count (what the other schedules leave in the shared slots), and consecutive generations never share a tag."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "ln_tag_test.hip")
CSRC = os.path.join(ROOT, "normalization_ln_forward_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")

pytestmark = pytest.mark.skipif(HIPCC is None, reason="hipcc not available")


def test_tags_reject_other_writers_words(tmp_path):
    exe = str(tmp_path / "ln_tag_test")
    subprocess.run([HIPCC, "-O1", "-std=c++17", "--offload-arch=gfx950", f"-I{CSRC}", SRC, "-o", exe],
                   check=True, capture_output=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ln_tag_test: ok" in r.stdout
