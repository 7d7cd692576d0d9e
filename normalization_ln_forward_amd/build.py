"""Build libnormfwd.so (the HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Every translation unit under csrc/ is compiled with
  -O3 --offload-arch=gfx950 -std=c++17 -fPIC
  -Xclang -target-feature -Xclang -packed-fp32-ops   (no packed fp32 VALU ops)
plus the per-file flags in EXTRA_FLAGS, and linked into
normalization_ln_forward_amd/libnormfwd.so.  No fast-math: sqrt and division
stay correctly rounded.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libnormfwd.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

SOURCES = ["api.hip", "ln.hip", "gn.hip", "rms.hip", "fc.hip", "ref.hip"]

# ln.hip: LLVM's AMDGPU atomic optimizer off.  Every atomic in ln.hip is
# issued by a single lane; the optimizer rewrites each one into a wave-wide
# form that broadcasts the returned value right after the atomic, so the wave
# waits out the atomic's round trip where it issues it.  The last-workgroup-
# merges control wave counts its arrival at a sample an iteration ahead so
# that this round trip overlaps the iteration (with the optimizer, each
# control wave waited for it before publishing its moments: 108-114 us per
# call at [16, 4M], 105-107 us without).
EXTRA_FLAGS = {"ln.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libnormfwd)")


def compile_flags(defines=()):
    return ["-O3", f"--offload-arch={ARCH}", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-I{INCLUDE}", f"-I{CSRC}", *[f"-D{d}" for d in defines]]


def build(out=LIB, defines=(), build_dir=BUILD_DIR, verbose=False, jobs=8) -> str:
    cc = hipcc()
    os.makedirs(build_dir, exist_ok=True)
    objs = []

    def one(src):
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *compile_flags(defines), *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        # hipcc's host pass does not know the packed-fp32 feature name; that warning is expected
        err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{err}")
        if err.strip() and verbose:
            print(err, file=sys.stderr)
        return obj

    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = out + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
