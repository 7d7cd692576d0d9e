"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, no GPU): libnormfwd with its
host code instrumented (each sanitizer flag given to hipcc after -Xarch_host, so device code is built as
usual) and the CPU oracle (built by ROCm's clang, whose sanitizer runtime the library's host code needs), driven by tests/c/sanitize_driver.c through every validation path of the C ABI,
the empty-work no-ops and small problems of every oracle function."""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "normalization_ln_forward_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")
# the C parts are built by ROCm's clang as well, so one sanitizer runtime serves the library and the driver
CLANG = "/opt/rocm/llvm/bin/clang"

pytestmark = pytest.mark.skipif(HIPCC is None or not os.path.exists(CLANG), reason="needs hipcc and ROCm's clang")

SAN = "address,undefined"


def test_host_code_and_oracle_under_sanitizers(tmp_path):
    from normalization_ln_forward_amd import build as nbuild

    d = str(tmp_path)

    def one(src):
        obj = os.path.join(d, os.path.splitext(src)[0] + ".o")
        subprocess.run([HIPCC, *nbuild.compile_flags(), "-O1", "-g", "-Xarch_host", f"-fsanitize={SAN}",
                        "-Xarch_host", "-fno-omit-frame-pointer", "-c", os.path.join(CSRC, src), "-o", obj],
                       check=True, capture_output=True)
        return obj

    with cf.ThreadPoolExecutor(max_workers=6) as ex:
        objs = list(ex.map(one, nbuild.SOURCES))
    lib = os.path.join(d, "libnormfwd.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", f"-fsanitize={SAN}", *objs,
                    "-o", lib], check=True, capture_output=True)
    orc = os.path.join(d, "oracle.o")
    subprocess.run([CLANG, "-std=c11", "-O1", "-g", "-fno-fast-math", "-ffp-contract=off", f"-fsanitize={SAN}",
                    "-fPIC", "-c", os.path.join(ROOT, "oracle", "oracle.c"), "-o", orc], check=True)
    exe = os.path.join(d, "sanitize_driver")
    subprocess.run([CLANG, "-std=c11", "-O1", "-g", f"-fsanitize={SAN}", f"-I{ROOT}/include",
                    os.path.join(ROOT, "tests", "c", "sanitize_driver.c"), orc, "-o", exe, f"-L{d}", "-lnormfwd",
                    "-L/opt/rocm/lib", "-lamdhip64", "-lm", f"-Wl,-rpath,{d}:/opt/rocm/lib"], check=True)
    # the library's host code really is instrumented (it imports the sanitizer runtime's report hooks)
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "sanitize_driver: ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
