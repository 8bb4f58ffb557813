"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU): the library's sources are compiled with both sanitizers on their
host pass (the device code as usual), linked with tests/abi_host_check.cpp,
and run.  The check program makes only calls
that validation rejects, or pure workspace-size queries, so no kernel is
launched; any sanitizer report aborts it."""
import os
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bwd_rope_apply_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["api.hip", "prep.hip", "simt.hip", "f32mfma.hip", "mfma.hip", "gram.hip", "noalloc.hip"]
# every -fsanitize applies to the host pass alone
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_validation_under_asan_ubsan():
    with tempfile.TemporaryDirectory() as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, src + ".o")
            r = subprocess.run([HIPCC, *FLAGS, *SAN, "-c", os.path.join(CSRC, src), "-o", obj],
                               capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-3000:]
            return obj

        with ThreadPoolExecutor(4) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        drv = os.path.join(tmp, "abi_host_check.o")
        r = subprocess.run([HIPCC, *FLAGS, *SAN, "-x", "hip",
                            os.path.join(ROOT, "tests", "abi_host_check.cpp"), "-c", "-o", drv],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        exe = os.path.join(tmp, "abi_host_check")
        r = subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN, drv, *objs, "-o", exe],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
        print(r.stdout, r.stderr[-3000:])
        assert r.returncode == 0, r.stdout + r.stderr[-3000:]
        assert "0 failed" in r.stdout
        assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
