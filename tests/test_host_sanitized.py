"""The library's host code (argument checks, tree layout, workspace sizing) built with
AddressSanitizer and UndefinedBehaviorSanitizer and driven by tests/host_check/
host_check.cpp at the long-context shapes (1M + 8192 and 2M tokens at fanout 64,
twenty-level trees, the widest parent-major fanout).  The kernels are compiled as
usual (the sanitizers apply to the host side only) but never launched: every call
the driver makes fails or answers on the host, so this runs on the CPU."""
import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_recsa_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "host_check")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _hipcc():
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    pytest.skip("hipcc not found")


def test_host_code_under_sanitizers():
    hipcc = _hipcc()
    os.makedirs(OUT, exist_ok=True)
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *SAN,
              f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [
        os.path.join(ROOT, "tests", "host_check", "host_check.cpp")]

    def compile_one(src):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        r = subprocess.run([hipcc, *common, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with ThreadPoolExecutor(8) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = os.path.join(OUT, "host_check")
    r = subprocess.run([hipcc, "--offload-arch=gfx950", *SAN, *objs, "-o", exe], capture_output=True,
                       text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-5000:]
    assert "host checks passed" in r.stdout
