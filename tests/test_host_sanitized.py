"""The C ABI's host code built with AddressSanitizer and UndefinedBehaviorSanitizer (host side only:
-Xarch_host on every sanitizer flag, the gfx950 device code is built as usual) and driven by
tests/abi_host_check.cpp: workspace sizing of every workload shape, argument errors of every call
(each must be reported before any device work), the stochastic-length and LITM planners on random
inputs.  Runs on the CPU; any sanitizer report fails the test."""
import hashlib
import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "target_cross_attention_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "abi_host_check.cpp")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


def _flags():
    return ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
            "-packed-fp32-ops", f"-I{os.path.join(ROOT, 'include')}",
            "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def test_abi_host_code_under_sanitizers():
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    h = hashlib.sha256()
    for p in srcs + [DRIVER] + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hpp")]:
        with open(p, "rb") as f:
            h.update(f.read())
    out = os.path.join(tempfile.gettempdir(), f"stca_host_check_{h.hexdigest()[:16]}")
    exe = os.path.join(out, "abi_host_check")
    if not os.path.exists(exe):
        os.makedirs(out, exist_ok=True)

        def compile_one(src):
            obj = os.path.join(out, os.path.basename(src) + ".o")
            r = subprocess.run([hipcc, *_flags(), "-c", src, "-o", obj], capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-4000:]
            return obj

        with ThreadPoolExecutor(min(8, len(os.sched_getaffinity(0)))) as ex:
            objs = list(ex.map(compile_one, srcs))
        r = subprocess.run([hipcc, *_flags(), "-x", "hip", DRIVER, "-x", "none", *objs, "-o", exe + ".tmp"],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        os.replace(exe + ".tmp", exe)
    nm = shutil.which("nm")
    if nm:   # the host objects really carry the sanitizers' instrumentation
        syms = subprocess.run([nm, exe], capture_output=True, text=True).stdout
        assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0, r.stderr[-4000:]
    assert "abi host checks passed" in r.stdout
