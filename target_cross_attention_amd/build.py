"""Build libstca.so (HIP for gfx950) in-tree with hipcc.

    python -m target_cross_attention_amd.build          # compile every source, link
    python -m target_cross_attention_amd.build --asm    # also write gfx950 assembly next to the objects
    python -m target_cross_attention_amd.build --debug-bounds   # libstca_debug.so: kernels check their
                                                                # ragged indices (STCA_DEBUG_BOUNDS)
    python -m target_cross_attention_amd.build --define STCA_ENC_STAGGER=0 --out /tmp/libstca_st0.so
        # a variant build with compile-time tuning macros set, for same-process comparisons
        # (bench.py --compare)
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libstca.so")
BUILD_DEBUG = os.path.join(PKG, "_build_debug")
LIB_DEBUG = os.path.join(PKG, "libstca_debug.so")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 add/mul/fma instructions.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-fvisibility=hidden", "-Wall", "-Wno-unused-function", f"-I{os.path.join(ROOT, 'include')}"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, asm: bool, debug_bounds: bool = False, bdir: str | None = None,
             defines: tuple[str, ...] = ()) -> str:
    bdir = bdir or (BUILD_DEBUG if debug_bounds else BUILD)
    obj = os.path.join(bdir, os.path.basename(src)[:-4] + ".o")
    cmd = [hipcc(), *FLAGS, *(["-DSTCA_DEBUG_BOUNDS"] if debug_bounds else []), *[f"-D{d}" for d in defines],
           "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if asm:
        s = os.path.join(BUILD, os.path.basename(src)[:-4] + f"-{ARCH}.s")
        subprocess.run([hipcc(), *FLAGS, "--cuda-device-only", "-S", src, "-o", s], check=True,
                       capture_output=True)
    return obj


def build(asm: bool = False, jobs: int | None = None, debug_bounds: bool = False,
          defines: tuple[str, ...] = (), out: str | None = None) -> str:
    """Compile every source and link.  With `defines` (NAME=VALUE macros, e.g. the encode's
    STCA_ENC_* tuning constants) the objects go to a build folder of their own and the library to
    `out`, so that a variant never replaces libstca.so."""
    if defines and not out:
        raise ValueError("a build with --define needs --out")
    bdir = BUILD_DEBUG if debug_bounds else BUILD
    if defines:
        bdir = os.path.join(PKG, "_build_variant", os.path.splitext(os.path.basename(out))[0])
    out = out or (LIB_DEBUG if debug_bounds else LIB)
    os.makedirs(bdir, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, asm and not debug_bounds and not defines, debug_bounds, bdir,
                                              tuple(defines)), srcs))
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", action="store_true")
    ap.add_argument("--debug-bounds", action="store_true")
    ap.add_argument("--define", action="append", default=[], metavar="NAME=VALUE",
                    help="compile-time macro for a variant build (repeatable; needs --out)")
    ap.add_argument("--out", default=None, help="library path of a variant build")
    a = ap.parse_args()
    print(build(asm=a.asm, debug_bounds=a.debug_bounds, defines=tuple(a.define), out=a.out))
    sys.exit(0)
