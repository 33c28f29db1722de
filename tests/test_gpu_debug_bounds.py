"""The debug build (libstca_debug.so, STCA_DEBUG_BOUNDS) on the GPU: its kernels check the indices
that ragged offsets and workspace plans drive, and record a failed check in a device word instead
of faulting.  A child process loads the debug build (STCA_LIB) and
  * records the self-test bit from a kernel and reads it back (the mechanism reports what it records),
  * runs forwards (one chunk per user and forced small chunks that go through the combine, d = 128,
    256 and 512, the single-launch multi-layer encode), a lone stca_attend and backwards on both
    precision paths over ragged batches, checking each against the CPU oracle,
  * and finds no check failed.
"""
import os
import subprocess
import sys

import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import numpy as np, torch
import stca_inputs as SI
from oracle import stca as O, grad as G
from stca_testlib import row_rel, tol_for
from target_cross_attention_amd import binding as B
assert B.LIB_PATH.endswith("libstca_debug.so"), B.LIB_PATH
dev = "cuda:0"
flags, enabled = B.debug_flags(clear=True)
assert enabled, "not the debug build"
B.debug_selftest()
flags, _ = B.debug_flags(clear=True)
assert flags == 0x80000000, hex(flags)
assert B.debug_flags(clear=True)[0] == 0
cases = [("ragged", dict(n_users=40), {}), ("ragged", dict(n_users=24), dict(attn_chunk=64)),
         ("uniform", dict(n_users=6), dict(attn_chunk=96)), ("dense10k", dict(n_users=3), dict(encode_layers=2)),
         ("stress20k", dict(n_users=2, length=("fixed", 1500)), dict(attn_chunk=512)),
         ("ragged", dict(n_users=12, dtype="f32", length=("lognormal", 300.0, 400.0, 1, 2000)), dict(attn_chunk=64))]
for key, change, kw in cases:
    cfg = SI.scaled(SI.get_config(key), **change)
    W = SI.make_weights(cfg); inp = SI.make_inputs(cfg)
    dw = B.DeviceWeights(W, cfg.dtype, dev); db = B.DeviceBatch(inp, dev)
    Z = B.stca_forward(B.dims_for(cfg, **kw), dw, db); torch.cuda.synchronize()
    err = row_rel(Z.cpu().numpy(), O.forward_batch(inp, W))
    f, _ = B.debug_flags(clear=True)
    print("forward", key, change, kw, "err %.3e" % err, "flags", hex(f), flush=True)
    assert err <= tol_for(cfg) and f == 0
for key, change in [("ragged", dict(n_users=5, length=("lognormal", 150.0, 200.0, 16, 600))),
                    ("ragged", dict(n_users=4, dtype="f32", length=("lognormal", 100.0, 150.0, 16, 400)))]:
    cfg = SI.scaled(SI.get_config(key), **change)
    W = SI.make_weights(cfg, random_ln=True); inp = SI.make_inputs(cfg)
    dZ = np.random.default_rng(5).standard_normal((inp.total_T, cfg.M, cfg.d)).astype(np.float32)
    g = B.stca_backward(B.dims_for(cfg), B.DeviceWeights(W, cfg.dtype, dev), B.DeviceBatch(inp, dev),
                        torch.from_numpy(dZ).to(dev))
    torch.cuda.synchronize()
    ref = G.backward_batch(inp, W, dZ.astype(np.float64))
    e = float(np.max(np.abs(g.dX[:inp.total_L].cpu().numpy() - ref.dX))) / float(np.max(np.abs(ref.dX)))
    f, _ = B.debug_flags(clear=True)
    print("backward", key, cfg.dtype, "dX err %.3e" % e, "flags", hex(f), flush=True)
    assert e <= (2e-2 if cfg.dtype == "bf16" else 1e-4) and f == 0
print("debug build: no check failed", flush=True)
"""


def test_debug_build_finds_no_index_out_of_range():
    lib = os.path.join(ROOT, "target_cross_attention_amd", "libstca_debug.so")
    if not os.path.exists(lib):
        pytest.skip("debug build missing")
    env = dict(os.environ, STCA_LIB=lib, PYTHONPATH=os.pathsep.join([ROOT, os.path.join(ROOT, "tests")]))
    print("[case] debug-bounds child process", flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    print(r.stdout[-3000:], r.stderr[-3000:], flush=True)
    assert r.returncode == 0
    assert "no check failed" in r.stdout
