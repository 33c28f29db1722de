"""C ABI checks that need no GPU: exports, status codes, workspace sizing and the host-side
argument validation (every error below is returned before any device work is enqueued, so
placeholder device addresses are never dereferenced)."""
import ctypes
import os
import re
import sys

import pytest

import stca_inputs as SI
from target_cross_attention_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000  # 16-byte aligned placeholder device address (never dereferenced)


def header_functions():
    txt = open(os.path.join(ROOT, "include", "stca.h")).read()
    return sorted(set(re.findall(r"STCA_API\s+(?:const\s+)?\w+\s*\*?\s*(stca_\w+)\s*\(", txt)))


def test_every_declared_function_is_exported():
    names = header_functions()
    assert len(names) >= 14
    assert set(names) == set(B.EXPORTS)
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_debug_build_exports_the_same_calls():
    """libstca_debug.so (kernels with index checks) exports every declared call too; the ordinary
    build reports that it does not check, with no device work (callable without a GPU)."""
    assert os.path.exists(B.DEBUG_LIB_PATH), "build() also builds the debug library"
    dbg = ctypes.CDLL(B.DEBUG_LIB_PATH)
    for n in header_functions():
        assert hasattr(dbg, n), n
    if os.path.realpath(B.LIB_PATH) != os.path.realpath(B.DEBUG_LIB_PATH):
        assert B.debug_flags() == (0, False)
    f = ctypes.c_uint32(0)
    assert B.LIB.stca_debug_flags(None, None, 0) == -1
    assert B.LIB.stca_debug_flags(ctypes.byref(f), None, 1) == 0


def test_status_strings_and_version():
    assert B.status_string(0) == "ok"
    for code in (-1, -2, -3, -4, -5):
        assert B.status_string(code) != "unknown status"
    assert "gfx950" in B.version()


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        B._load()


def _fake_weights(M, with_wc=True):
    w = B.WeightsC()
    for i in range(M):
        w.hist[i] = B.Ffn(FAKE, FAKE, FAKE, FAKE, FAKE)
        w.query[i] = B.Ffn(FAKE, FAKE, FAKE, FAKE, FAKE)
        w.WQ[i] = w.WK[i] = w.WV[i] = w.WO[i] = FAKE
        w.WC[i] = FAKE if (with_wc and i >= 1) else None
    return w


def _batch(n=4, L=100, T=3, max_L=None, max_T=None):
    return B.BatchC(n, FAKE, FAKE, n * L, n * T, L if max_L is None else max_L, T if max_T is None else max_T)


def _forward(dims, w, batch, X=FAKE, xt=FAKE, Z=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return B.LIB.stca_forward(ctypes.byref(dims) if dims is not None else None, ctypes.byref(w),
                              ctypes.byref(batch), X, xt, Z, ws, ws_bytes, None)


def test_workspace_sizes():
    cfg = SI.get_config("dense10k")
    dims = B.dims_for(cfg)
    b = _batch(n=1024, L=10000, T=16)
    fw = B.forward_workspace_size(dims, b)
    aw = B.attend_workspace_size(dims, b)
    ew = B.encode_workspace_size(dims, 10_240_000)
    # the forward holds one encoded history (sum L x d bf16) plus the attention workspace
    assert fw >= 10_240_000 * 256 * 2 + aw
    assert ew == (4 * 256 // 32) * (3 * 256 // 16) * 1024  # packed weights only
    assert B.forward_workspace_size(dims, _batch(n=2048, L=10000, T=16)) > fw
    f32 = B.make_dims(64, 4, 1, 2, "f32")
    assert B.encode_workspace_size(f32, 256) > 0


@pytest.mark.parametrize("change,code", [
    (dict(d=96), -2), (dict(d=0), -2), (dict(h=3), -2), (dict(h=0), -2), (dict(r=0), -2), (dict(r=9), -2),
    (dict(M=0), -2), (dict(M=9), -2), (dict(dtype=7), -2), (dict(ln_eps=0.0), -2), (dict(attn_chunk=33), -2),
    (dict(attn_chunk=-32), -2), (dict(encode_layers=3), -2), (dict(encode_layers=-1), -2),
])
def test_forward_rejects_bad_dims(change, code):
    kw = dict(d=256, h=8, M=3, r=4, dtype="bf16", ln_eps=1e-5, attn_chunk=0)
    dt = change.pop("dtype", None)
    kw.update(change)
    dims = B.make_dims(**kw)
    if dt is not None:
        dims.dtype = dt
    assert _forward(dims, _fake_weights(3), _batch()) == code
    assert B.last_error()


def test_forward_rejects_bad_pointers_and_sizes():
    dims = B.make_dims(256, 8, 3, 4)
    w = _fake_weights(3)
    b = _batch()
    assert B.LIB.stca_forward(None, ctypes.byref(w), ctypes.byref(b), FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == -1
    assert _forward(dims, w, b, X=None) == -1
    assert _forward(dims, w, b, Z=None) == -1
    assert _forward(dims, w, b, X=FAKE + 8) == -4
    assert _forward(dims, w, b, ws=FAKE + 4) == -4
    assert _forward(dims, w, b, ws_bytes=1024) == -3
    assert _forward(dims, w, b, ws=None) == -3
    w2 = _fake_weights(3, with_wc=False)
    assert _forward(dims, w2, b) == -1
    w3 = _fake_weights(3)
    w3.hist[1] = B.Ffn(FAKE, FAKE, FAKE + 2, FAKE, FAKE)
    assert _forward(dims, w3, b) == -4
    w4 = _fake_weights(3)
    w4.hist[0] = B.Ffn(FAKE, FAKE, FAKE, None, FAKE)  # history LayerNorm needs gamma
    assert _forward(dims, w4, b) == -1
    # the layer-1.. query FFN has no LayerNorm unless query_ln: gamma may be NULL there
    w5 = _fake_weights(3)
    w5.query[1] = B.Ffn(FAKE, FAKE, FAKE, None, None)
    assert _forward(dims, w5, b, ws_bytes=1024) == -3  # passes weight checks, fails on workspace
    dims_qln = B.make_dims(256, 8, 3, 4, query_ln=True)
    assert _forward(dims_qln, w5, b) == -1


def test_forward_rejects_inconsistent_batch():
    dims = B.make_dims(256, 8, 3, 4)
    w = _fake_weights(3)
    assert _forward(dims, w, _batch(max_L=50)) == -1         # max_L * n < total_L
    assert _forward(dims, w, _batch(max_T=1)) == -1          # max_T * n < total_T
    assert _forward(dims, w, _batch(max_L=1000)) == -1       # max_L > total_L
    assert _forward(dims, w, B.BatchC(-1, FAKE, FAKE, 0, 0, 0, 0)) == -1
    assert _forward(dims, w, B.BatchC(2, None, FAKE, 10, 2, 5, 1)) == -1
    assert _forward(dims, w, B.BatchC(2, FAKE + 8, FAKE, 10, 2, 5, 1)) == -4
    assert _forward(dims, w, B.BatchC(0, None, None, 5, 0, 0, 0)) == -1


def test_forward_with_no_targets_is_a_no_op():
    dims = B.make_dims(256, 8, 3, 4)
    b = B.BatchC(2, FAKE, FAKE, 10, 0, 5, 0)
    need = B.forward_workspace_size(dims, b)
    assert _forward(dims, _fake_weights(3), b, ws_bytes=need) == 0


def test_encode_and_attend_validation():
    dims = B.make_dims(128, 8, 2, 2)
    ffn = B.Ffn(FAKE, FAKE, FAKE, FAKE, FAKE)
    L = B.LIB
    assert L.stca_encode(ctypes.byref(dims), ctypes.byref(ffn), -1, FAKE, FAKE, FAKE, 1 << 30, None) == -1
    assert L.stca_encode(ctypes.byref(dims), ctypes.byref(ffn), 10, FAKE + 2, FAKE, FAKE, 1 << 30, None) == -4
    assert L.stca_encode(ctypes.byref(dims), ctypes.byref(ffn), 10, FAKE, FAKE, FAKE, 16, None) == -3
    assert L.stca_encode(ctypes.byref(dims), ctypes.byref(ffn), 0, FAKE, FAKE, FAKE, 1 << 30, None) == 0
    w = _fake_weights(2)
    b = _batch()
    for layer in (-1, 2):
        assert L.stca_attend(ctypes.byref(dims), ctypes.byref(w), layer, ctypes.byref(b), FAKE, FAKE, FAKE, FAKE,
                             1 << 40, None) == -1
    assert L.stca_attend(ctypes.byref(dims), ctypes.byref(w), 0, ctypes.byref(b), FAKE, FAKE, FAKE, FAKE, 64,
                         None) == -3


def test_predict_validation():
    dims = B.make_dims(128, 8, 3, 2)
    ffn = B.Ffn(FAKE, FAKE, FAKE, None, None)   # eq. (9) has no LayerNorm: gamma/beta may be NULL
    L = B.LIB
    n = ctypes.c_size_t(0)
    assert L.stca_predict_workspace_size(ctypes.byref(dims), 1000, ctypes.byref(n)) == 0
    # c (T x d fp32) plus the generic FFN scratch (two T x rd fp32 blocks)
    assert n.value >= 1000 * 128 * 4 + 2 * 1000 * 256 * 4
    assert L.stca_predict_workspace_size(ctypes.byref(dims), -1, ctypes.byref(n)) == -1

    def call(WZ=FAKE, ffn_=ffn, T=10, Z=FAKE, xt=FAKE, z=FAKE, ws=FAKE, wsb=1 << 40):
        return L.stca_predict(ctypes.byref(dims), WZ, ctypes.byref(ffn_) if ffn_ is not None else None, T, Z, xt, z,
                              ws, wsb, None)
    assert call(WZ=None) == -1
    assert call(ffn_=None) == -1
    assert call(ffn_=B.Ffn(FAKE, None, FAKE, None, None)) == -1
    assert call(T=-1) == -1
    assert call(Z=None) == -1
    assert call(z=FAKE + 4) == -4
    assert call(WZ=FAKE + 2) == -4
    assert call(wsb=64) == -3
    assert call(T=0) == 0            # no targets: nothing enqueued
    bad = B.make_dims(128, 8, 3, 2)
    bad.d = 96
    assert L.stca_predict(ctypes.byref(bad), FAKE, ctypes.byref(ffn), 10, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                          None) == -2


def test_profiler_lifecycle_without_launches():
    p = B.Profiler()
    p.reset()
    rep = p.read()
    assert set(rep) == set(B.PHASE_NAMES)
    assert all(v == (0.0, 0) for v in rep.values())
    p.close()


def test_one_hip_runtime_in_process():
    """libstca binds to the HIP runtime torch already loaded (one copy per process)."""
    maps = open("/proc/self/maps").read().splitlines()
    hip = {ln.split()[-1] for ln in maps if "libamdhip64" in ln}
    hsa = {ln.split()[-1] for ln in maps if "libhsa-runtime64" in ln}
    assert len(hip) == 1 and len(hsa) == 1, (hip, hsa)


def _fake_grads(M, query_ln=False):
    g = B.GradsC()
    g.dX = g.dxt = FAKE
    for i in range(M):
        g.hist[i] = B.FfnGrad(FAKE, FAKE, FAKE, FAKE, FAKE)
        ln = FAKE if (i == 0 or query_ln) else None
        g.query[i] = B.FfnGrad(FAKE, FAKE, FAKE, ln, ln)
        g.dWQ[i] = g.dWK[i] = g.dWV[i] = g.dWO[i] = FAKE
        g.dWC[i] = FAKE if i >= 1 else None
    return g


def _backward(dims, w, batch, g, X=FAKE, xt=FAKE, dZ=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return B.LIB.stca_backward(ctypes.byref(dims), ctypes.byref(w), ctypes.byref(batch), X, xt, dZ,
                               ctypes.byref(g) if g is not None else None, ws, ws_bytes, None)


def test_backward_validation():
    dims = B.make_dims(256, 8, 3, 4)
    w, batch, g = _fake_weights(3), _batch(), _fake_grads(3)
    need = B.backward_workspace_size(dims, batch)
    # M x total_L x d fp32 encoded histories dominate the workspace
    assert need >= 3 * 400 * 256 * 4
    assert _backward(B.make_dims(96, 8, 3, 4), w, batch, g) == -2
    assert _backward(dims, w, batch, None) == -1
    bad = _fake_grads(3)
    bad.dWC[2] = None
    assert _backward(dims, w, batch, bad) == -1
    bad = _fake_grads(3)
    bad.query[1] = B.FfnGrad(FAKE, None, FAKE, None, None)
    assert _backward(dims, w, batch, bad) == -1
    bad = _fake_grads(3)
    bad.hist[2] = B.FfnGrad(FAKE, FAKE, FAKE, FAKE, FAKE + 8)
    assert _backward(dims, w, batch, bad) == -4
    # the query LayerNorm slots of layers >= 1 are needed once eq. (7) applies the LayerNorm
    ln = B.make_dims(256, 8, 3, 4, query_ln=True)
    assert _backward(ln, w, batch, _fake_grads(3)) == -1
    assert _backward(dims, w, batch, g, X=None) == -1
    assert _backward(dims, w, batch, g, dZ=FAKE + 4) == -4
    assert _backward(dims, w, batch, g, ws=None) == -3
    assert _backward(dims, w, batch, g, ws_bytes=need - 1) == -3
    assert _backward(dims, _fake_weights(3, with_wc=False), batch, g) == -1
    assert _backward(dims, w, B.BatchC(4, FAKE, FAKE, 400, 1 << 23, 100, 1 << 21), g) == -1


def test_forward_graph_validation():
    """Graph capture checks its arguments before recording anything (no device work here)."""
    dims = B.make_dims(256, 8, 2, 4)
    w, batch = _fake_weights(2), _batch()
    out = ctypes.c_void_p()
    g = B.LIB.stca_forward_graph_create
    assert g(ctypes.byref(dims), ctypes.byref(w), ctypes.byref(batch), FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == -1
    assert g(ctypes.byref(B.make_dims(96, 8, 2, 4)), ctypes.byref(w), ctypes.byref(batch), FAKE, FAKE, FAKE, FAKE,
             1 << 40, ctypes.byref(out)) == -2
    assert g(ctypes.byref(dims), ctypes.byref(w), ctypes.byref(batch), FAKE, FAKE, FAKE, FAKE, 16,
             ctypes.byref(out)) == -3
    assert g(ctypes.byref(dims), ctypes.byref(w), ctypes.byref(batch), None, FAKE, FAKE, FAKE, 1 << 40,
             ctypes.byref(out)) == -1
    assert g(ctypes.byref(dims), ctypes.byref(w), ctypes.byref(batch), FAKE, FAKE, FAKE + 4, FAKE, 1 << 40,
             ctypes.byref(out)) == -4
    assert g(ctypes.byref(dims), ctypes.byref(_fake_weights(2, with_wc=False)), ctypes.byref(batch), FAKE, FAKE,
             FAKE, FAKE, 1 << 40, ctypes.byref(out)) == -1
    assert out.value is None
    assert B.LIB.stca_graph_destroy(None) == 0
    assert B.LIB.stca_graph_launch(None, None) == -1


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: a request for several exits with status 2 and says why, before
    touching a device."""
    import json
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_bench_traffic_summary(tmp_path, monkeypatch):
    """bench.py --traffic-summary scales the counters by the copy calibration and records the
    encode's and the attention's bytes per launch with their source hashes."""
    import csv
    import json
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import bench
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]

    def write(d, counter, rows):
        os.makedirs(d, exist_ok=True)
        with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
            w = csv.writer(f)
            w.writerow(cols)
            for i, (k, v) in enumerate(rows):
                w.writerow([i, k, counter, v])

    enc, att = "encode_pair_kernel<256>", "void stca::attend_mfma_kernel<256>(...)"
    write(tmp_path / "f", "FETCH_SIZE", [(enc, 1000.0), (enc, 3000.0), (att, 500.0), ("other", 7.0)])
    write(tmp_path / "w", "WRITE_SIZE", [(enc, 2000.0), (enc, 2000.0), (att, 100.0), ("other", 1.0)])
    # a 2 GiB copy that reads back half its bytes (factor 2) and writes all of them (factor 1)
    write(tmp_path / "cf", "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 4.0), ("__amd_rocclr_copyBuffer", 1 << 20)])
    write(tmp_path / "cw", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 1 << 21)])
    rec_file = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(rec_file))
    bench.traffic_summary("ragged", str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"),
                          str(tmp_path / "cw"))
    rec = json.loads(rec_file.read_text())["ragged"]
    assert rec["encode"]["bytes_per_launch"] == int(2000 * 1024 * 2 + 2000 * 1024)
    assert rec["attend"]["bytes_per_launch"] == int(500 * 1024 * 2 + 100 * 1024)
    assert rec["encode"]["source_hash"] == bench.kernel_source_hash(["encode_mfma.hip", "device_common.hpp"])
    assert bench.measured_traffic("ragged", "attend", ["attend.hip", "device_common.hpp"]) == \
        rec["attend"]["bytes_per_launch"]


def test_bench_metric_names_the_workload():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import bench
    import stca_inputs as SI
    assert bench.metric_for(SI.get_config("dense10k")) == \
        "STCA fwd history-tokens/s at L=10k; achieved HBM GB/s & MFMA % of peak"
    for key in ("tiny", "uniform", "ragged", "stress20k"):
        m = bench.metric_for(SI.get_config(key))
        assert key in m and "L=10k" not in m


def test_bench_attention_roof_follows_the_intensity():
    """The attention is priced against HBM below the ridge (2500 TFLOP/s over 8000 GB/s = 312.5 FLOP/B)
    and against the MFMA peak above it; the intensity of a workload is 2 m h FLOP per byte of X~."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import bench
    d, L = 256, 1000
    for m, h, bound in ((16, 8, "hbm"), (32, 16, "mfma"), (6, 8, "hbm")):
        flops, nbytes = 4.0 * h * d * L * m, 2.0 * d * L
        assert flops / nbytes == 2 * m * h
        b, unit, peak, achieved, ridge, _ = bench.attention_roof(flops, nbytes, 1e-3, bf16=True)
        assert ridge == 312.5 and b == bound
        if bound == "hbm":
            assert (unit, peak) == ("GB/s", bench.PEAK_HBM_GBS) and achieved == nbytes / 1e-3 / 1e9
        else:
            assert (unit, peak) == ("TFLOP/s", bench.PEAK_BF16_TFLOPS) and achieved == flops / 1e-3 / 1e12
    # fp32 (4 bytes per element): the ridge is the fp32 peak over HBM, about 19.7 FLOP/B
    b, _, peak, _, ridge, _ = bench.attention_roof(4.0 * 4 * 64 * 256 * 4, 4.0 * 64 * 256, 1e-3, bf16=False)
    assert b == "hbm" and abs(ridge - 157.3 / 8) < 1e-9


def test_variant_build_needs_an_output_path():
    """A build with compile-time macros never replaces libstca.so: it is refused without --out."""
    from target_cross_attention_amd import build as Bd
    with pytest.raises(ValueError):
        Bd.build(defines=("STCA_ENC_RING=3",))


def test_forward_workspace_holds_every_layer_when_encodes_share_a_launch():
    """encode_layers = 2 (all history encodes in one launch) keeps M encoded buffers, 1 keeps one;
    automatic picks the single launch only where one layer's X~ exceeds 1 GiB at d <= 256."""
    import numpy as np
    for key, auto_fused in [("dense10k", True), ("ragged", False), ("uniform", False), ("stress20k", False)]:
        cfg = SI.get_config(key)
        L, m = SI.batch_layout(cfg)
        hist = np.concatenate([[0], np.cumsum(L)]).astype(np.int64)
        tgt = np.concatenate([[0], np.cumsum(m)]).astype(np.int64)
        c = B.BatchC(cfg.n_users, FAKE, FAKE + 4096, int(hist[-1]), int(tgt[-1]), int(L.max()), int(m.max()))
        sizes = {k: B.forward_workspace_size(B.dims_for(cfg, encode_layers=k), c) for k in (0, 1, 2)}
        xt = int(hist[-1]) * cfg.d * 2
        assert sizes[2] - sizes[1] == (cfg.M - 1) * xt
        assert sizes[0] == (sizes[2] if auto_fused else sizes[1])
