"""STCA benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dense10k] [--no-cpu-baseline]
    python bench.py --backward [--workload ragged] [--no-keep]
    python bench.py --sl | --litm

Default mode: one step = one stca_forward over the whole batch (M history encodes, the query path
and M split-L attention passes).  Inputs are seeded synthetic data resident in HBM before timing.
Prints one JSON line (history tokens per second, whole job) with the roofline of the dominant
kernel (the encode), the attention's, the oracle timed on the host, the graph-replay time and the
prediction token of eq. (9).  --backward times stca_backward on the training-shaped batch, --sl a
stochastic-length batch and --litm a batch after local same-ID token merging.  --flush-cache evicts
the 256 MB Infinity Cache (a 512 MiB write) before every timed forward and times each forward
alone.  --vendor-gemm times the vendor library's bf16 GEMMs (torch.matmul) at the encode's shapes
instead, as a ceiling reference for the fused encode.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash(names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "target_cross_attention_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str, src_files):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match the current source."""
    try:
        with open(COUNTERS_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    e = rec.get(workload, {}).get(kernel)
    if not e or e.get("source_hash") != kernel_source_hash(src_files):
        return None
    return e.get("bytes_per_launch")


INFINITY_CACHE_BYTES = 256 << 20   # MI355X last-level cache (MALL)
DENSE10K_METRIC = "STCA fwd history-tokens/s at L=10k; achieved HBM GB/s & MFMA % of peak"


def metric_for(cfg) -> str:
    """The dense-inference workload carries the headline metric; every other workload names itself."""
    if cfg.key == "dense10k":
        return DENSE10K_METRIC
    return f"STCA fwd history-tokens/s ({cfg.key} workload)"


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(cfg, W, target_s: float = 12.0, max_users: int = 64):
    """The oracle, as it stands, on users of the same workload until ~target_s of CPU work."""
    import numpy as np
    import stca_inputs as SI
    from oracle import stca as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    L, m = SI.batch_layout(cfg)
    tokens = targets = 0
    users = 0
    t0 = time.perf_counter()
    elapsed = 0.0
    for u in range(min(cfg.n_users, max_users)):
        inp = SI.make_inputs(cfg, users=[u], threads=1)
        ts = time.perf_counter()
        O.forward_batch(inp, W)
        elapsed += time.perf_counter() - ts
        tokens += int(L[u])
        targets += int(m[u])
        users += 1
        if time.perf_counter() - t0 >= target_s:
            break
    return {"value": tokens / elapsed, "unit": "history-tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"{users} of {cfg.n_users} users ({tokens} history tokens, {targets} targets), "
                      f"numpy float64 per-user forward, {elapsed:.1f} s",
            "targets_per_s": targets / elapsed}


def bench_sl(a, cfg, dev):
    """Stochastic-length training batch from the workload's full histories: the host plan, the
    device suffix gather (timed against HBM), then the forward on the packed batch."""
    from types import SimpleNamespace

    import numpy as np
    import torch

    import stca_inputs as SI
    from target_cross_attention_amd import binding as B

    alpha, L_min, L_max, L_avg, L_infer = 0.02, 8, 10000, 2000, 10000
    prm = B.SlParams(L_min, L_max, L_avg, L_infer)
    W = SI.make_weights(cfg)
    inp = SI.make_inputs(cfg)
    s, order = SI.make_sl_draws(cfg, inp.n_users, alpha, B.sl_beta(prm, alpha))
    t = time.perf_counter()
    L, off = B.sl_plan(prm, inp.L, s, order)
    plan_ms = (time.perf_counter() - t) * 1e3
    total = int(off[-1])
    dims = B.dims_for(cfg, attn_chunk=a.attn_chunk, encode_layers=a.encode_layers)
    Xf = B.to_device(inp.X, cfg.dtype, dev)
    del inp.X
    full_off = torch.from_numpy(inp.hist_off.astype(np.int64)).to(dev)
    hist_off = torch.from_numpy(off).to(dev)
    Xp = torch.empty((total, cfg.d), dtype=Xf.dtype, device=dev)
    stream = torch.cuda.current_stream()
    B.sl_pack(dims, full_off, hist_off, total, int(L.max()), Xf, Xp, stream=stream)
    n_pack = max(a.steps, 5)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n_pack):
        B.sl_pack(dims, full_off, hist_off, total, int(L.max()), Xf, Xp, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    pack_ms = e0.elapsed_time(e1) / n_pack
    del Xf
    pack_bytes = 2.0 * total * cfg.d * (2 if cfg.dtype == "bf16" else 4)   # read + write each row

    tgt_off = torch.from_numpy(inp.tgt_off.astype(np.int64)).to(dev)
    xt = B.to_device(inp.xt, cfg.dtype, dev)
    T = int(inp.tgt_off[-1])
    batch = SimpleNamespace(X=Xp, xt=xt, total_T=T,
                            c=B.batch_struct(inp.n_users, hist_off, tgt_off, total, T, int(L.max()), int(inp.m.max())))
    dw = B.DeviceWeights(W, cfg.dtype, dev)
    ws = B.workspace(B.forward_workspace_size(dims, batch.c), dev)
    Z = torch.empty((T, cfg.M, cfg.d), dtype=torch.float32, device=dev)
    for _ in range(a.warmup):
        B.stca_forward(dims, dw, batch, Z=Z, ws=ws, stream=stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        B.stca_forward(dims, dw, batch, Z=Z, ws=ws, stream=stream)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    assert np.isfinite(Z.sum().item()), "non-finite output"
    print(json.dumps({
        "metric": "STCA fwd history-tokens/s on a stochastic-length batch",
        "value": total * a.steps / dt, "unit": "history-tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": dt * 1e3 / a.steps, "higher_is_better": True,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": f"stochastic-length batch from {cfg.description}", "alpha": alpha,
                   "L_min": L_min, "L_max": L_max, "L_avg": L_avg, "L_infer": L_infer, "users": inp.n_users,
                   "packed_tokens": total, "budget": inp.n_users * L_avg, "mean_len": float(L.mean()),
                   "users_at_L_max": int((L >= 8 * (L_max // 8)).sum())},
        "sl_plan_host_ms": plan_ms,
        "sl_pack": {"bound": "hbm", "avg_ms": pack_ms, "achieved": pack_bytes / pack_ms / 1e6,
                    "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": pack_bytes / pack_ms / 1e6 / PEAK_HBM_GBS,
                    "algorithmic_bytes_per_launch": pack_bytes},
    }))


def bench_litm(a, cfg, dev):
    """Local same-ID token merging of the workload's histories (its repeats carry shared item IDs):
    the host plan, the device merge (timed against HBM), then the forward on the merged batch."""
    from types import SimpleNamespace

    import numpy as np
    import torch

    import stca_inputs as SI
    from target_cross_attention_amd import binding as B

    T_gap = 3
    W = SI.make_weights(cfg)
    inp = SI.make_inputs(cfg, with_ids=True)
    t = time.perf_counter()
    mo, go, mem = B.litm_plan(inp.hist_off, inp.item_id, T_gap)
    plan_ms = (time.perf_counter() - t) * 1e3
    n_groups = len(go) - 1
    dims = B.dims_for(cfg, attn_chunk=a.attn_chunk, encode_layers=a.encode_layers)
    Xf = B.to_device(inp.X, cfg.dtype, dev)
    del inp.X
    god, memd = torch.from_numpy(go).to(dev), torch.from_numpy(mem).to(dev)
    Xm = torch.empty((n_groups, cfg.d), dtype=Xf.dtype, device=dev)
    stream = torch.cuda.current_stream()
    B.litm_merge(dims, god, memd, Xf, Xm, stream=stream)
    n_rep = max(a.steps, 5)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n_rep):
        B.litm_merge(dims, god, memd, Xf, Xm, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    merge_ms = e0.elapsed_time(e1) / n_rep
    del Xf
    row = cfg.d * (2 if cfg.dtype == "bf16" else 4)
    # every source row read once, every merged row written once, members and group offsets read
    merge_bytes = float(inp.total_L * row + n_groups * row + inp.total_L * 8 + (n_groups + 1) * 8)

    hist_off = torch.from_numpy(mo).to(dev)
    tgt_off = torch.from_numpy(inp.tgt_off.astype(np.int64)).to(dev)
    T = int(inp.tgt_off[-1])
    Lm = np.diff(mo)
    batch = SimpleNamespace(X=Xm, xt=B.to_device(inp.xt, cfg.dtype, dev), total_T=T,
                            c=B.batch_struct(inp.n_users, hist_off, tgt_off, n_groups, T, int(Lm.max()),
                                             int(inp.m.max())))
    dw = B.DeviceWeights(W, cfg.dtype, dev)
    ws = B.workspace(B.forward_workspace_size(dims, batch.c), dev)
    Z = torch.empty((T, cfg.M, cfg.d), dtype=torch.float32, device=dev)
    for _ in range(a.warmup):
        B.stca_forward(dims, dw, batch, Z=Z, ws=ws, stream=stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        B.stca_forward(dims, dw, batch, Z=Z, ws=ws, stream=stream)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    assert np.isfinite(Z.sum().item()), "non-finite output"
    print(json.dumps({
        "metric": "STCA fwd history-tokens/s after local same-ID token merging (tokens before merging)",
        "value": inp.total_L * a.steps / dt, "unit": "history-tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": dt * 1e3 / a.steps, "higher_is_better": True,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": f"LITM (T = {T_gap}) on {cfg.description}", "users": inp.n_users,
                   "tokens": inp.total_L, "merged_tokens": n_groups,
                   "merged_fraction": 1.0 - n_groups / inp.total_L},
        "merged_tokens_per_s": n_groups * a.steps / dt,
        "litm_plan_host_ms": plan_ms,
        "litm_merge": {"bound": "hbm", "avg_ms": merge_ms, "achieved": merge_bytes / merge_ms / 1e6,
                       "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": merge_bytes / merge_ms / 1e6 / PEAK_HBM_GBS,
                       "algorithmic_bytes_per_launch": merge_bytes},
    }))


def bench_backward(a, cfg, dev):
    """One training step's backward on the training-shaped ragged batch: stca_backward for an
    upstream dZ of the forward (the forward is recomputed inside the call), timed per phase with
    HIP events on the call's stream."""
    import numpy as np
    import torch

    import stca_inputs as SI
    from target_cross_attention_amd import binding as B

    W = SI.make_weights(cfg)
    inp = SI.make_inputs(cfg)
    log(f"inputs {cfg.key}: {inp.n_users} users, {inp.total_L} history tokens, {inp.total_T} targets")
    dims = B.dims_for(cfg)
    dw = B.DeviceWeights(W, cfg.dtype, dev)
    db = B.DeviceBatch(inp, dev)
    del inp.X
    dZ = torch.from_numpy(np.random.default_rng(11).standard_normal((db.total_T, cfg.M, cfg.d), np.float32)).to(dev)
    grads = B.DeviceGrads(dims, db.total_L, db.total_T, dev)
    mixed = cfg.dtype == "bf16"   # bf16 storage: the mixed-precision path
    keep = not a.no_keep and not mixed
    ws = B.workspace(B.backward_workspace_size(dims, db.c, keep), dev)
    stream = torch.cuda.current_stream()
    log(f"backward workspace {ws.numel() / 2**30:.2f} GiB; warmup {a.warmup}")
    for _ in range(a.warmup):
        B.stca_backward(dims, dw, db, dZ, grads, ws=ws, stream=stream)
    torch.cuda.synchronize()
    log(f"timing {a.steps} steps")
    prof = B.Profiler()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        B.stca_backward(dims, dw, db, dZ, grads, ws=ws, stream=stream, profiler=prof)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    phases = prof.read()
    prof.close()
    assert np.isfinite(grads.dX.sum().item()), "non-finite gradient"
    L, T, d, r, M, h = db.total_L, db.total_T, cfg.d, cfg.r, cfg.M, cfg.h
    pairs = float((db.inp.L * db.inp.m).sum()) * h
    # Dominant phase: the derivative of eq. (2) over the history rows, one per layer.  Algorithmic
    # FLOP per history token: the products dW_o, dH, dW_u, dW_v, dx (12 r d^2, 2 FLOP per
    # multiply-add), plus, unless the fp32 path's keep workspace holds them, the recomputed
    # A = x W_u, G = x W_v and Y = H W_o (6 r d^2).
    enc_ms, enc_n = phases["bwd_encode"]
    enc_avg_s = enc_ms / max(enc_n, 1) / 1e3
    enc_flops = (12.0 if keep else 18.0) * r * d * d * L
    achieved = enc_flops / enc_avg_s / 1e12
    peak = PEAK_BF16_TFLOPS if mixed else PEAK_FP32_TFLOPS
    # Per (target, head, history token) pair: the scores twice (statistics, then again for alpha), abar,
    # dA, du and the two products of dX~, each 2d FLOP.
    att_layer_ms = phases["bwd_attend"][0] / a.steps / M
    out = {
        "metric": "STCA backward history-tokens/s (gradients of every weight, X and x_t)",
        "value": L * a.steps / dt, "unit": "history-tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": dt * 1e3 / a.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if mixed else "f32",
        "precision": ("mixed: bf16 operands, fp32 accumulation (encode and attention derivatives); LayerNorm "
                      "and softmax statistics, weight-gradient sums and per-target steps in fp32" if mixed
                      else "fp32 throughout"),
        "data": "synthetic (seeded; training-shaped ragged batch)",
        "config": {"workload": cfg.description, "key": cfg.key, "users": db.inp.n_users, "history_tokens": L,
                   "targets": T, "storage": cfg.dtype,
                   "workspace": ("keep (encode intermediates kept from the recompute)" if keep else
                                 "mixed path (encode recomputed per row chunk)" if mixed else "minimum"),
                   "workspace_gib": ws.numel() / 2**30},
        "roofline": {"kernel": ("encode backward (bf16 matrix-core GEMMs with fused SwiGLU epilogues, fp32 "
                                "LayerNorm derivative)" if mixed else
                                "encode backward (fp32 matrix-core GEMMs + SwiGLU/LayerNorm derivatives)"),
                     "bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": None,
                     "algorithmic_flops_per_launch": enc_flops, "avg_launch_ms": enc_avg_s * 1e3,
                     "launches": enc_n},
        "attention_backward": {"kernels": ("ragged per-user bf16 matrix-core products (fp32 operands rounded as "
                                           "they are staged) + softmax/dS row passes" if mixed else
                                           "ragged per-user fp32 matrix-core products + softmax/dS row passes"),
                               "ms_per_layer": att_layer_ms, "pairs_per_layer": pairs, "bound": "mfma",
                               "achieved": 14.0 * d * pairs / (att_layer_ms / 1e3) / 1e12,
                               "peak": PEAK_BF16_TFLOPS if mixed else PEAK_FP32_TFLOPS, "unit": "TFLOP/s"},
        "phase_ms_per_step": {k: v[0] / a.steps for k, v in phases.items() if k.startswith("bwd")},
    }
    if not a.no_cpu_baseline:
        log("cpu baseline (gradient oracle on a user sample)")
        out["cpu_baseline"] = cpu_baseline_backward(cfg, W)
    print(json.dumps(out))


def cpu_baseline_backward(cfg, W, target_s: float = 12.0, max_users: int = 64):
    """The gradient oracle, as it stands, on users of the same workload until ~target_s of CPU work."""
    import numpy as np
    import stca_inputs as SI
    from oracle import grad as G
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    L, m = SI.batch_layout(cfg)
    rng = np.random.default_rng(3)
    tokens = users = 0
    elapsed = 0.0
    t0 = time.perf_counter()
    for u in range(min(cfg.n_users, max_users)):
        inp = SI.make_inputs(cfg, users=[u], threads=1)
        dZ = rng.standard_normal((inp.total_T, cfg.M, cfg.d))
        ts = time.perf_counter()
        G.backward_batch(inp, W, dZ)
        elapsed += time.perf_counter() - ts
        tokens += int(L[u])
        users += 1
        if time.perf_counter() - t0 >= target_s:
            break
    return {"value": tokens / elapsed, "unit": "history-tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"{users} of {cfg.n_users} users ({tokens} history tokens), numpy float64 per-user "
                      f"backward (oracle.grad), {elapsed:.1f} s"}


# Kernels whose HBM traffic the bench line reports: role -> (name fragment, source files).
TRAFFIC_KERNELS = {"encode": (("encode_",), ["encode_mfma.hip", "device_common.hpp"]),
                   "attend": (("attend_mfma_kernel", "attend16_kernel"), ["attend.hip", "device_common.hpp"])}


def attention_roof(flops: float, nbytes: float, seconds: float, bf16: bool):
    """The roof that binds one attention launch: (bound, unit, peak, achieved, ridge, mfma peak).

    The intensity is 2 m h FLOP per byte of X~ (m targets of h heads per user, averaged over the
    batch).  Below the ridge, peak FLOP/s over peak HBM bytes/s, the launch is HBM-bound and priced
    against the HBM peak; above it against the MFMA peak of its dtype (stress20k: 2 x 32 x 16 =
    1024 FLOP/B against a 312.5 FLOP/B bf16 ridge)."""
    mfma_peak = PEAK_BF16_TFLOPS if bf16 else PEAK_FP32_TFLOPS
    ridge = mfma_peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    if flops / nbytes > ridge:
        return "mfma", "TFLOP/s", mfma_peak, flops / seconds / 1e12, ridge, mfma_peak
    return "hbm", "GB/s", PEAK_HBM_GBS, nbytes / seconds / 1e9, ridge, mfma_peak


def _counter_rows(d: str, counter: str):
    """(kernel name, value) per dispatch from a rocprofv3 --pmc run's counter_collection.csv under d."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    out = []
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return out


def traffic_summary(workload: str, fetch_dir: str, write_dir: str, cfetch_dir: str, cwrite_dir: str,
                    copy_bytes: int = 2 << 30):
    """Markdown table of HBM bytes per dispatch from two counter passes (FETCH_SIZE, WRITE_SIZE, KiB
    per dispatch), each scaled by what the same counter reads for a plain device copy of copy_bytes
    (bench.py --calib-copy); records the encode's and the attention's bytes per launch in
    profiles/hbm_traffic.txt with the current source hash of each kernel."""
    from collections import defaultdict

    def per_kernel(rows):
        acc = defaultdict(list)
        for k, v in rows:
            acc[k].append(v)
        return {k: (len(v), sum(v) / len(v)) for k, v in acc.items()}

    def calib(d, counter):
        vals = [v for k, v in _counter_rows(d, counter) if "copyBuffer" in k]
        return copy_bytes / (max(vals) * 1024.0)   # the 2 GiB copies are the largest copy dispatches

    fs, ws = calib(cfetch_dir, "FETCH_SIZE"), calib(cwrite_dir, "WRITE_SIZE")
    fetch = per_kernel(_counter_rows(fetch_dir, "FETCH_SIZE"))
    write = per_kernel(_counter_rows(write_dir, "WRITE_SIZE"))
    lines = [f"Calibration: a {copy_bytes >> 30} GiB device copy gives bytes = FETCH_SIZE x 1024 x {fs:.3f} and "
             f"WRITE_SIZE x 1024 x {ws:.3f}.", "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read GB (scaled) | HBM write GB (scaled) |",
             "|---|---|---|---|---|---|"]
    for k in sorted(fetch, key=lambda k: -fetch[k][1]):
        n, fv = fetch[k]
        wv = write.get(k, (0, 0.0))[1]
        lines.append(f"| `{k[:80]}` | {n} | {fv:.0f} | {wv:.0f} | {fv * 1024 * fs / 1e9:.3f} | "
                     f"{wv * 1024 * ws / 1e9:.3f} |")
    try:
        with open(COUNTERS_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    rec["_note"] = ("HBM bytes per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE passes scaled by a device copy of "
                    "known size (bench.py --traffic-summary); valid only while the kernel source hash matches")
    entry = rec.setdefault(workload, {})
    for role, (frags, files) in TRAFFIC_KERNELS.items():
        cands = [k for k in fetch if any(f in k for f in frags)]
        if not cands:
            continue
        k = max(cands, key=lambda k: fetch[k][1])
        b = fetch[k][1] * 1024 * fs + write.get(k, (0, 0.0))[1] * 1024 * ws
        entry[role] = {"kernel": k[:80], "bytes_per_launch": int(b), "source_hash": kernel_source_hash(files)}
        lines.append(f"\n{role}: `{k[:80]}`: {b / 1e9:.3f} GB per launch")
    with open(COUNTERS_FILE, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print("\n".join(lines))


def bench_compare(a, cfg, dev):
    """Whole forwards of the same inputs through several builds of the library in one process, the
    builds taken in turn for `reps` rounds of `steps` forwards each (after `warmup` forwards), so that
    clock and power drift fall on every build alike.  Reports per build the median and minimum ms per
    forward, the median per-phase times and whether its Z equals the first build's bit for bit."""
    import numpy as np
    import torch

    import stca_inputs as SI
    from target_cross_attention_amd import binding as B

    W = SI.make_weights(cfg)
    inp = SI.make_inputs(cfg)
    dw = B.DeviceWeights(W, cfg.dtype, dev)
    db = B.DeviceBatch(inp, dev)
    del inp.X
    runs = []
    for spec in a.compare:
        label, _, path = spec.partition("=")
        lib = B.load_library(path or label)
        for el in (a.compare_encode_layers or [a.encode_layers]):
            runs.append({"label": label, "lib": path or label, "encode_layers": el, "handle": lib,
                         "ms": [], "phases": {}, "Z": None})
    stream = torch.cuda.current_stream()
    default_lib = B.LIB
    try:
        for rep in range(a.reps):
            for r in runs:
                B.LIB = r["handle"]
                dims = B.dims_for(cfg, attn_chunk=a.attn_chunk, encode_layers=r["encode_layers"])
                ws = B.workspace(B.forward_workspace_size(dims, db.c), dev)
                Z = torch.empty((db.total_T, cfg.M, cfg.d), dtype=torch.float32, device=dev)
                for _ in range(max(a.warmup, 1)):
                    B.stca_forward(dims, dw, db, Z=Z, ws=ws, stream=stream)
                prof = B.Profiler()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(a.steps):
                    B.stca_forward(dims, dw, db, Z=Z, ws=ws, stream=stream, profiler=prof)
                e1.record(stream)
                torch.cuda.synchronize()
                r["ms"].append(e0.elapsed_time(e1) / a.steps)
                for k, (ms, _) in prof.read().items():
                    r["phases"].setdefault(k, []).append(ms / a.steps)
                prof.close()
                if r["Z"] is None:
                    r["Z"] = Z.clone()
                del ws, Z
                log(f"round {rep} {r['label']} encode_layers={r['encode_layers']}: {r['ms'][-1]:.3f} ms per forward")
    finally:
        B.LIB = default_lib
    ref = runs[0]["Z"]
    out = {"compare": cfg.key, "workload": cfg.description, "rounds": a.reps, "forwards_per_round": a.steps,
           "results": [{"label": r["label"], "lib": r["lib"], "encode_layers": r["encode_layers"],
                        "ms_per_forward_median": float(np.median(r["ms"])), "ms_per_forward_min": float(min(r["ms"])),
                        "ms_per_forward": [round(x, 3) for x in r["ms"]],
                        "phase_ms_median": {k: round(float(np.median(v)), 4) for k, v in r["phases"].items()
                                            if np.median(v) > 0},
                        "bitwise_equal_to_first": bool(torch.equal(r["Z"], ref))} for r in runs]}
    print(json.dumps(out))


def bench_vendor_gemm(a, dev):
    """torch.matmul (hipBLASLt) bf16 GEMMs at the encode's shapes for the workload (1 Mi history
    rows: up and gate as one [rows x d] x [d x 2rd] product, the down product [rows x rd] x [rd x d])
    and at a large square shape, as a ceiling reference for the fused encode.  GEMMs only: the
    vendor path would still need the gate and LayerNorm kernels."""
    import torch

    import stca_inputs as SI
    cfg = SI.get_config(a.workload)
    rows = 1 << 20
    d, rd = cfg.d, cfg.r * cfg.d
    g = torch.Generator(device=dev)
    g.manual_seed(0)

    def rnd(m, n):
        return torch.randn(m, n, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)

    def timed(A, Bm, reps):
        C = A @ Bm
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.matmul(A, Bm, out=C)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        fl = 2.0 * A.shape[0] * A.shape[1] * Bm.shape[1]
        return {"shape": f"[{A.shape[0]} x {A.shape[1]}] x [{Bm.shape[0]} x {Bm.shape[1]}]", "avg_ms": ms,
                "tflops": fl / ms / 1e9, "frac": fl / ms / 1e9 / PEAK_BF16_TFLOPS}

    reps = max(a.steps, 10)
    X, Wuv = rnd(rows, d), rnd(d, 2 * rd)
    up = timed(X, Wuv, reps)
    del X, Wuv
    H, Wo = rnd(rows, rd), rnd(rd, d)
    down = timed(H, Wo, reps)
    del H, Wo
    S1, S2 = rnd(16384, 16384), rnd(16384, 16384)
    square = timed(S1, S2, reps)
    del S1, S2
    enc_ms = up["avg_ms"] + down["avg_ms"]
    enc_flops = 6.0 * cfg.r * d * d * rows
    print(json.dumps({
        "metric": "vendor bf16 GEMM throughput at the encode's shapes (ceiling reference)",
        "library": "torch.matmul (hipBLASLt), torch " + torch.__version__, "workload": cfg.key,
        "up_gate": up, "down": down, "square_16384": square,
        "encode_gemms_only": {"rows": rows, "ms": enc_ms, "tflops": enc_flops / enc_ms / 1e9,
                              "frac": enc_flops / enc_ms / 1e9 / PEAK_BF16_TFLOPS},
        "peak_tflops": PEAK_BF16_TFLOPS, "reps": reps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dense10k")
    ap.add_argument("--users", type=int, default=0, help="override the number of users (0 = workload's)")
    ap.add_argument("--attn-chunk", type=int, default=0)
    ap.add_argument("--encode-layers", type=int, default=0, choices=(0, 1, 2),
                    help="history encodes: 0 automatic, 1 one launch per layer, 2 every layer in one launch")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sl", action="store_true",
                    help="time a stochastic-length batch built from the workload's histories instead "
                         "(L_avg 2000, L_max = L_infer = 10000, alpha 0.02)")
    ap.add_argument("--litm", action="store_true",
                    help="merge same-ID tokens at most 3 positions apart first (host plan, device merge), then "
                         "time the forward on the merged batch")
    ap.add_argument("--backward", action="store_true",
                    help="time stca_backward instead (default workload: the training-shaped ragged batch)")
    ap.add_argument("--no-keep", action="store_true",
                    help="with --backward: the minimum workspace (recompute the encode's intermediates)")
    ap.add_argument("--flush-cache", action="store_true",
                    help="write a 512 MiB buffer before every timed forward (evicts the Infinity Cache) and time "
                         "each forward on its own with HIP events")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="time torch.matmul (hipBLASLt) bf16 GEMMs at the encode's shapes instead")
    ap.add_argument("--calib-copy", type=int, default=0,
                    help="instead of STCA, run K device copies of 2 GiB (counter calibration)")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "CALIB_FETCH_DIR",
                                                           "CALIB_WRITE_DIR"),
                    help="summarise four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE of this workload's "
                         "bench, then of --calib-copy) and record the traffic per launch; no GPU needed")
    ap.add_argument("--compare", nargs="+", metavar="LABEL=LIB",
                    help="same-process comparison of whole forwards across builds of the library (variants from "
                         "build.py --define ... --out LIB), alternating between them; prints one JSON line")
    ap.add_argument("--compare-encode-layers", nargs="+", type=int, choices=(0, 1, 2), default=None,
                    help="with --compare: run every build at each of these encode_layers settings")
    ap.add_argument("--reps", type=int, default=4, help="with --compare: rounds over the builds")
    a = ap.parse_args()
    if a.traffic_summary:
        return traffic_summary(a.workload, *a.traffic_summary)

    if a.gpus != 1:
        print(json.dumps({"error": "the STCA path here runs on one GPU; --gpus must be 1 "
                          "(the forward would shard by user with no exchange; no multi-GPU path exists)"}))
        sys.exit(2)

    import numpy as np
    import torch

    import stca_inputs as SI
    from target_cross_attention_amd import binding as B

    dev = torch.device("cuda:0")
    if a.calib_copy:
        n = 2 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(a.calib_copy):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n, "copies": a.calib_copy}))
        return

    if a.vendor_gemm:
        return bench_vendor_gemm(a, dev)
    if a.backward and a.workload == "dense10k":
        a.workload = "ragged"
    cfg = SI.get_config(a.workload)
    if a.users:
        cfg = SI.scaled(cfg, n_users=a.users)
    if a.sl:
        return bench_sl(a, cfg, dev)
    if a.litm:
        return bench_litm(a, cfg, dev)
    if a.backward:
        return bench_backward(a, cfg, dev)
    if a.compare:
        return bench_compare(a, cfg, dev)
    t = time.perf_counter()
    W = SI.make_weights(cfg)
    inp = SI.make_inputs(cfg)
    log(f"inputs {cfg.key}: {inp.n_users} users, {inp.total_L} history tokens, {inp.total_T} targets "
        f"({time.perf_counter() - t:.1f} s)")
    dims = B.dims_for(cfg, attn_chunk=a.attn_chunk, encode_layers=a.encode_layers)
    dw = B.DeviceWeights(W, cfg.dtype, dev)
    db = B.DeviceBatch(inp, dev)
    del inp.X
    ws = B.workspace(B.forward_workspace_size(dims, db.c), dev)
    Z = torch.empty((db.total_T, cfg.M, cfg.d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    log(f"workspace {ws.numel() / 2**30:.2f} GiB; warmup {a.warmup}")
    for _ in range(a.warmup):
        B.stca_forward(dims, dw, db, Z=Z, ws=ws, stream=stream)
    torch.cuda.synchronize()

    prof = B.Profiler()
    log(f"timing {a.steps} steps" + (" (Infinity Cache flushed before each)" if a.flush_cache else ""))
    flush = torch.empty(2 * INFINITY_CACHE_BYTES, dtype=torch.uint8, device=dev) if a.flush_cache else None
    torch.cuda.synchronize()
    if a.flush_cache:
        # each forward timed on its own, after a write of twice the cache's size; the flush is
        # outside the events
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(a.steps)]
        t0 = time.perf_counter()
        for k in range(a.steps):
            flush.fill_(k & 0xFF)
            ev[k][0].record(stream)
            B.stca_forward(dims, dw, db, Z=Z, ws=ws, stream=stream, profiler=prof)
            ev[k][1].record(stream)
        torch.cuda.synchronize()
        step_ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
        dt = sum(step_ms) / 1e3
        del flush
    else:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
        t0 = time.perf_counter()
        ev[0].record(stream)
        for k in range(a.steps):
            B.stca_forward(dims, dw, db, Z=Z, ws=ws, stream=stream, profiler=prof)
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        step_ms = sorted(ev[k].elapsed_time(ev[k + 1]) for k in range(a.steps))
    phases = prof.read()
    prof.close()
    assert np.isfinite(Z.sum().item()), "non-finite output"

    # The same forward replayed from a HIP graph (stca_forward_graph_create): identical kernels with
    # the per-call host work and launch gaps removed; reported beside the eager figure.
    graph = B.ForwardGraph(dims, dw, db, ws=ws)
    graph.launch(stream)
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for _ in range(a.steps):
        graph.launch(stream)
    g1.record(stream)
    torch.cuda.synchronize()
    graph_ms = g0.elapsed_time(g1) / a.steps
    assert torch.equal(graph.Z, Z), "graph replay differs from the eager forward"
    graph.close()

    # The prediction token of eq. (9) is the next step downstream of the forward (outside the timed
    # forward): timed on its own, from the forward's Z, on the call's stream.
    pw = B.DevicePredict(SI.make_predict_weights(cfg), cfg.dtype, dev)
    zbuf = torch.empty((db.total_T, cfg.d), dtype=torch.float32, device=dev)
    pws = B.workspace(B.predict_workspace_size(dims, db.total_T), dev)
    B.stca_predict(dims, pw, Z, db.xt, z=zbuf, ws=pws, stream=stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_pred = max(a.steps, 5)
    e0.record(stream)
    for _ in range(n_pred):
        B.stca_predict(dims, pw, Z, db.xt, z=zbuf, ws=pws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    pred_ms = e0.elapsed_time(e1) / n_pred
    pred_flops = float(db.total_T) * (2.0 * (cfg.M + 1) * cfg.d * cfg.d + 6.0 * cfg.r * cfg.d * cfg.d)
    assert np.isfinite(zbuf.sum().item()), "non-finite prediction token"

    ms_per_step = dt * 1e3 / a.steps
    tokens_per_s = db.total_L * a.steps / dt
    targets_per_s = db.total_T * a.steps / dt

    # Dominant kernel: the fused encode.  bf16: one launch per step encodes all M layers; fp32: one
    # launch sequence per layer.  Algorithmic work: 6 r d^2 FLOP per history token and layer (up +
    # gate d x rd, down rd x d, 2 FLOP per multiply-add); bytes: X read once per launch (2d per
    # token in bf16), X~ written once per layer (2d).
    bf16 = cfg.dtype == "bf16"
    enc_ms, enc_n = phases["encode"]
    enc_avg_s = enc_ms / max(enc_n, 1) / 1e3
    layers_per_launch = cfg.M * a.steps / max(enc_n, 1)
    esz = 2.0 if bf16 else 4.0
    enc_flops = 6.0 * cfg.r * cfg.d * cfg.d * db.total_L * layers_per_launch
    enc_bytes = esz * cfg.d * db.total_L * (1.0 + layers_per_launch)
    peak_mm = PEAK_BF16_TFLOPS if bf16 else PEAK_FP32_TFLOPS
    achieved = enc_flops / enc_avg_s / 1e12
    traffic = measured_traffic(cfg.key, "encode", ["encode_mfma.hip", "device_common.hpp"])
    # Attention: reads each encoded history once per layer, 2d bytes per token (bf16).
    att_ms, att_n = phases["attend"]
    att_avg_s = att_ms / max(att_n, 1) / 1e3
    att_bytes = (2.0 if bf16 else 4.0) * cfg.d * db.total_L
    att_flops = 4.0 * cfg.h * cfg.d * float((db.inp.L * db.inp.m).sum())
    att_traffic = measured_traffic(cfg.key, "attend", ["attend.hip", "device_common.hpp"])
    att_bound, att_unit, att_peak, att_achieved, att_ridge, att_mfma_peak = attention_roof(
        att_flops, att_bytes, att_avg_s, bf16)

    # The attention reads the X~ that the encode wrote just before it; when one layer's X~ fits the
    # Infinity Cache it is read from there, not from HBM, and the GB/s figure is not an HBM fraction.
    att_cache_resident = att_bytes <= INFINITY_CACHE_BYTES
    enc_label = ("encode (fused SwiGLU FFN + LayerNorm, bf16 MFMA)" if bf16 else
                 "encode (SwiGLU FFN + LayerNorm, fp32 GEMMs: matrix cores for large products, vector ALU "
                 "otherwise)")

    out = {
        "metric": metric_for(cfg),
        "value": tokens_per_s,
        "unit": "history-tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_median": step_ms[len(step_ms) // 2],
        "ms_per_step_min": step_ms[0],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": f"synthetic (seeded; shapes of the pages' {cfg.key} workload)",
        "config": {"workload": cfg.description, "key": cfg.key, "users": db.inp.n_users,
                   "history_tokens": db.total_L, "targets": db.total_T, "d": cfg.d, "h": cfg.h, "M": cfg.M,
                   "r": cfg.r, "attn_chunk": a.attn_chunk or "auto",
                   "encode_layers": {0: "auto", 1: "one launch per layer", 2: "one launch"}[a.encode_layers],
                   "infinity_cache": "flushed before each timed forward" if a.flush_cache else "not flushed"},
        "roofline": {"kernel": enc_label,
                     "bound": "mfma", "achieved": achieved, "peak": peak_mm, "unit": "TFLOP/s",
                     "frac": achieved / peak_mm, "traffic": traffic,
                     "algorithmic_flops_per_launch": enc_flops, "algorithmic_bytes_per_launch": enc_bytes,
                     "avg_launch_ms": enc_avg_s * 1e3, "launches": enc_n,
                     "layers_per_launch": layers_per_launch},
        "attention_roofline": {"kernel": "split-L attention", "bound": att_bound,
                               "achieved": att_achieved, "peak": att_peak, "unit": att_unit,
                               "frac": att_achieved / att_peak, "traffic": att_traffic,
                               "intensity_flop_per_byte": att_flops / att_bytes,
                               "ridge_flop_per_byte": att_ridge,
                               "hbm_gbs": att_bytes / att_avg_s / 1e9,
                               "hbm_frac": att_bytes / att_avg_s / 1e9 / PEAK_HBM_GBS,
                               "mfma_tflops": att_flops / att_avg_s / 1e12,
                               "mfma_frac": att_flops / att_avg_s / 1e12 / att_mfma_peak,
                               "avg_launch_ms": att_avg_s * 1e3, "launches": att_n,
                               "cache_resident": att_cache_resident,
                               "note": ("one layer's X~ fits the 256 MB Infinity Cache and is read from there "
                                        "right after the encode writes it: the GB/s figure is not an HBM "
                                        "fraction" if att_cache_resident else
                                        "one layer's X~ exceeds the Infinity Cache: read from HBM")},
        "targets_per_s": targets_per_s,
        "graph_replay": {"ms_per_step": graph_ms, "history_tokens_per_s": db.total_L / graph_ms * 1e3,
                         "replays": a.steps},
        "phase_ms_per_step": {k: v[0] / a.steps for k, v in phases.items() if not k.startswith("bwd")},
        "prediction_token": {"eq": 9, "rows": db.total_T, "avg_ms": pred_ms, "calls": n_pred,
                             "targets_per_s": db.total_T / pred_ms * 1e3, "bound": "mfma",
                             "achieved": pred_flops / pred_ms / 1e9, "peak": PEAK_FP32_TFLOPS,
                             "unit": "TFLOP/s", "frac": pred_flops / pred_ms / 1e9 / PEAK_FP32_TFLOPS},
    }
    if not a.no_cpu_baseline:
        log("cpu baseline (oracle on a user sample)")
        out["cpu_baseline"] = cpu_baseline(cfg, W)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
