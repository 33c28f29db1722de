"""GPU parity of stca_backward against ``oracle.grad`` (float64 chain rule, pinned by finite
differences of the forward oracle in test_oracle_grad.py) on identical seeded inputs.

Both sides differentiate the same function of the same stored values (bf16 workloads: the
bf16-rounded X, x_t and weights); the oracle computes in float64.  Bar: for every gradient tensor,
max |gpu - oracle| / max |oracle| <= tol, per tensor rather than per row (weight gradients are sums
over all rows and have no natural row scale).

* fp32 path (dtype f32): fp32 arithmetic throughout, tol 1e-4.  Each gradient is a short chain
  (<= 4 layers x ~10 products) of fp32 sums; at these sizes a sum runs over at most ~1500 terms,
  whose relative error is of order sqrt(K) u in the mean and K u at worst (u = 2^-24: 2e-6 ..
  9e-5), and no step divides by a small quantity (LayerNorm rows have unit scale, far from
  rstd = 1/sqrt(eps)).
* mixed-precision path (dtype bf16): the history encode's derivative and the attention derivative
  run their products on bf16 operands with fp32 accumulation, and the recomputed X~ comes from the
  forward's bf16 encode.  Every operand rounding is a relative error of at most u = 2^-8 (8
  significant bits); an element of a gradient passes through up to about six such roundings (in
  the attention derivative alpha or dS, X~, U and dA-bar; in the encode derivative dY, dU or dG,
  the bf16 H and the recomputed pre-activations), whose independent errors largely cancel in the
  fp32 sums: a sum of K terms with independent relative errors of at most u has a relative error
  of about u / sqrt(3) per rounding stage, so six stages give about sqrt(6) u / sqrt(3) = 5.5e-3
  in the mean; the worst tensors observed reach 9.3e-3.  tol 2e-2 (about 5 u), the forward's bf16
  bar.
A wrong term (a dropped softmax centring, a transposed operand, a missing LayerNorm mean) gives
errors of order 1e-2 .. 1 in the fp32 path, where the bar is tight; the mixed path's cases also run
through the fp32 path (dtype f32) at 1e-4.
"""
import dataclasses

import numpy as np
import pytest

import stca_inputs as SI
from oracle import grad as G
from stca_testlib import announce

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
GRAD_TOL = 1e-4    # fp32 path
MIXED_TOL = 2e-2   # mixed-precision path (bf16 storage)
SLOTS = ["Wu", "Wv", "Wo", "gamma", "beta", "qWu", "qWv", "qWo", "qgamma", "qbeta", "WQ", "WK", "WV", "WO", "WC"]


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from target_cross_attention_amd import binding
    return binding


def tensor_rel(g, o) -> float:
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    if o.size == 0:
        return 0.0
    den = max(float(np.max(np.abs(o))), 1e-30)
    r = float(np.max(np.abs(g - o))) / den
    return float("inf") if np.isnan(r) else r


def without_targets(inp, drop):
    """The batch with the users at positions ``drop`` given no targets (their histories stay)."""
    m = inp.m.copy()
    keep_rows = []
    for k in range(inp.n_users):
        if k in drop:
            m[k] = 0
        else:
            keep_rows.extend(range(inp.tgt_off[k], inp.tgt_off[k + 1]))
    return dataclasses.replace(inp, m=m, tgt_off=SI.offsets(m), xt=inp.xt[np.asarray(keep_rows, np.int64)])


def run_case(B, cfg, inp, W, query_ln=False, seed=5, keep=False):
    dims = B.dims_for(cfg, query_ln=query_ln)
    dZ = np.random.default_rng(seed).standard_normal((inp.total_T, cfg.M, cfg.d)).astype(np.float32)
    dw = B.DeviceWeights(W, cfg.dtype, DEV)
    db = B.DeviceBatch(inp, DEV)
    grads = B.stca_backward(dims, dw, db, torch.from_numpy(dZ).to(DEV), keep=keep)
    torch.cuda.synchronize()
    ref = G.backward_batch(inp, W, dZ.astype(np.float64), query_ln=query_ln)
    errs = {"dX": tensor_rel(grads.dX[:inp.total_L].cpu().numpy(), ref.dX),
            "dxt": tensor_rel(grads.dxt[:inp.total_T].cpu().numpy(), ref.dxt)}
    for name in SLOTS:
        for i, t in enumerate(grads.slot(name)):
            want = getattr(ref, name)[i]
            if t is None:
                assert want is None or not np.any(want), (name, i)   # unused slot: zero in the oracle
                continue
            errs[f"{name}[{i}]"] = tensor_rel(t.cpu().numpy(), want)
    worst = max(errs, key=errs.get)
    tol = GRAD_TOL if cfg.dtype == "f32" else MIXED_TOL
    print(f"  {cfg.dtype} users={inp.n_users} L={inp.total_L} T={inp.total_T} worst {worst}={errs[worst]:.3e} "
          f"(tol {tol})", flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad
    return errs


CASES = [
    ("tiny", dict(), False, False),
    ("tiny", dict(M=3, n_users=3, length=("fixed", 40), targets=("fixed", 3)), True, True),
    ("tiny", dict(M=4, n_users=2, length=("fixed", 33), targets=("fixed", 2), dtype="bf16"), False, True),
    ("uniform", dict(n_users=3, length=("fixed", 200)), False, False),
    ("ragged", dict(n_users=5, length=("lognormal", 150.0, 200.0, 16, 600)), False, True),
    ("ragged", dict(n_users=4, dtype="f32", length=("lognormal", 100.0, 150.0, 16, 400)), True, False),
    ("stress20k", dict(n_users=2, M=2, length=("fixed", 150), targets=("fixed", 3)), False, False),
    # large enough that the encode products run on the fp32 matrix-core GEMM (>= 128 output tiles)
    ("ragged", dict(n_users=40, length=("lognormal", 150.0, 200.0, 16, 600)), False, False),
    ("stress20k", dict(n_users=2, M=2, length=("fixed", 600), targets=("fixed", 3)), False, True),
]


@pytest.mark.parametrize("key,change,query_ln,separate", CASES,
                         ids=[f"{k}-{i}" for i, (k, *_) in enumerate(CASES)])
def test_backward_matches_oracle(B, key, change, query_ln, separate):
    cfg = SI.scaled(SI.get_config(key), **change)
    announce("backward", cfg.key, cfg.dtype, change, "query_ln" if query_ln else "", "separate" if separate else "")
    W = SI.make_weights(cfg, random_ln=True, separate_query_ffn=separate)
    run_case(B, cfg, SI.make_inputs(cfg), W, query_ln=query_ln)


@pytest.mark.parametrize("key,change,query_ln,separate", [c for c in CASES if SI.scaled(SI.get_config(c[0]), **c[1]).dtype == "bf16"],
                         ids=[f"{k}-{i}-f32" for i, (k, ch, *_) in enumerate(CASES)
                              if SI.scaled(SI.get_config(k), **ch).dtype == "bf16"])
def test_backward_fp32_path_on_mixed_cases(B, key, change, query_ln, separate):
    """The cases the mixed-precision path runs, through the fp32 debug path (fp32 storage) at 1e-4."""
    cfg = SI.scaled(SI.get_config(key), **dict(change, dtype="f32"))
    announce("backward-f32", cfg.key, change, "query_ln" if query_ln else "", "separate" if separate else "")
    W = SI.make_weights(cfg, random_ln=True, separate_query_ffn=separate)
    run_case(B, cfg, SI.make_inputs(cfg), W, query_ln=query_ln)


@pytest.mark.parametrize("key,change,query_ln,separate", [CASES[1], CASES[4], CASES[7]],
                         ids=["tiny-M3", "ragged-small", "ragged-40"])
def test_backward_keep_workspace(B, key, change, query_ln, separate):
    """The fp32 path's larger workspace, which keeps the encode's intermediates from the forward
    recompute, gives the same gradients (the same bar against the oracle)."""
    cfg = SI.scaled(SI.get_config(key), **dict(change, dtype="f32"))
    announce("backward-keep", cfg.key, cfg.dtype, change)
    W = SI.make_weights(cfg, random_ln=True, separate_query_ffn=separate)
    run_case(B, cfg, SI.make_inputs(cfg), W, query_ln=query_ln, keep=True)


def test_backward_short_histories_and_targetless_users(B):
    """Many users with 1..40 history rows (the key-side kernel's rows straddle users) and some
    users without targets (their history gets zero gradient)."""
    cfg = SI.scaled(SI.get_config("ragged"), n_users=23, M=2, length=("lognormal", 4.0, 8.0, 1, 40))
    announce("backward-short", cfg.key)
    inp = without_targets(SI.make_inputs(cfg), {0, 5, 6, 22})
    W = SI.make_weights(cfg, random_ln=True)
    run_case(B, cfg, inp, W)


def test_backward_no_targets_gives_zero(B):
    cfg = SI.scaled(SI.get_config("tiny"), n_users=2, M=2)
    inp = without_targets(SI.make_inputs(cfg), {0, 1})
    announce("backward-no-targets", cfg.key)
    dims = B.dims_for(cfg)
    dw = B.DeviceWeights(SI.make_weights(cfg), cfg.dtype, DEV)
    db = B.DeviceBatch(inp, DEV)
    grads = B.DeviceGrads(dims, inp.total_L, 0, DEV)
    for t in [grads.dX] + [x for k in SLOTS for x in grads.slot(k) if x is not None]:
        t.fill_(7.0)                                  # every output is overwritten
    B.stca_backward(dims, dw, db, torch.zeros((1, cfg.M, cfg.d), device=DEV), grads)
    torch.cuda.synchronize()
    assert float(grads.dX.abs().max()) == 0.0
    for k in SLOTS:
        for x in grads.slot(k):
            if x is not None:
                assert float(x.abs().max()) == 0.0, k


def test_backward_full_size_ragged_sampled(B):
    """The whole training-shaped batch (512 users, ~1M history tokens, the size the backward bench
    times) in one call, on the mixed-precision path.  Every gradient is linear in dZ and a user's dX and
    dx_t depend only on its own dZ, so: (a) with dZ random everywhere, the dX / dx_t rows of sampled
    users equal the oracle run on those users alone; (b) with dZ zero outside the sampled users, every
    weight gradient equals the oracle's over those users and every other dX / dx_t row is exactly
    zero.  Bar: the mixed path's 2e-2."""
    cfg = SI.get_config("ragged")
    announce("backward-fullsize", cfg.key)
    W = SI.make_weights(cfg)
    inp = SI.make_inputs(cfg)
    L = inp.L
    sample = sorted({0, int(np.argmax(L)), inp.n_users - 1})
    dims = B.dims_for(cfg)
    dw = B.DeviceWeights(W, cfg.dtype, DEV)
    db = B.DeviceBatch(inp, DEV)
    rng = np.random.default_rng(9)
    dZ = rng.standard_normal((inp.total_T, cfg.M, cfg.d)).astype(np.float32)
    ga = B.stca_backward(dims, dw, db, torch.from_numpy(dZ).to(DEV))
    mask = np.zeros(inp.total_T, bool)
    for k in sample:
        mask[inp.tgt_off[k]:inp.tgt_off[k + 1]] = True
    gb = B.stca_backward(dims, dw, db, torch.from_numpy(dZ * mask[:, None, None]).to(DEV))
    torch.cuda.synchronize()
    sub = SI.make_inputs(cfg, users=sample)
    ref = G.backward_batch(sub, W, dZ[mask].astype(np.float64))
    errs = {}
    hrows = np.concatenate([np.arange(inp.hist_off[k], inp.hist_off[k + 1]) for k in sample])
    trows = np.nonzero(mask)[0]
    for tag, g in (("a", ga), ("b", gb)):
        dX = g.dX[:inp.total_L].cpu().numpy()
        dxt = g.dxt[:inp.total_T].cpu().numpy()
        errs[f"{tag}:dX"] = tensor_rel(dX[hrows], ref.dX)
        errs[f"{tag}:dxt"] = tensor_rel(dxt[trows], ref.dxt)
        if tag == "b":
            other = np.ones(inp.total_L, bool)
            other[hrows] = False
            assert not np.any(dX[other]) and not np.any(dxt[~mask])
    for name in SLOTS:
        for i, t in enumerate(gb.slot(name)):
            if t is not None:
                errs[f"{name}[{i}]"] = tensor_rel(t.cpu().numpy(), getattr(ref, name)[i])
    worst = max(errs, key=errs.get)
    print(f"  users={inp.n_users} L={inp.total_L} T={inp.total_T} sampled={sample} (L={L[sample].tolist()}) "
          f"worst {worst}={errs[worst]:.3e}", flush=True)
    bad = {k: v for k, v in errs.items() if not v <= MIXED_TOL}
    assert not bad, bad
