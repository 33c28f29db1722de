"""GPU parity at the workloads' full sizes.

The whole batch runs through stca_forward in the launch configuration bench.py uses (automatic
split-L chunking), followed by stca_predict (the prediction token of eq. (9)); the CPU oracle
recomputes Z and z for every target of sampled users: for ragged length
mixes the shortest and the longest user plus seeded random ones.  The bar is the bf16 bar,
2e-2 max row-relative error (fp32 for the tiny fp32 workload: 1e-4, checked on all outputs).
"""
import time

import numpy as np
import pytest

import stca_inputs as SI
from oracle import stca as O
from stca_testlib import announce, row_rel, tol_for

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from target_cross_attention_amd import binding
    return binding


def sample_users(inp, n, seed=0):
    L = inp.L
    picks = {int(np.argmin(L)), int(np.argmax(L)), 0, inp.n_users - 1}
    rng = np.random.default_rng(seed)
    while len(picks) < min(n, inp.n_users):
        picks.add(int(rng.integers(inp.n_users)))
    return sorted(picks)


@pytest.mark.parametrize("key,n_sample", [("tiny", 1), ("uniform", 8), ("ragged", 8), ("dense10k", 8),
                                          ("stress20k", 4)])
def test_full_size_workload(B, key, n_sample):
    cfg = SI.get_config(key)
    announce("full-size", key, cfg.description)
    t = time.perf_counter()
    W = SI.make_weights(cfg)
    inp = SI.make_inputs(cfg)
    print(f"  inputs: {inp.n_users} users, {inp.total_L} tokens, {inp.total_T} targets "
          f"({time.perf_counter() - t:.1f} s)", flush=True)
    P = SI.make_predict_weights(cfg)
    dw = B.DeviceWeights(W, cfg.dtype, DEV)
    db = B.DeviceBatch(inp, DEV)
    dims = B.dims_for(cfg)
    Zd = B.stca_forward(dims, dw, db)
    zd = B.stca_predict(dims, B.DevicePredict(P, cfg.dtype, DEV), Zd, db.xt)   # eq. (9)
    torch.cuda.synchronize()
    Z, z = Zd.cpu().numpy(), zd.cpu().numpy()
    assert np.all(np.isfinite(Z)) and np.all(np.isfinite(z))
    del db, Zd, zd
    users = sample_users(inp, n_sample)
    worst = 0.0
    t = time.perf_counter()
    for k in users:
        ref = O.forward_user(inp.user_X(k), inp.user_xt(k), W, cfg.h, cfg.M)
        rows = slice(inp.tgt_off[k], inp.tgt_off[k + 1])
        err = row_rel(Z[rows], ref)
        zref = O.prediction_token(ref, inp.as_f32(inp.user_xt(k)), P.WZ, P.Wu, P.Wv, P.Wo)
        zerr = row_rel(z[rows], zref)
        worst = max(worst, err, zerr)
        print(f"  user {k}: L={inp.L[k]} m={inp.m[k]} err={err:.3e} z err={zerr:.3e}", flush=True)
    print(f"  {key}: {len(users)} users checked in {time.perf_counter() - t:.1f} s, worst {worst:.3e}", flush=True)
    assert worst <= tol_for(cfg)
