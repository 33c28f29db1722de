"""GPU parity at the workloads' full sizes.

The whole batch runs through stca_forward in the launch configuration bench.py uses (automatic
split-L chunking), followed by stca_predict (the prediction token of eq. (9)); the CPU oracle
recomputes Z and z for the targets of every user where the whole oracle finishes in seconds
(tiny, uniform, ragged: every user, checked in shards so that each test stays short) and for
sampled users elsewhere (dense10k, stress20k: the first, the last and seeded random ones, at
least eight).  The bar is the bf16 bar, 2e-2 max row-relative error (fp32 for the tiny fp32
workload: 1e-4).
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


_RUN = {}


def gpu_run(B, key):
    """The workload's inputs and the GPU's Z and z, for the last workload asked for (one at a time:
    the large workloads hold several GB of host memory)."""
    if key in _RUN:
        return _RUN[key]
    _RUN.clear()
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
    del db, dw, Zd, zd
    torch.cuda.empty_cache()
    assert np.all(np.isfinite(Z)) and np.all(np.isfinite(z))
    _RUN[key] = (cfg, W, P, inp, Z, z)
    return _RUN[key]


def sample_users(inp, n, seed=0):
    L = inp.L
    picks = {int(np.argmin(L)), int(np.argmax(L)), 0, inp.n_users - 1}
    rng = np.random.default_rng(seed)
    while len(picks) < min(n, inp.n_users):
        picks.add(int(rng.integers(inp.n_users)))
    return sorted(picks)


def check_users(key, users, cfg, W, P, inp, Z, z):
    worst = 0.0
    t = time.perf_counter()
    for k in users:
        ref = O.forward_user(inp.user_X(k), inp.user_xt(k), W, cfg.h, cfg.M)
        rows = slice(inp.tgt_off[k], inp.tgt_off[k + 1])
        err = row_rel(Z[rows], ref)
        zref = O.prediction_token(ref, inp.as_f32(inp.user_xt(k)), P.WZ, P.Wu, P.Wv, P.Wo)
        zerr = row_rel(z[rows], zref)
        worst = max(worst, err, zerr)
        if len(users) <= 16:
            print(f"  user {k}: L={inp.L[k]} m={inp.m[k]} err={err:.3e} z err={zerr:.3e}", flush=True)
    print(f"  {key}: users {users[0]}..{users[-1]} ({len(users)}) checked in {time.perf_counter() - t:.1f} s, "
          f"worst row-relative error {worst:.3e}", flush=True)
    return worst


# (workload, shard, shards): every user of tiny, uniform and ragged, split into shards of about 128
# users (the oracle's cost per shard stays within seconds to tens of seconds).
EVERY_USER = [("tiny", 0, 1), ("uniform", 0, 2), ("uniform", 1, 2),
              ("ragged", 0, 4), ("ragged", 1, 4), ("ragged", 2, 4), ("ragged", 3, 4)]


@pytest.mark.parametrize("key,shard,shards", EVERY_USER, ids=[f"{k}-{i}of{n}" for k, i, n in EVERY_USER])
def test_full_size_every_user(B, key, shard, shards):
    cfg, W, P, inp, Z, z = gpu_run(B, key)
    users = list(range(shard, inp.n_users, shards))
    worst = check_users(key, users, cfg, W, P, inp, Z, z)
    assert worst <= tol_for(cfg)


# (workload, sample seed, users): sampled users of the two largest workloads, >= 8 each.
SAMPLED = [("dense10k", 0, 8), ("stress20k", 0, 4), ("stress20k", 1, 4)]


@pytest.mark.slow
@pytest.mark.parametrize("key,seed,n", SAMPLED, ids=[f"{k}-sample{s}" for k, s, _ in SAMPLED])
def test_full_size_sampled_users(B, key, seed, n):
    cfg, W, P, inp, Z, z = gpu_run(B, key)
    if seed == 0:
        users = sample_users(inp, n, seed=0)
    else:  # further seeded picks, disjoint from the first sample
        first = set(sample_users(inp, n, seed=0))
        rng = np.random.default_rng(1000 + seed)
        users = []
        while len(users) < n:
            u = int(rng.integers(inp.n_users))
            if u not in first and u not in users:
                users.append(u)
        users.sort()
    worst = check_users(key, users, cfg, W, P, inp, Z, z)
    assert worst <= tol_for(cfg)
