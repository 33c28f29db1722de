"""GPU checks of stochastic-length batches (stca_sl_pack), against ``oracle.sl`` and the oracle
forward.

* The suffix gather is byte work: bit-exact against the oracle's gather of the same plan.
* A forward on the packed batch (the training-shaped ragged batch the load balancer produces)
  meets the forward's bars against the oracle forward on the oracle's packed histories.
"""
from types import SimpleNamespace

import numpy as np
import pytest

import stca_inputs as SI
from oracle import sl
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


def _sl_batch(B, cfg, alpha, L_min, L_max, L_avg, L_infer):
    inp = SI.make_inputs(cfg)
    beta = sl.beta_param(alpha, L_min, L_max, L_avg)
    s, order = SI.make_sl_draws(cfg, inp.n_users, alpha, beta)
    prm = B.SlParams(L_min, L_max, L_avg, L_infer)
    L, off = B.sl_plan(prm, inp.L, s, order)
    Lr, offr = sl.plan(inp.L, s, order, L_min, L_max, L_avg, L_infer)
    assert np.array_equal(L, Lr) and np.array_equal(off, offr)
    return inp, L, off


@pytest.mark.parametrize("key,change,params", [
    ("ragged", dict(n_users=40, length=("lognormal", 3000.0, 4000.0, 1, 15000)), (0.02, 8, 10000, 2000, 10000)),
    ("uniform", dict(n_users=16, dtype="f32"), (0.5, 64, 2048, 512, 1500)),
    ("stress20k", dict(n_users=6, length=("fixed", 20000)), (2.0, 512, 10000, 2500, 10000)),
], ids=["ragged-bf16", "uniform-f32", "stress20k-bf16"])
def test_pack_is_bit_exact(B, key, change, params):
    cfg = SI.scaled(SI.get_config(key), **change)
    announce("sl-pack", key, cfg.dtype, params)
    inp, L, off = _sl_batch(B, cfg, *params)
    dims = B.dims_for(cfg)
    full_off = torch.from_numpy(inp.hist_off.astype(np.int64)).to(DEV)
    hist_off = torch.from_numpy(off).to(DEV)
    Xf = B.to_device(inp.X, cfg.dtype, DEV)
    Xp = B.sl_pack(dims, full_off, hist_off, int(off[-1]), int(L.max()), Xf)
    torch.cuda.synchronize()
    want, _ = sl.pack(inp.X, inp.hist_off, L)
    got = Xp.cpu().view(torch.int16 if cfg.dtype == "bf16" else torch.int32).numpy()
    want = want.view(np.int16 if cfg.dtype == "bf16" else np.int32)
    print(f"  {key}: users={inp.n_users} full={inp.total_L} packed={int(off[-1])}", flush=True)
    assert got.shape == want.shape and np.array_equal(got, want)


def test_forward_on_packed_batch(B):
    cfg = SI.scaled(SI.get_config("ragged"), n_users=24, length=("lognormal", 3000.0, 4000.0, 1, 15000))
    params = (0.02, 8, 10000, 2000, 10000)
    announce("sl-forward", cfg.key, params)
    inp, L, off = _sl_batch(B, cfg, *params)
    W = SI.make_weights(cfg)
    dims = B.dims_for(cfg)
    full_off = torch.from_numpy(inp.hist_off.astype(np.int64)).to(DEV)
    hist_off = torch.from_numpy(off).to(DEV)
    Xp = B.sl_pack(dims, full_off, hist_off, int(off[-1]), int(L.max()), B.to_device(inp.X, cfg.dtype, DEV))
    tgt_off = torch.from_numpy(inp.tgt_off.astype(np.int64)).to(DEV)
    xt = B.to_device(inp.xt, cfg.dtype, DEV)
    T = int(inp.tgt_off[-1])
    batch = SimpleNamespace(X=Xp, xt=xt, total_T=T,
                            c=B.batch_struct(inp.n_users, hist_off, tgt_off, int(off[-1]), T, int(L.max()),
                                             int(inp.m.max())))
    Z = B.stca_forward(dims, B.DeviceWeights(W, cfg.dtype, DEV), batch)
    torch.cuda.synchronize()
    Z = Z.cpu().numpy()
    Xpk, _ = sl.pack(inp.as_f32(inp.X), inp.hist_off, L)
    ref = np.concatenate([O.forward_user(Xpk[off[u]:off[u + 1]], inp.user_xt(u), W, cfg.h, cfg.M)
                          for u in range(inp.n_users)])
    err = row_rel(Z, ref)
    print(f"  users={inp.n_users} packed tokens={int(off[-1])} T={T} err={err:.3e}", flush=True)
    assert err <= tol_for(cfg)
