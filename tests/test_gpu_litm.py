"""GPU checks of local same-ID token merging (stca_litm_merge), against ``oracle.litm`` and the
oracle forward.

* Merged rows are fp32 sums of bf16 (or fp32) rows rounded once: within one bf16 rounding of the
  oracle's float64 sums (bf16 rows), or within the fp32 summation bound (fp32 rows).
* At the full dense10k size (the workload's ~10% repeats) sampled groups are checked one by one.
* A forward on the merged batch meets the forward's bar against the oracle forward on the
  oracle's merged rows (both sides merge on their own; the oracle's sums are rounded to bf16).
"""
from types import SimpleNamespace

import numpy as np
import pytest

import stca_inputs as SI
from oracle import litm
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


def _merge_on_gpu(B, dims, dtype, X, go, mem):
    got = B.litm_merge(dims, torch.from_numpy(go).to(DEV), torch.from_numpy(mem).to(DEV), B.to_device(X, dtype, DEV))
    torch.cuda.synchronize()
    if dtype == "bf16":
        return SI.bits_to_f32(got.cpu().view(torch.int16).numpy().view(np.uint16)).astype(np.float64)
    return got.cpu().numpy().astype(np.float64)


def _check_groups(got, X32, go, mem, groups, dtype):
    for g in groups:
        rows = X32[mem[go[g]:go[g + 1]]].astype(np.float64)
        want = rows.sum(0)
        if dtype == "bf16":   # one rounding of an (almost always exact) fp32 sum to bf16
            tol = 2.0 ** -8 * np.abs(want) + 1e-30
        else:                 # fp32 summation of len(rows) terms
            tol = 4 * len(rows) * 2.0 ** -24 * np.abs(rows).sum(0) + 1e-30
        assert np.all(np.abs(got[g] - want) <= tol), (g, np.max(np.abs(got[g] - want) / tol))


@pytest.mark.parametrize("d,dtype,alphabet", [(64, "f32", 3), (128, "bf16", 5), (256, "bf16", 4), (512, "bf16", 50)])
def test_merge_matches_oracle(B, d, dtype, alphabet):
    announce("litm-merge", d, dtype, alphabet)
    rng = np.random.default_rng(d)
    L = rng.integers(1, 300, 11)
    off = np.concatenate([[0], np.cumsum(L)]).astype(np.int64)
    ids = rng.integers(0, alphabet, int(off[-1])).astype(np.int64)
    X = rng.standard_normal((int(off[-1]), d)).astype(np.float32)
    X = SI.bf16_round(X) if dtype == "bf16" else X
    mo, go, mem = B.litm_plan(off, ids, 3)
    ro, rgo, rmem = litm.plan(ids, off, 3)
    assert np.array_equal(mo, ro) and np.array_equal(go, rgo) and np.array_equal(mem, rmem)
    dims = B.make_dims(d, 8, 1, 2, dtype)
    got = _merge_on_gpu(B, dims, dtype, X, go, mem)
    ref = litm.merge(X, go, mem)
    assert got.shape == ref.shape
    _check_groups(got, X, go, mem, range(len(go) - 1), dtype)
    print(f"  rows={int(off[-1])} groups={len(go) - 1}", flush=True)


def test_merge_full_size_dense10k_sampled(B):
    cfg = SI.get_config("dense10k")
    announce("litm-merge-fullsize", cfg.key)
    inp = SI.make_inputs(cfg, with_ids=True)
    mo, go, mem = B.litm_plan(inp.hist_off, inp.item_id, 3)
    n_groups = len(go) - 1
    dims = B.dims_for(cfg)
    Xd = B.to_device(inp.X, cfg.dtype, DEV)
    out = B.litm_merge(dims, torch.from_numpy(go).to(DEV), torch.from_numpy(mem).to(DEV), Xd)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    sample = np.unique(np.concatenate([rng.integers(0, n_groups, 2000), [0, n_groups - 1],
                                       np.nonzero(np.diff(go) > 1)[0][:500]]))
    got = SI.bits_to_f32(out[torch.from_numpy(sample).to(DEV)].cpu().view(torch.int16).numpy().view(np.uint16))
    full = np.zeros((n_groups, cfg.d))
    full[sample] = got
    X32 = SI.bits_to_f32(inp.X)
    _check_groups(full, X32, go, mem, sample, cfg.dtype)
    print(f"  tokens={inp.total_L} merged={n_groups} ({1 - n_groups / inp.total_L:.1%} fewer)", flush=True)
    assert n_groups == int(mo[-1]) and 0.05 < 1 - n_groups / inp.total_L < 0.15


def test_forward_on_merged_batch(B):
    cfg = SI.scaled(SI.get_config("dense10k"), n_users=10)
    announce("litm-forward", cfg.key)
    inp = SI.make_inputs(cfg, with_ids=True)
    W = SI.make_weights(cfg)
    dims = B.dims_for(cfg)
    mo, go, mem = B.litm_plan(inp.hist_off, inp.item_id, 3)
    Xm = B.litm_merge(dims, torch.from_numpy(go).to(DEV), torch.from_numpy(mem).to(DEV),
                      B.to_device(inp.X, cfg.dtype, DEV))
    hist_off = torch.from_numpy(mo).to(DEV)
    tgt_off = torch.from_numpy(inp.tgt_off.astype(np.int64)).to(DEV)
    T = int(inp.tgt_off[-1])
    Lm = np.diff(mo)
    batch = SimpleNamespace(X=Xm, xt=B.to_device(inp.xt, cfg.dtype, DEV), total_T=T,
                            c=B.batch_struct(inp.n_users, hist_off, tgt_off, int(mo[-1]), T, int(Lm.max()),
                                             int(inp.m.max())))
    Z = B.stca_forward(dims, B.DeviceWeights(W, cfg.dtype, DEV), batch)
    torch.cuda.synchronize()
    Z = Z.cpu().numpy()
    rgo, rmem = litm.plan(inp.item_id, inp.hist_off, 3)[1:]
    Xr = SI.bf16_round(litm.merge(inp.as_f32(inp.X), rgo, rmem).astype(np.float32))
    ref = np.concatenate([O.forward_user(Xr[mo[u]:mo[u + 1]], inp.user_xt(u), W, cfg.h, cfg.M)
                          for u in range(inp.n_users)])
    err = row_rel(Z, ref)
    print(f"  users={inp.n_users} tokens={inp.total_L} merged={int(mo[-1])} T={T} err={err:.3e}", flush=True)
    assert err <= tol_for(cfg)
