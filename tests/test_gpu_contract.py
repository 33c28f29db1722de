"""GPU tests of the batch contract and of the binding's stream handling.

* stca_validate_batch names the broken condition of a batch whose device offsets disagree with its
  host fields, and returns 0 for the workloads' batches.
* A forward over such a batch writes NaN to every output row: the ragged kernels check the offsets
  before they use them, so nothing is read or written outside the buffers (every kernel still runs
  to its normal end; the offsets are only inconsistent with the host-side sizes, never used to
  address memory).
* A call on a stream that is not torch's current stream allocates its workspace for that stream:
  reusing the freed memory on the current stream straight away does not disturb the call.
"""
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


def small_batch():
    cfg = SI.scaled(SI.get_config("ragged"), n_users=3, length=("lognormal", 100.0, 120.0, 8, 300))
    return cfg, SI.make_weights(cfg), SI.make_inputs(cfg)


def test_validate_consistent_batches(B):
    for key, change in [("tiny", {}), ("ragged", dict(n_users=40)), ("uniform", dict(n_users=5))]:
        cfg = SI.scaled(SI.get_config(key), **change)
        announce("validate", key)
        db = B.DeviceBatch(SI.make_inputs(cfg), DEV)
        assert B.validate_batch(db) == 0


def test_validate_names_each_violation(B):
    cfg, W, inp = small_batch()
    db = B.DeviceBatch(inp, DEV)
    L = inp.L.astype(np.int64)
    announce("validate-violations", L.tolist(), inp.m.tolist())
    # a user longer than the stated max_L (host check still passes: max_L * n_users >= total_L)
    db.c.max_L = int(max(int(np.ceil(inp.total_L / inp.n_users)), L.min()))
    if db.c.max_L < L.max():
        assert B.validate_batch(db) & 8
    db.c.max_L = int(L.max())
    # decreasing history offsets, start and end intact
    h = inp.hist_off.copy()
    h[1], h[2] = h[2], h[1]
    db.hist_off.copy_(torch.from_numpy(h))
    assert B.validate_batch(db) & 4
    # a last offset that is not total_T
    db.hist_off.copy_(torch.from_numpy(inp.hist_off))
    t = inp.tgt_off.copy()
    t[-1] += 1
    db.tgt_off.copy_(torch.from_numpy(t))
    assert B.validate_batch(db) & 2
    db.tgt_off.copy_(torch.from_numpy(inp.tgt_off))
    assert B.validate_batch(db) == 0
    # an empty history with targets is flagged (allowed: its targets get NaN); user 1 takes user
    # 0's rows, so max_L must cover both
    db.c.max_L = int(inp.total_L)
    h = inp.hist_off.copy()
    h[1] = 0
    db.hist_off.copy_(torch.from_numpy(h))
    assert B.validate_batch(db) == 32


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_over_inconsistent_batch_is_all_nan(B, dtype):
    cfg, W, inp = small_batch()
    cfg = SI.scaled(cfg, dtype=dtype)
    W = SI.make_weights(cfg)
    inp = SI.make_inputs(cfg)
    announce("inconsistent-batch", dtype, inp.L.tolist())
    dw = B.DeviceWeights(W, cfg.dtype, DEV)
    db = B.DeviceBatch(inp, DEV)
    dims = B.dims_for(cfg)
    # history offsets out of order: user 1 appears to have a negative length
    h = inp.hist_off.copy()
    h[1], h[2] = h[2], h[1]
    db.hist_off.copy_(torch.from_numpy(h))
    Z = B.stca_forward(dims, dw, db)
    torch.cuda.synchronize()
    assert torch.isnan(Z).all()
    # restored offsets: the same buffers give the oracle's result again
    db.hist_off.copy_(torch.from_numpy(inp.hist_off))
    Z = B.stca_forward(dims, dw, db)
    torch.cuda.synchronize()
    assert row_rel(Z.cpu().numpy(), O.forward_batch(inp, W)) <= tol_for(cfg)


def test_forward_on_side_stream_keeps_its_workspace(B):
    cfg = SI.scaled(SI.get_config("ragged"), n_users=64)
    announce("side-stream", cfg.key, 64)
    W = SI.make_weights(cfg)
    inp = SI.make_inputs(cfg)
    dw = B.DeviceWeights(W, cfg.dtype, DEV)
    db = B.DeviceBatch(inp, DEV)
    dims = B.dims_for(cfg)
    ref = B.stca_forward(dims, dw, db)
    torch.cuda.synchronize()
    nbytes = B.forward_workspace_size(dims, db.c)
    side = torch.cuda.Stream()
    for _ in range(3):
        Z = B.stca_forward(dims, dw, db, stream=side)   # workspace allocated inside, dropped on return
        junk = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV)   # current stream
        junk.fill_(0xA5)
        side.synchronize()
        torch.cuda.synchronize()
        assert torch.equal(Z, ref)
        del junk
