"""Graph replay of the forward (stca_forward_graph_create / stca_graph_launch) against the eager
stca_forward on the same buffers.  Both run the same kernels in the same order on the same data,
so every replay must reproduce the eager output bit for bit; the eager output itself is checked
against the oracle by the parity tests.  Replays are interleaved with other eager work, and the
inputs are rewritten in place between replays (a replay reads the buffers as they are then).  Also:
forwards on two streams at once, each with its own workspace, against the same forwards in turn."""
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


CASES = [("tiny", dict()), ("ragged", dict(n_users=5, length=("lognormal", 300.0, 400.0, 1, 1200))),
         ("stress20k", dict(n_users=1, length=("fixed", 700), targets=("fixed", 3)))]


@pytest.mark.parametrize("key,change", CASES, ids=[k for k, _ in CASES])
def test_graph_replays_match_eager(B, key, change):
    cfg = SI.scaled(SI.get_config(key), **change)
    announce("graph", cfg.key, change)
    W = SI.make_weights(cfg)
    inp = SI.make_inputs(cfg)
    dims = B.dims_for(cfg)
    dw = B.DeviceWeights(W, cfg.dtype, DEV)
    db = B.DeviceBatch(inp, DEV)
    eager = B.stca_forward(dims, dw, db).clone()
    torch.cuda.synchronize()
    assert row_rel(eager.cpu().numpy(), O.forward_batch(inp, W)) <= tol_for(cfg)
    graph = B.ForwardGraph(dims, dw, db)
    other = torch.empty_like(eager)
    for rep in range(3):
        graph.Z.fill_(float("nan"))
        B.stca_forward(dims, dw, db, Z=other)          # eager work between replays
        torch.cuda.synchronize()
        graph.launch()
        torch.cuda.synchronize()
        assert torch.equal(graph.Z, eager), rep
        assert torch.equal(other, eager)
    # new inputs in the same buffers: the next replay follows them
    inp2 = SI.make_inputs(SI.scaled(cfg, seed=cfg.seed + 1))
    if inp2.X.shape == inp.X.shape and inp2.xt.shape == inp.xt.shape:
        db.X.copy_(B.to_device(inp2.X, cfg.dtype, DEV))
        db.xt.copy_(B.to_device(inp2.xt, cfg.dtype, DEV))
        graph.launch()
        fresh = B.stca_forward(dims, dw, db)
        torch.cuda.synchronize()
        assert torch.equal(graph.Z, fresh)
        assert not torch.equal(fresh, eager)
    graph.close()


def test_graph_of_batch_without_targets(B):
    cfg = SI.get_config("tiny")
    inp = SI.make_inputs(cfg)
    import dataclasses
    inp = dataclasses.replace(inp, m=np.zeros(1, np.int64), tgt_off=SI.offsets(np.zeros(1, np.int64)),
                              xt=inp.xt[:0])
    announce("graph-no-targets")
    dims = B.dims_for(cfg)
    graph = B.ForwardGraph(dims, B.DeviceWeights(SI.make_weights(cfg), cfg.dtype, DEV), B.DeviceBatch(inp, DEV))
    graph.launch()
    torch.cuda.synchronize()
    graph.close()


def test_concurrent_forwards_on_two_streams(B):
    """The library keeps no mutable state: two forwards of different batches, each with its own
    workspace, enqueued on two streams at once give the same bits as one after the other."""
    announce("two-streams")
    cfg_a = SI.scaled(SI.get_config("ragged"), n_users=6, length=("lognormal", 400.0, 500.0, 1, 2000))
    cfg_b = SI.scaled(SI.get_config("uniform"), n_users=5, length=("fixed", 700))
    runs = []
    for cfg in (cfg_a, cfg_b):
        W = SI.make_weights(cfg)
        inp = SI.make_inputs(cfg)
        dims = B.dims_for(cfg)
        dw, db = B.DeviceWeights(W, cfg.dtype, DEV), B.DeviceBatch(inp, DEV)
        ref = B.stca_forward(dims, dw, db).clone()
        torch.cuda.synchronize()
        ws = B.workspace(B.forward_workspace_size(dims, db.c), DEV)
        runs.append((dims, dw, db, ref, ws))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.full_like(r[3], float("nan")) for r in runs]
    torch.cuda.synchronize()
    for _ in range(3):
        for (dims, dw, db, ref, ws), st, Z in zip(runs, streams, outs):
            with torch.cuda.stream(st):
                B.stca_forward(dims, dw, db, Z=Z, ws=ws, stream=st)
    torch.cuda.synchronize()
    for (dims, dw, db, ref, ws), Z in zip(runs, outs):
        assert torch.equal(Z, ref)
