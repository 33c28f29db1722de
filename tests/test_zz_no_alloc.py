"""The allocation-free attention call (stca_attend_noalloc) against stca_attend.

Both run the same kernels; the first works in the library's fixed per-GPU scratch array, the second
in a caller workspace.  Two calls in a row, the second on a smaller batch (the array then still
holds the first call's values), must each reproduce stca_attend bit for bit, and so lie within the
bf16 bar of the oracle as stca_attend does.  A batch beyond the array's size is refused on the host.
"""
import numpy as np
import pytest

import stca_inputs as SI
from oracle import stca as O
from stca_testlib import announce, row_rel

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from target_cross_attention_amd import binding
    return binding


def _case(B, n_users, seed_users):
    cfg = SI.scaled(SI.get_config("ragged"), M=2)
    W = SI.make_weights(cfg)
    inp = SI.make_inputs(cfg, users=list(range(seed_users, seed_users + n_users)))
    dims = B.dims_for(cfg, attn_chunk=512)   # several chunks per long user: the combine runs too
    dw = B.DeviceWeights(W, cfg.dtype, DEV)
    db = B.DeviceBatch(inp, DEV)
    rng = np.random.default_rng(n_users)
    Xt = B.to_device(SI.bf16_round(rng.standard_normal((inp.total_L, cfg.d)).astype(np.float32)), "bf16", DEV)
    q = torch.from_numpy(rng.standard_normal((inp.total_T, cfg.d)).astype(np.float32)).to(DEV)
    return cfg, W, inp, dims, dw, db, Xt, q


@pytest.mark.parametrize("layer", [0, 1])
def test_noalloc_matches_attend_twice_second_smaller(B, layer):
    for n_users, first in ((48, 0), (9, 100)):
        cfg, W, inp, dims, dw, db, Xt, q = _case(B, n_users, first)
        announce("noalloc", layer, n_users, int(inp.total_L), int(inp.total_T))
        ref = B.stca_attend(dims, dw, layer, db, Xt, q)
        o = torch.full_like(ref, float("nan"))
        B.stca_attend_noalloc(dims, dw, layer, db, Xt, q, o)
        torch.cuda.synchronize()
        assert torch.equal(o, ref), f"{n_users} users: differs from stca_attend"
        # and the oracle's bar, on a few users
        Xh = Xt.float().cpu().numpy()
        qh = q.cpu().numpy()
        for k in (0, inp.n_users - 1):
            hs, ts = slice(inp.hist_off[k], inp.hist_off[k + 1]), slice(inp.tgt_off[k], inp.tgt_off[k + 1])
            want = O.attend_reordered(qh[ts], Xh[hs], W.WQ[layer], W.WK[layer], W.WV[layer], W.WO[layer], cfg.h)[0]
            assert row_rel(o[ts].cpu().numpy(), want) <= 2e-2


def test_noalloc_refuses_a_batch_beyond_its_scratch(B):
    cfg = SI.get_config("dense10k")
    dims = B.dims_for(cfg)
    L, m = SI.batch_layout(cfg)
    hoff = torch.from_numpy(SI.offsets(L)).to(DEV)
    toff = torch.from_numpy(SI.offsets(m)).to(DEV)
    c = B.batch_struct(cfg.n_users, hoff, toff, int(L.sum()), int(m.sum()), int(L.max()), int(m.max()))
    assert B.attend_workspace_size(dims, c) > 64 << 20
    W = B.DeviceWeights(SI.make_weights(SI.scaled(cfg, M=1)), cfg.dtype, DEV)
    dims1 = B.dims_for(SI.scaled(cfg, M=1))
    with pytest.raises(B.StcaError) as e:
        B.LIB and B._check(B.LIB.stca_attend_noalloc(B._ref(dims1), B._ref(W.c), 0, B._ref(c), 16, 16, 16, None),
                           "stca_attend_noalloc")
    assert e.value.status == -3
