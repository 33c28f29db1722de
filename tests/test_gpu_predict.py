"""GPU parity of the prediction token (eq. (9) of the STCA notes page) through stca_predict.

End to end: stca_forward then stca_predict on the device, against the oracle's forward and
prediction_token on the same seeded inputs.  In isolation: stca_predict on a seeded random Z
(drawn here, on the host) against the oracle on the same Z.  Bars as for the forward: 2e-2 max
row-relative error for bf16 storage, 1e-4 for the fp32 debug path.
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


CASES = [
    ("tiny", dict()),
    ("uniform", dict(n_users=5)),
    ("ragged", dict(n_users=20)),
    ("stress20k", dict(n_users=2, length=("fixed", 700))),
]


@pytest.mark.parametrize("key,change", CASES, ids=[k for k, _ in CASES])
def test_forward_then_predict(B, key, change):
    cfg = SI.scaled(SI.get_config(key), **change)
    announce("predict", cfg.key, cfg.dtype, change)
    W = SI.make_weights(cfg)
    P = SI.make_predict_weights(cfg)
    inp = SI.make_inputs(cfg)
    dims = B.dims_for(cfg)
    db = B.DeviceBatch(inp, DEV)
    Z = B.stca_forward(dims, B.DeviceWeights(W, cfg.dtype, DEV), db)
    z = B.stca_predict(dims, B.DevicePredict(P, cfg.dtype, DEV), Z, db.xt)
    torch.cuda.synchronize()
    Zr = O.forward_batch(inp, W)
    zr = O.prediction_token(Zr, inp.as_f32(inp.xt), P.WZ, P.Wu, P.Wv, P.Wo)
    err = row_rel(z.cpu().numpy(), zr)
    print(f"  {key}: T={inp.total_T} err={err:.3e}", flush=True)
    assert np.all(np.isfinite(z.cpu().numpy()))
    assert err <= tol_for(cfg)


@pytest.mark.parametrize("dtype,T", [("f32", 1), ("f32", 333), ("bf16", 4097)])
def test_predict_isolated(B, dtype, T):
    cfg = SI.scaled(SI.get_config("ragged"), dtype=dtype, M=3)
    announce("predict-isolated", dtype, T)
    P = SI.make_predict_weights(cfg)
    rng = np.random.default_rng(7)
    Z = rng.standard_normal((T, cfg.M, cfg.d)).astype(np.float32)
    xt = rng.standard_normal((T, cfg.d)).astype(np.float32)
    if dtype == "bf16":
        xt = SI.bf16_round(xt)
    dims = B.dims_for(cfg)
    z = B.stca_predict(dims, B.DevicePredict(P, dtype, DEV), torch.from_numpy(Z).to(DEV),
                       B.to_device(xt, dtype, DEV))
    torch.cuda.synchronize()
    zr = O.prediction_token(Z, xt, P.WZ, P.Wu, P.Wv, P.Wo)
    err = row_rel(z.cpu().numpy(), zr)
    print(f"  T={T} err={err:.3e}", flush=True)
    assert err <= tol_for(cfg)
