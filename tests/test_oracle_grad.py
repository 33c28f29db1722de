"""Pins for the backward oracle (``oracle.grad``): central finite differences of L = sum(dZ * Z),
with Z from the forward oracle ``oracle.stca`` (not from grad's own forward), for every input
and weight slot, with and without the LayerNorm of eq. (7), with separate and with shared FFN
weights; batch linearity; and planted mistakes that the finite differences catch."""
import copy

import numpy as np
import pytest

import stca_inputs as SI
from oracle import grad as G
from oracle import stca as O

SLOTS = ["Wu", "Wv", "Wo", "gamma", "beta", "qWu", "qWv", "qWo", "qgamma", "qbeta", "WQ", "WK", "WV", "WO", "WC"]


def tiny_problem(separate=True, seed=0):
    cfg = SI.scaled(SI.get_config("tiny"), d=8, h=2, M=3, r=2, n_users=2, length=("fixed", 6),
                    targets=("fixed", 3), seed=seed)
    W = SI.make_weights(cfg, random_ln=True, separate_query_ffn=separate)
    W = copy.deepcopy(W)
    for name in SLOTS:                                     # float64 copies (aliases kept if shared)
        lst = getattr(W, name)
        memo = {}
        for i, a in enumerate(lst):
            if a is not None:
                lst[i] = memo.setdefault(id(a), np.asarray(a, np.float64))
    if not separate:                                       # re-alias query slots to history ones
        for i in range(cfg.M):
            W.qWu[i], W.qWv[i], W.qWo[i], W.qgamma[i], W.qbeta[i] = W.Wu[i], W.Wv[i], W.Wo[i], W.gamma[i], W.beta[i]
    inp = SI.make_inputs(cfg)
    X = inp.user_X(0).astype(np.float64)
    xt = inp.user_xt(0).astype(np.float64)
    dZ = np.random.default_rng(seed + 7).standard_normal((xt.shape[0], cfg.M, cfg.d))
    return cfg, W, X, xt, dZ


def loss(X, xt, W, cfg, dZ, query_ln):
    return float((O.forward_user(X, xt, W, cfg.h, cfg.M, query_ln=query_ln) * dZ).sum())


def fd(f, arr, idx, eps=1e-6):
    old = arr[idx]
    arr[idx] = old + eps
    up = f()
    arr[idx] = old - eps
    dn = f()
    arr[idx] = old
    return (up - dn) / (2 * eps)


def check_fd(query_ln, separate, n_pick=3):
    cfg, W, X, xt, dZ = tiny_problem(separate)
    g, dX, dxt = G.backward_user(X, xt, W, cfg.h, dZ, cfg.M, query_ln)
    f = lambda: loss(X, xt, W, cfg, dZ, query_ln)  # noqa: E731
    rng = np.random.default_rng(3)
    worst = 0.0

    def compare(arr, analytic):
        nonlocal worst
        for _ in range(n_pick):
            idx = tuple(rng.integers(0, s) for s in arr.shape)
            num = fd(f, arr, idx)
            err = abs(num - analytic[idx]) / max(1.0, abs(num))
            worst = max(worst, err)
            assert err < 1e-6, (idx, num, analytic[idx])

    compare(X, dX)
    compare(xt, dxt)
    for name in SLOTS:
        for i in range(cfg.M):
            arr = getattr(W, name)[i]
            if arr is None:
                continue
            an = getattr(g, name)[i]
            if not separate and name in ("Wu", "Wv", "Wo", "gamma", "beta"):
                an = an + getattr(g, "q" + name)[i]          # one shared array, two uses
            if not separate and name.startswith("q"):
                continue                                     # same arrays as checked above
            if not query_ln and name in ("qgamma", "qbeta") and i > 0:
                assert np.all(an == 0)                       # unused without eq. (7)'s LayerNorm
                continue
            compare(arr, an)
    return worst


@pytest.mark.parametrize("query_ln", [False, True])
def test_finite_differences_separate_weights(query_ln):
    check_fd(query_ln, separate=True)


def test_finite_differences_shared_weights():
    check_fd(False, separate=False)


def test_batch_is_sum_of_users():
    cfg = SI.scaled(SI.get_config("tiny"), d=8, h=2, M=2, r=2, n_users=3, length=("fixed", 5), targets=("fixed", 2))
    W = SI.make_weights(cfg, random_ln=True)
    inp = SI.make_inputs(cfg)
    dZ = np.random.default_rng(0).standard_normal((inp.total_T, cfg.M, cfg.d))
    gb = G.backward_batch(inp, W, dZ)
    acc = G.Grads.zeros(W, cfg.M)
    for k in range(inp.n_users):
        a, b = inp.tgt_off[k], inp.tgt_off[k + 1]
        _, dXk, dxtk = G.backward_user(inp.user_X(k), inp.user_xt(k), W, cfg.h, dZ[a:b], cfg.M, grads=acc)
        np.testing.assert_array_equal(gb.dX[inp.hist_off[k]:inp.hist_off[k + 1]], dXk)
        np.testing.assert_array_equal(gb.dxt[a:b], dxtk)
    for name in SLOTS:
        for x, y in zip(getattr(gb, name), getattr(acc, name)):
            if x is not None:
                np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-14)


def test_planted_mistakes_are_caught(monkeypatch):
    real_ffn, real_ln = G._ffn_bwd, G._ln_bwd

    def ffn_wrong_silu(dY, cache, Wu, Wv, Wo):               # SiLU derivative taken as sigma(g)
        x, A, Gt, H = cache
        s = G._sig(Gt)
        dH = dY @ Wo.T
        dA, dG = dH * Gt * s, dH * A * s
        return dA @ Wu.T + dG @ Wv.T, x.T @ dA, x.T @ dG, H.T @ dY

    def ln_no_centering(dout, cache, gamma):                # drops the mean term
        xh, rstd = cache
        dxh = dout * gamma
        return rstd * (dxh - xh * (dxh * xh).mean(axis=-1, keepdims=True)), (dout * xh).sum(0), dout.sum(0)

    for name, fn in [("_ffn_bwd", ffn_wrong_silu), ("_ln_bwd", ln_no_centering)]:
        monkeypatch.setattr(G, name, fn)
        with pytest.raises(AssertionError):
            check_fd(False, separate=True)
        monkeypatch.undo()
    assert G._ffn_bwd is real_ffn and G._ln_bwd is real_ln
