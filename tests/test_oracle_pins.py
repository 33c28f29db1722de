"""Pins for the CPU oracle: each checks it against something other than itself.

* library routines (torch CPU float64): SiLU, LayerNorm, scaled dot-product attention;
* closed forms: LayerNorm moments, single-token history, identical tokens;
* invariants the pages state: eq. (13) equals eq. (12) (associativity), exact softmax
  rows summing to one, request-level batching changes only the layout, each query sees
  only its own user's segment;
* brute force: an independent pure-Python scalar-loop forward at tiny sizes;
* planted mistakes: plausible bugs injected into the oracle must each fail a pin.
"""
import numpy as np
import pytest
import torch

from oracle import brute
from oracle import stca as O
import stca_inputs as SI

torch.set_default_dtype(torch.float64)


def rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def tiny_cfg(d=16, h=4, M=3, r=2, n_users=2, L=6, m=3, dtype="f32"):
    return SI.scaled(SI.get_config("tiny"), d=d, h=h, M=M, r=r, n_users=n_users,
                     length=("fixed", L), targets=("fixed", m), dtype=dtype)


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ----------------------------------------------------------------------------
# eq. (1) and the LayerNorm of eq. (2) against library routines and closed forms
# ----------------------------------------------------------------------------
def test_silu_matches_torch():
    g = np.linspace(-30, 30, 4001)
    ref = torch.nn.functional.silu(torch.tensor(g)).numpy()
    assert np.max(np.abs(O.silu(g) - ref)) < 1e-14


def test_layer_norm_matches_torch():
    rng = np.random.default_rng(1)
    y = rand(rng, 7, 33, scale=3.0) + 5.0
    g, b = rand(rng, 33), rand(rng, 33)
    ref = torch.nn.functional.layer_norm(torch.tensor(y), (33,), torch.tensor(g), torch.tensor(b), 1e-5).numpy()
    assert rel(O.layer_norm(y, g, b, 1e-5), ref) < 1e-13


def test_layer_norm_closed_forms():
    rng = np.random.default_rng(2)
    d = 64
    y = rand(rng, 5, d, scale=0.01)           # small variance: eps matters
    out = O.layer_norm(y, np.ones(d), np.zeros(d), 1e-5)
    var = y.var(axis=1)
    assert np.max(np.abs(out.mean(axis=1))) < 1e-14
    assert rel((out ** 2).sum(axis=1), d * var / (var + 1e-5)) < 1e-12
    # a constant row normalises to beta exactly
    beta = rand(rng, d)
    const = O.layer_norm(np.full((1, d), 3.25), rand(rng, d), beta, 1e-5)
    assert np.array_equal(const[0], beta)


def test_swiglu_ffn_matches_brute_rows():
    rng = np.random.default_rng(3)
    d, rd = 8, 16
    x = rand(rng, 4, d)
    Wu, Wv, Wo = rand(rng, d, rd), rand(rng, d, rd), rand(rng, rd, d)
    ref = np.array([brute.ffn_row(list(row), Wu.tolist(), Wv.tolist(), Wo.tolist()) for row in x])
    assert rel(O.swiglu_ffn(x, Wu, Wv, Wo), ref) < 1e-13


# ----------------------------------------------------------------------------
# eqs. (4)-(6), (12), (13)
# ----------------------------------------------------------------------------
def _layer(rng, d):
    return [rand(rng, d, d, scale=d ** -0.5) for _ in range(4)]


def test_attention_heads_match_sdpa():
    """With W_O = I, o is the concatenation of the heads; each head is textbook SDPA."""
    rng = np.random.default_rng(4)
    d, h, L, m = 32, 4, 37, 5
    dh = d // h
    q, Xt = rand(rng, m, d), rand(rng, L, d)
    WQ, WK, WV, _ = _layer(rng, d)
    for fn in (O.attend_standard, O.attend_reordered):
        o = fn(q, Xt, WQ, WK, WV, np.eye(d), h)[0]
        for j in range(h):
            c = slice(j * dh, (j + 1) * dh)
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.tensor(q @ WQ[:, c])[None], torch.tensor(Xt @ WK[:, c])[None],
                torch.tensor(Xt @ WV[:, c])[None])[0].numpy()
            assert rel(o[:, c], ref) < 1e-12


def test_reordered_equals_standard():
    rng = np.random.default_rng(5)
    for d, h, L, m in [(64, 4, 256, 4), (128, 8, 97, 3), (256, 8, 50, 2)]:
        q, Xt = rand(rng, m, d), rand(rng, L, d)
        WQ, WK, WV, WO = _layer(rng, d)
        o_std, a_std = O.attend_standard(q, Xt, WQ, WK, WV, WO, h)
        o_re, a_re, _ = O.attend_reordered(q, Xt, WQ, WK, WV, WO, h)
        assert rel(o_re, o_std) < 1e-12
        assert np.max(np.abs(a_re - a_std)) < 1e-13


def test_alpha_is_a_distribution():
    rng = np.random.default_rng(6)
    q, Xt = rand(rng, 3, 64, scale=4.0), rand(rng, 500, 64, scale=4.0)
    _, alpha, _ = O.attend_reordered(q, Xt, *_layer(rng, 64), 8)
    assert np.all(alpha >= 0)
    assert np.max(np.abs(alpha.sum(axis=-1) - 1.0)) < 1e-12


def test_single_token_history():
    """L = 1: alpha = [1], so o = x~_1 W_V W_O for every query."""
    rng = np.random.default_rng(7)
    d, h = 32, 4
    x1 = rand(rng, 1, d)
    WQ, WK, WV, WO = _layer(rng, d)
    o, alpha, _ = O.attend_reordered(rand(rng, 6, d), x1, WQ, WK, WV, WO, h)
    assert np.all(alpha == 1.0)
    assert rel(o, np.repeat(x1 @ WV @ WO, 6, axis=0)) < 1e-13


def test_identical_tokens_and_repeated_history():
    rng = np.random.default_rng(8)
    d, h = 32, 4
    W4 = _layer(rng, d)
    q = rand(rng, 3, d)
    x1 = rand(rng, 1, d)
    o1 = O.attend_reordered(q, x1, *W4, h)[0]
    same = np.repeat(x1, 50, axis=0)
    o, alpha, _ = O.attend_reordered(q, same, *W4, h)
    assert np.max(np.abs(alpha - 1.0 / 50)) < 1e-15
    assert rel(o, o1) < 1e-13
    # repeating a whole history k times leaves the output unchanged
    Xt = rand(rng, 20, d)
    base = O.attend_reordered(q, Xt, *W4, h)[0]
    assert rel(O.attend_reordered(q, np.tile(Xt, (3, 1)), *W4, h)[0], base) < 1e-12


def test_scores_use_head_width_scale():
    """With a single head the textbook routine's default scale 1/sqrt(d) coincides with 1/sqrt(d_h)."""
    rng = np.random.default_rng(9)
    d = 16
    q, Xt = rand(rng, 2, d, scale=3.0), rand(rng, 11, d, scale=3.0)
    WQ, WK, WV, _ = _layer(rng, d)
    o = O.attend_reordered(q, Xt, WQ, WK, WV, np.eye(d), 1)[0]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q @ WQ)[None], torch.tensor(Xt @ WK)[None], torch.tensor(Xt @ WV)[None])[0].numpy()
    assert rel(o, ref) < 1e-12


# ----------------------------------------------------------------------------
# eqs. (1)-(8) against the brute-force scalar loops
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("query_ln,separate,random_ln", [(False, False, False), (True, True, True),
                                                         (False, True, True)])
def test_forward_matches_brute_force(query_ln, separate, random_ln):
    cfg = tiny_cfg(d=16, h=4, M=3, r=2, n_users=2, L=7, m=2)
    W = SI.make_weights(cfg, random_ln=random_ln, separate_query_ffn=separate)
    inp = SI.make_inputs(cfg)
    for k in range(inp.n_users):
        Z = O.forward_user(inp.user_X(k), inp.user_xt(k), W, cfg.h, cfg.M, query_ln)
        Zb = np.array(brute.forward_user(inp.user_X(k), inp.user_xt(k), W, cfg.h, cfg.M, query_ln))
        assert Z.shape == Zb.shape == (2, 3, 16)
        assert rel(Z, Zb) < 1e-12


def test_forward_matches_brute_force_shapes():
    for (d, h, M, r, L, m) in [(8, 2, 1, 1, 1, 1), (12, 3, 2, 2, 8, 3), (16, 1, 2, 1, 5, 2)]:
        cfg = tiny_cfg(d=d, h=h, M=M, r=r, n_users=1, L=L, m=m)
        W = SI.make_weights(cfg, random_ln=True)
        inp = SI.make_inputs(cfg)
        Z = O.forward_user(inp.user_X(0), inp.user_xt(0), W, h, M)
        Zb = np.array(brute.forward_user(inp.user_X(0), inp.user_xt(0), W, h, M))
        assert rel(Z, Zb) < 1e-12


# ----------------------------------------------------------------------------
# request level batching: a layout change only
# ----------------------------------------------------------------------------
def test_rlb_batch_equals_single_user_calls_and_permutations():
    cfg = SI.scaled(SI.get_config("ragged"), d=32, h=4, M=2, r=2, n_users=5,
                    length=("lognormal", 12.0, 16.0, 1, 40))
    W = SI.make_weights(cfg)
    inp = SI.make_inputs(cfg)
    Z = O.forward_batch(inp, W)
    assert Z.shape == (inp.total_T, 2, 32)
    for k in range(inp.n_users):
        one = SI.make_inputs(cfg, users=[k])
        Zk = O.forward_batch(one, W)
        assert np.array_equal(Zk, Z[inp.tgt_off[k]:inp.tgt_off[k + 1]])
    # permuting a user's history tokens leaves its outputs unchanged (no positional term)
    X0, xt0 = inp.user_X(0), inp.user_xt(0)
    perm = np.random.default_rng(0).permutation(len(X0))
    assert rel(O.forward_user(X0[perm], xt0, W, cfg.h), O.forward_user(X0, xt0, W, cfg.h)) < 1e-12
    # permuting targets permutes output rows
    tp = np.arange(len(xt0))[::-1]
    assert rel(O.forward_user(X0, xt0[tp], W, cfg.h), O.forward_user(X0, xt0, W, cfg.h)[tp]) < 1e-13


def test_zero_target_user_and_empty_history():
    cfg = tiny_cfg(n_users=1, L=4, m=2)
    W = SI.make_weights(cfg)
    inp = SI.make_inputs(cfg)
    Z = O.forward_user(inp.user_X(0), np.zeros((0, cfg.d)), W, cfg.h)
    assert Z.shape == (0, cfg.M, cfg.d)
    with pytest.raises(ValueError):
        O.forward_user(np.zeros((0, cfg.d)), inp.user_xt(0), W, cfg.h)


# ----------------------------------------------------------------------------
# planted mistakes: each must be caught by one of the pins above
# ----------------------------------------------------------------------------
def _pins_fail(monkeypatch, name, fn):
    monkeypatch.setattr(O, name, fn)
    failures = 0
    for test in (test_attention_heads_match_sdpa, test_reordered_equals_standard,
                 test_layer_norm_matches_torch, test_silu_matches_torch, test_single_token_history,
                 lambda: test_forward_matches_brute_force(True, True, True),
                 lambda: test_forward_matches_brute_force(False, False, False)):
        try:
            test()
        except AssertionError:
            failures += 1
    monkeypatch.undo()
    return failures


def test_planted_mistakes_are_caught(monkeypatch):
    orig_attend = O.attend_reordered
    orig_update = O.update_query
    orig_ln = O.layer_norm
    orig_silu = O.silu

    def wrong_scale(q, Xt, WQ, WK, WV, WO, h):     # 1/sqrt(d) instead of 1/sqrt(d_h)
        return orig_attend(q * np.sqrt(1.0 / h), Xt, WQ, WK, WV, WO, h)

    def transposed_wk(q, Xt, WQ, WK, WV, WO, h):
        return orig_attend(q, Xt, WQ, WK.T, WV, WO, h)

    def concat_reversed(o_prev, xt, WC, Wu, Wv, Wo, gamma=None, beta=None, query_ln=False, eps=1e-5):
        # x_t placed first in the concatenation instead of last
        c = np.concatenate([np.asarray(xt, np.float64)] + [np.asarray(o, np.float64) for o in o_prev], 1) @ WC
        y = O.swiglu_ffn(c, Wu, Wv, Wo)
        return O.layer_norm(y, gamma, beta, eps) if query_ln else y

    def unbiased_ln(y, gamma, beta, eps=1e-5):
        y = np.asarray(y, np.float64)
        n = y.shape[-1]
        return orig_ln(y, gamma, beta, eps) * np.sqrt((n - 1) / n)

    def silu_sign(g):
        return np.asarray(g) / (1.0 + np.exp(np.asarray(g)))

    def dropped_wo(q, Xt, WQ, WK, WV, WO, h):
        o, a, ab = orig_attend(q, Xt, WQ, WK, WV, np.eye(WO.shape[0]), h)
        return o, a, ab

    for name, fn in [("attend_reordered", wrong_scale), ("attend_reordered", transposed_wk),
                     ("update_query", concat_reversed), ("layer_norm", unbiased_ln),
                     ("silu", silu_sign), ("attend_reordered", dropped_wo)]:
        assert _pins_fail(monkeypatch, name, fn) >= 1, f"planted mistake via {name}/{fn.__name__} not caught"
    assert O.attend_reordered is orig_attend and O.update_query is orig_update
    assert O.layer_norm is orig_ln and O.silu is orig_silu


# ----------------------------------------------------------------------------
# eq. (9): the prediction token
# ----------------------------------------------------------------------------
def _swiglu_torch(x, Wu, Wv, Wo):
    x, Wu, Wv, Wo = (torch.as_tensor(np.asarray(a, np.float64)) for a in (x, Wu, Wv, Wo))
    return ((x @ Wu) * torch.nn.functional.silu(x @ Wv) @ Wo).numpy()


def test_prediction_token_matches_brute_force():
    cfg = tiny_cfg(d=12, h=3, M=2, r=2, n_users=2, L=5, m=3)
    W = SI.make_weights(cfg, random_ln=True)
    P = SI.make_predict_weights(cfg)
    inp = SI.make_inputs(cfg)
    Z = O.forward_batch(inp, W)
    xt = inp.as_f32(inp.xt)
    z = O.prediction_token(Z, xt, P.WZ, P.Wu, P.Wv, P.Wo)
    zb = np.array(brute.prediction_token(Z.tolist(), xt, P.WZ, P.Wu, P.Wv, P.Wo))
    assert z.shape == zb.shape == (inp.total_T, cfg.d)
    assert rel(z, zb) < 1e-12


def test_prediction_token_block_order():
    """W_Z selecting one block of the concatenation reduces eq. (9) to the FFN of that block."""
    rng = np.random.default_rng(3)
    m, M, d, r = 4, 3, 8, 2
    Z, xt = rand(rng, m, M, d), rand(rng, m, d)
    Wu, Wv, Wo = rand(rng, d, r * d, scale=0.3), rand(rng, d, r * d, scale=0.3), rand(rng, r * d, d, scale=0.3)
    for blk in range(M + 1):
        WZ = np.zeros(((M + 1) * d, d))
        WZ[blk * d:(blk + 1) * d] = np.eye(d)
        src = xt if blk == M else Z[:, blk, :]
        assert rel(O.prediction_token(Z, xt, WZ, Wu, Wv, Wo), _swiglu_torch(src, Wu, Wv, Wo)) < 1e-13


def test_prediction_token_planted_mistakes(monkeypatch):
    orig = O.prediction_token

    def reversed_concat(Z, xt, WZ, Wu, Wv, Wo):
        Z = np.asarray(Z, np.float64)
        blocks = [np.asarray(xt, np.float64)] + [Z[:, i, :] for i in range(Z.shape[1])]
        return O.swiglu_ffn(np.concatenate(blocks, axis=1) @ WZ, Wu, Wv, Wo)

    def gate_on_up(Z, xt, WZ, Wu, Wv, Wo):   # SiLU applied to the W_u branch instead of W_v
        return orig(Z, xt, WZ, Wv, Wu, Wo)

    for fn in (reversed_concat, gate_on_up):
        monkeypatch.setattr(O, "prediction_token", fn)
        caught = 0
        for test in (test_prediction_token_matches_brute_force, test_prediction_token_block_order):
            try:
                test()
            except AssertionError:
                caught += 1
        monkeypatch.undo()
        assert caught >= 1, fn.__name__
    assert O.prediction_token is orig
