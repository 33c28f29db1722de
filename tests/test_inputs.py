"""Seeded input generator: determinism, sampling consistency, layouts, bf16 rounding."""
import numpy as np
import torch

import stca_inputs as SI


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    a = rng.standard_normal(100000).astype(np.float32) * 10.0
    # add exact ties (low 16 bits = 0x8000) on both parities
    ties = (np.arange(64, dtype=np.uint32) << 16 | 0x8000 | 0x3F800000).view(np.float32)
    a = np.concatenate([a, ties, -ties])
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(SI.bf16_bits(a), ref)
    assert np.array_equal(SI.bf16_round(SI.bf16_round(a)), SI.bf16_round(a))


def test_generation_is_deterministic_and_sample_consistent():
    cfg = SI.scaled(SI.get_config("ragged"), n_users=40, d=32)
    full = SI.make_inputs(cfg)
    again = SI.make_inputs(cfg)
    assert np.array_equal(full.X, again.X) and np.array_equal(full.xt, again.xt)
    sample = SI.make_inputs(cfg, users=[3, 17, 39])
    for j, u in enumerate([3, 17, 39]):
        assert np.array_equal(sample.user_X(j), full.user_X(u))
        assert np.array_equal(sample.user_xt(j), full.user_xt(u))
    assert full.X.dtype == np.uint16        # bf16 storage


def test_ragged_layout_statistics():
    cfg = SI.get_config("ragged")
    L, m = SI.batch_layout(cfg)
    assert L.min() >= 64 and L.max() <= 10000
    assert 1700 < L.mean() < 2300          # log-normal, median 1500, unclipped mean 2000
    assert 1200 < np.median(L) < 1800
    assert m.min() >= 1 and 5.0 < m.mean() < 7.0
    off = SI.offsets(L)
    assert off[0] == 0 and off[-1] == L.sum() and np.all(np.diff(off) == L)


def test_dense_duplicates_are_nearby_copies():
    cfg = SI.scaled(SI.get_config("dense10k"), n_users=2, d=16)
    X = SI.user_history(cfg, 0, 10000)
    same_as_prev = np.zeros(len(X), bool)
    for k in (1, 2, 3):
        same_as_prev[k:] |= np.all(X[k:] == X[:-k], axis=1)
    frac = same_as_prev.mean()
    assert 0.08 < frac < 0.13, frac


def test_weight_shapes_and_scale():
    cfg = SI.get_config("ragged")
    W = SI.make_weights(cfg)
    d, rd = cfg.d, cfg.r * cfg.d
    assert W.Wu[0].shape == (d, rd) and W.Wv[2].shape == (d, rd) and W.Wo[1].shape == (rd, d)
    assert W.WC[0] is None and W.WC[1].shape == (2 * d, d) and W.WC[2].shape == (3 * d, d)
    assert abs(W.Wo[0].std() * np.sqrt(rd) - 1.0) < 0.02
    assert abs(W.WC[2].std() * np.sqrt(3 * d) - 1.0) < 0.02
    assert W.qWu[1] is W.Wu[1]
    assert np.array_equal(SI.bf16_round(W.WQ[0]), W.WQ[0])


def test_item_ids_follow_the_repeats():
    """Rows sharing an item ID are bitwise copies; asking for IDs changes no draw."""
    cfg = SI.scaled(SI.get_config("dense10k"), n_users=3)
    a = SI.make_inputs(cfg)
    b = SI.make_inputs(cfg, with_ids=True)
    assert a.item_id is None and np.array_equal(a.X, b.X) and np.array_equal(a.xt, b.xt)
    ids = b.item_id
    assert ids.shape == (b.total_L,)
    first = {}
    for p, i in enumerate(ids.tolist()):
        first.setdefault(i, p)
        assert np.array_equal(b.X[p], b.X[first[i]])
    assert 0.05 < 1 - len(first) / len(ids) < 0.15        # ~10% repeats in this workload
    u = SI.make_inputs(SI.get_config("uniform"), users=[0, 1], with_ids=True)
    assert len(set(u.item_id.tolist())) == u.total_L       # no repeats: all IDs distinct
