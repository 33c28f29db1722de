"""Pins for the stochastic-length batch oracle (``oracle.sl``): closed forms and library routines
for eqs. (15)-(17), brute force for the integer steps, and planted mistakes that must fail them.
"""
import numpy as np
import pytest
from scipy import stats

import stca_inputs as SI
from oracle import sl

PARAMS = [(0.02, 8, 10000, 2000), (0.5, 64, 4096, 1024), (2.0, 512, 10000, 2500), (1.0, 8, 2048, 512)]


@pytest.mark.parametrize("alpha,L_min,L_max,L_avg", PARAMS)
def test_beta_mean_constraint(alpha, L_min, L_max, L_avg):
    """eq. (17) puts the mean of eq. (16) at L_avg: closed form and the library's Beta mean."""
    beta = sl.beta_param(alpha, L_min, L_max, L_avg)
    mean_s = stats.beta(alpha, beta).mean()
    assert abs(L_min + mean_s * (L_max - L_min) - L_avg) < 1e-9 * L_avg
    assert sl.sequence_sparsity(L_avg, L_max) == pytest.approx(L_avg / L_max)


def test_sampled_lengths_have_the_target_mean():
    """Monte Carlo over the seeded draws: mean length within sampling error (+ alignment) of L_avg."""
    cfg = SI.get_config("dense10k")
    for alpha, L_min, L_max, L_avg in PARAMS:
        beta = sl.beta_param(alpha, L_min, L_max, L_avg)
        s, _ = SI.make_sl_draws(cfg, 200_000, alpha, beta)
        L = sl.train_lengths(s, L_min, L_max)
        sd = stats.beta(alpha, beta).std() * (L_max - L_min) / np.sqrt(len(s))
        assert abs(L.mean() - L_avg) < 5 * sd + 4.0, (alpha, L.mean())
        assert abs(L.mean() / L_max - sl.sequence_sparsity(L_avg, L_max)) < (5 * sd + 4.0) / L_max


def test_alignment_to_8():
    L_raw = np.array([8.0, 11.9, 12.0, 12.1, 19.99, 20.0, 9999.0, 10003.0, 3.0, 0.0])
    L = sl.align8(L_raw, 8, 10000)
    assert np.all(L % 8 == 0)
    assert list(L) == [8, 8, 16, 16, 16, 24, 10000, 10000, 8, 8]
    inner = np.random.default_rng(1).uniform(8, 10000, 1000)
    Li = sl.align8(inner, 8, 10000)
    assert np.all(np.abs(Li - inner) <= 4.0)


def test_allocation_hits_the_budget_exactly():
    rng = np.random.default_rng(2)
    for _ in range(50):
        B = int(rng.integers(1, 40))
        L = 8 * rng.integers(1, 300, B)
        order = rng.permutation(B)
        budget = 8 * int(rng.integers(B, 300 * B))
        out = sl.allocate(L, budget, order, 8)
        assert np.all(out >= 8) and np.all(out <= L)
        if L.sum() <= budget:
            assert np.array_equal(out, L)
        else:
            assert out.sum() == budget
            # sequences are cut in the given order: one cut later in the order implies every
            # earlier sequence was already at the floor
            cut = np.nonzero(out < L)[0]
            pos = {int(u): i for i, u in enumerate(order)}
            last = max(pos[int(u)] for u in cut)
            assert all(out[order[i]] == 8 for i in range(last))


def test_allocation_absorbs_unaligned_excess():
    """Lengths capped by short histories are not multiples of 8; the budget is still met exactly."""
    L = np.array([8003, 8, 5, 4000, 17])
    out = sl.allocate(L, 5000, [3, 0, 1, 2, 4], 8)   # user 3 down to the floor, then user 0
    assert out.sum() == 5000 and out.tolist() == [4962, 8, 5, 8, 17]


def test_suffix_selection_and_packing_brute_force():
    rng = np.random.default_rng(3)
    full_len = rng.integers(1, 60, 9)
    full_off = np.concatenate([[0], np.cumsum(full_len)])
    X = rng.standard_normal((int(full_off[-1]), 5))
    L = np.array([min(int(rng.integers(0, 70)), int(n)) for n in full_len])
    packed, idx = sl.pack(X, full_off, L)
    want = []
    for u in range(len(L)):           # the last L[u] rows of user u, oldest first
        rows = list(range(int(full_off[u]), int(full_off[u + 1])))
        want += rows[len(rows) - int(L[u]):]
    assert idx.tolist() == want
    assert packed.shape == (int(L.sum()), 5) and np.array_equal(packed, X[want])


def test_plan_composition_and_rows_view():
    cfg = SI.get_config("dense10k")
    alpha, L_min, L_max, L_avg, L_infer = 0.02, 8, 10000, 2000, 10000
    B = 64
    rng = np.random.default_rng(4)
    full_len = rng.integers(50, 15000, B)
    s, order = SI.make_sl_draws(cfg, B, alpha, sl.beta_param(alpha, L_min, L_max, L_avg))
    L, off = sl.plan(full_len, s, order, L_min, L_max, L_avg, L_infer)
    assert np.all(L <= np.minimum(full_len, L_infer)) and off[-1] == L.sum() <= B * L_avg
    assert np.all(np.diff(off) == L)
    view = sl.rows_view(off, L_avg)
    owner = np.repeat(np.arange(B), L)
    for r, (first, last) in enumerate(view):
        seg = owner[r * L_avg:(r + 1) * L_avg]
        assert first == seg.min() and last == seg.max()


def test_planted_mistakes_are_caught(monkeypatch):
    def prefix_rows(full_off, L):      # oldest rows instead of the temporal suffix
        full_off = np.asarray(full_off, np.int64)
        return np.concatenate([np.arange(full_off[u], full_off[u] + L[u]) for u in range(len(L))])

    def beta_inverted(alpha, L_min, L_max, L_avg):
        return alpha * (L_avg - L_min) / (L_max - L_avg)

    def align_floor(L_raw, L_min, L_max):
        lo, hi = 8 * -(-L_min // 8), 8 * (L_max // 8)
        return np.clip(8 * np.floor(np.asarray(L_raw, np.float64) / 8.0).astype(np.int64), lo, hi)

    for name, fn, test in [("suffix_rows", prefix_rows, test_suffix_selection_and_packing_brute_force),
                           ("beta_param", beta_inverted, lambda: test_beta_mean_constraint(*PARAMS[1])),
                           ("align8", align_floor, test_alignment_to_8)]:
        monkeypatch.setattr(sl, name, fn)
        with pytest.raises(AssertionError):
            test()
        monkeypatch.undo()
