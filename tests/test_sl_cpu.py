"""The stochastic-length planner of libstca (host code, no GPU) against ``oracle.sl``.

The plan is integer work taken from float64 draws in the same operation order on both sides,
so lengths and offsets must agree exactly.  Argument checks return STCA_E_ARG (-1).
"""
import ctypes

import numpy as np
import pytest

import stca_inputs as SI
from oracle import sl
from target_cross_attention_amd import binding as B

CASES = [  # alpha, L_min, L_max, L_avg, L_infer, n_users, history lengths
    (0.02, 8, 10000, 2000, 10000, 1024, ("fixed", 10000)),
    (0.02, 8, 10000, 2000, 10000, 300, ("uniform", 1, 20000)),
    (0.5, 64, 4096, 1024, 3000, 77, ("uniform", 0, 5000)),
    (2.0, 512, 10000, 2500, 10000, 64, ("fixed", 10000)),
    (5.0, 8, 2048, 256, 2048, 1, ("fixed", 100)),
]


def _lengths(rng, n, spec):
    if spec[0] == "fixed":
        return np.full(n, spec[1], np.int64)
    return rng.integers(spec[1], spec[2] + 1, n).astype(np.int64)


@pytest.mark.parametrize("case", CASES, ids=[f"a{c[0]}-B{c[5]}" for c in CASES])
def test_plan_matches_oracle(case):
    alpha, L_min, L_max, L_avg, L_infer, n, spec = case
    prm = B.SlParams(L_min, L_max, L_avg, L_infer)
    beta = B.sl_beta(prm, alpha)
    assert beta == pytest.approx(sl.beta_param(alpha, L_min, L_max, L_avg), rel=1e-15)
    s, order = SI.make_sl_draws(SI.get_config("dense10k"), n, alpha, sl.beta_param(alpha, L_min, L_max, L_avg))
    full_len = _lengths(np.random.default_rng(n), n, spec)
    L, off = B.sl_plan(prm, full_len, s, order)
    Lr, offr = sl.plan(full_len, s, order, L_min, L_max, L_avg, L_infer)
    assert np.array_equal(L, Lr) and np.array_equal(off, offr)
    assert off[-1] <= n * L_avg


def test_plan_with_forced_truncation_matches_oracle():
    """Draws near 1 overshoot the budget, so the truncation pass does real work."""
    rng = np.random.default_rng(9)
    n = 200
    s = rng.uniform(0.7, 1.0, n)
    order = rng.permutation(n).astype(np.int32)
    full_len = rng.integers(0, 12000, n)
    prm = B.SlParams(8, 10000, 2000, 10000)
    L, off = B.sl_plan(prm, full_len, s, order)
    Lr, offr = sl.plan(full_len, s, order, 8, 10000, 2000, 10000)
    assert np.array_equal(L, Lr) and np.array_equal(off, offr)
    assert off[-1] == n * 2000


def test_plan_argument_checks():
    ok = B.SlParams(8, 10000, 2000, 10000)
    full_len, s, order = np.array([10, 20], np.int64), np.array([0.2, 0.9]), np.array([1, 0], np.int32)
    for bad in (B.SlParams(8, 10000, 10000, 10000), B.SlParams(0, 100, 50, 100), B.SlParams(8, 100, 50, 0)):
        with pytest.raises(B.StcaError):
            B.sl_plan(bad, full_len, s, order)
    with pytest.raises(B.StcaError):
        B.sl_plan(ok, full_len, s, np.array([0, 0], np.int32))      # not a permutation
    with pytest.raises(B.StcaError):
        B.sl_plan(ok, full_len, np.array([0.2, 1.5]), order)        # draw outside [0, 1]
    with pytest.raises(B.StcaError):
        B.sl_plan(ok, np.array([10, -1], np.int64), s, order)       # negative history length
    with pytest.raises(B.StcaError):
        B.sl_beta(ok, 0.0)
    L, off = B.sl_plan(ok, np.zeros(0, np.int64), np.zeros(0), np.zeros(0, np.int32))
    assert L.size == 0 and off.tolist() == [0]


def test_pack_argument_checks():
    FAKE = 0x7F0000000000   # 16-byte aligned placeholder device address (never dereferenced)
    dims = B.make_dims(256, 8, 3, 4)
    L = B.LIB
    ref = ctypes.byref
    assert L.stca_sl_pack(ref(dims), 2, FAKE, FAKE, 0, 0, FAKE, FAKE, None) == 0   # nothing to copy
    assert L.stca_sl_pack(ref(dims), 2, None, FAKE, 10, 8, FAKE, FAKE, None) == -1
    assert L.stca_sl_pack(ref(dims), 0, FAKE, FAKE, 10, 8, FAKE, FAKE, None) == -1
    assert L.stca_sl_pack(ref(dims), 2, FAKE, FAKE, 10, 11, FAKE, FAKE, None) == -1   # max_len > total
    assert L.stca_sl_pack(ref(dims), 2, FAKE, FAKE, 10, 8, FAKE + 8, FAKE, None) == -4
    bad = B.make_dims(256, 8, 3, 4)
    bad.d = 4                                                         # 8-byte bf16 rows
    assert L.stca_sl_pack(ref(bad), 2, FAKE, FAKE, 10, 8, FAKE, FAKE, None) == -2
