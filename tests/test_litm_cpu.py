"""The LITM planner of libstca (host code, no GPU) against ``oracle.litm``, and the argument
checks of both LITM calls (errors are returned before any launch).

Grouping is integer work, so merged offsets, group offsets and members must agree exactly."""
import ctypes

import numpy as np
import pytest

import stca_inputs as SI
from oracle import litm
from target_cross_attention_amd import binding as B


def _random(rng, n_users, alphabet, max_len=60):
    L = rng.integers(0, max_len, n_users)
    off = np.concatenate([[0], np.cumsum(L)]).astype(np.int64)
    return off, rng.integers(0, alphabet, int(off[-1])).astype(np.int64)


@pytest.mark.parametrize("T", [0, 1, 2, 3, 7, 1000])
def test_plan_matches_oracle_random(T):
    rng = np.random.default_rng(100 + T)
    for n_users, alphabet in [(1, 2), (9, 3), (30, 8), (5, 1000)]:
        off, ids = _random(rng, n_users, alphabet)
        got = B.litm_plan(off, ids, T)
        want = litm.plan(ids, off, T)
        for a, b in zip(got, want):
            assert np.array_equal(a, b)


def test_plan_matches_oracle_on_workload_ids():
    inp = SI.make_inputs(SI.scaled(SI.get_config("dense10k"), n_users=6), with_ids=True)
    for T in (1, 3):
        got = B.litm_plan(inp.hist_off, inp.item_id, T)
        want = litm.plan(inp.item_id, inp.hist_off, T)
        for a, b in zip(got, want):
            assert np.array_equal(a, b)
        assert got[0][-1] < inp.total_L                      # the repeats do merge


def test_empty_batches():
    mo, go, mem = B.litm_plan(np.zeros(4, np.int64), np.zeros(0, np.int64), 3)
    assert mo.tolist() == [0, 0, 0, 0] and go.tolist() == [0] and mem.size == 0
    mo, go, mem = B.litm_plan(np.array([0, 0, 3, 3]), np.array([5, 5, 5]), 3)
    assert mo.tolist() == [0, 0, 1, 1] and go.tolist() == [0, 3] and mem.tolist() == [0, 1, 2]


def test_plan_argument_checks():
    P = ctypes.c_void_p
    off = np.array([0, 2, 4], np.int64)
    ids = np.array([1, 1, 2, 2], np.int64)
    out = [np.zeros(3, np.int64), np.zeros(5, np.int64), np.zeros(4, np.int64)]
    ng = ctypes.c_int64()
    ptr = lambda a: a.ctypes.data_as(P)  # noqa: E731
    call = lambda n, o, i, T, mo, go, mem, g: B.LIB.stca_litm_plan(n, o, i, T, mo, go, mem, g)  # noqa: E731
    args = [2, ptr(off), ptr(ids), 3, ptr(out[0]), ptr(out[1]), ptr(out[2]), ctypes.byref(ng)]
    assert call(*args) == 0 and ng.value == 2
    assert call(-1, *args[1:]) == -1                            # n_users < 0
    assert call(args[0], args[1], args[2], -1, *args[4:]) == -1  # T < 0
    for k in (1, 2, 4, 5, 6):                                     # NULL pointers
        bad = list(args)
        bad[k] = None
        assert call(*bad) == -1, k
    assert call(2, ptr(np.array([0, 3, 2], np.int64)), *args[2:]) == -1   # decreasing offsets
    assert call(2, ptr(np.array([1, 2, 4], np.int64)), *args[2:]) == -1   # hist_off[0] != 0


def test_merge_argument_checks():
    dims = B.make_dims(256, 8, 1, 4)
    P = ctypes.c_void_p
    fake = P(1 << 20)                                             # never dereferenced: every case fails early
    m = B.LIB.stca_litm_merge
    assert m(None, 10, 5, fake, fake, fake, fake, None) == -1
    assert m(ctypes.byref(dims), 10, 0, None, None, None, None, None) == 0    # no groups: no-op
    assert m(ctypes.byref(dims), 10, 11, fake, fake, fake, fake, None) == -1  # more groups than rows
    assert m(ctypes.byref(dims), 10, -1, fake, fake, fake, fake, None) == -1
    assert m(ctypes.byref(dims), 10, 5, None, fake, fake, fake, None) == -1
    assert m(ctypes.byref(dims), 10, 5, fake, fake, P((1 << 20) + 8), fake, None) == -4  # misaligned rows
    bad = B.make_dims(96, 8, 1, 4)
    assert m(ctypes.byref(bad), 10, 5, fake, fake, fake, fake, None) == -2
