"""Pins for the LITM oracle (``oracle.litm``): an independent union-find formulation of the
grouping, special cases that reduce to the identity or to one token per user, exact sum
invariants of the merge, user isolation, and planted mistakes that must fail them."""
import numpy as np
import pytest

from oracle import litm


def components(item_id, hist_off, T):
    """Groups as connected components: consecutive occurrences of an ID within a user that are at
    most T apart are joined (union-find), independent of the scan in ``litm.group_roots``."""
    n = len(item_id)
    parent = list(range(n))

    def find(x):
        while parent[x] != x:
            parent[x] = parent[parent[x]]
            x = parent[x]
        return x

    for u in range(len(hist_off) - 1):
        last = {}
        for p in range(int(hist_off[u]), int(hist_off[u + 1])):
            i = int(item_id[p])
            if i in last and p - last[i] <= T:
                ra, rb = find(last[i]), find(p)
                parent[max(ra, rb)] = min(ra, rb)
            last[i] = p
    return np.array([find(p) for p in range(n)], np.int64)


def random_case(rng, n_users=5, alphabet=6):
    L = rng.integers(1, 40, n_users)
    off = np.concatenate([[0], np.cumsum(L)]).astype(np.int64)
    ids = rng.integers(0, alphabet, int(off[-1])).astype(np.int64)
    return ids, off


@pytest.mark.parametrize("T", [0, 1, 2, 3, 5, 50])
def test_roots_match_union_find(T):
    rng = np.random.default_rng(11 + T)
    for _ in range(20):
        ids, off = random_case(rng)
        assert np.array_equal(litm.group_roots(ids, off, T), components(ids, off, T))


def test_plan_structure():
    rng = np.random.default_rng(5)
    ids, off = random_case(rng, n_users=7)
    mo, go, mem = litm.plan(ids, off, 3)
    root = components(ids, off, 3)
    assert sorted(mem.tolist()) == list(range(int(off[-1])))          # every token exactly once
    for u in range(len(off) - 1):
        firsts = [int(mem[go[g]]) for g in range(int(mo[u]), int(mo[u + 1]))]
        assert firsts == sorted(firsts)                                   # order of first occurrence
        assert len(set(root[off[u]:off[u + 1]])) == mo[u + 1] - mo[u]
        for g in range(int(mo[u]), int(mo[u + 1])):
            m = mem[go[g]:go[g + 1]]
            assert np.all(np.diff(m) > 0) and len(set(root[m])) == 1 and root[m[0]] == m[0]
            assert np.all((m >= off[u]) & (m < off[u + 1]))


def test_special_cases():
    off = np.array([0, 6, 10], np.int64)
    ids = np.array([1, 2, 3, 4, 5, 6, 7, 8, 9, 10], np.int64)
    for T in (0, 3, 100):                                  # all distinct: identity
        mo, go, mem = litm.plan(ids, off, T)
        assert mo.tolist() == [0, 6, 10] and np.array_equal(mem, np.arange(10)) and np.array_equal(go, np.arange(11))
    same = np.full(10, 7, np.int64)
    mo, go, mem = litm.plan(same, off, 1)                  # one ID, gaps of 1: one token per user
    assert mo.tolist() == [0, 1, 2] and go.tolist() == [0, 6, 10]
    mo, _, _ = litm.plan(same, off, 0)                     # T = 0 merges nothing
    assert mo.tolist() == [0, 6, 10]
    gap = np.array([5, 1, 2, 5, 3, 4, 9, 9, 9, 9], np.int64)  # the two 5s are 3 apart
    assert litm.plan(gap, off, 3)[0].tolist() == [0, 5, 6]
    assert litm.plan(gap, off, 2)[0].tolist() == [0, 6, 7]
    # chaining: 8 at 0, 3, 6 (gaps 3, 3) is one group at T = 3 though 0 and 6 are 6 apart
    chain = np.array([8, 1, 2, 8, 3, 4, 8, 9, 9, 9], np.int64)
    mo, go, mem = litm.plan(chain, np.array([0, 7, 10], np.int64), 3)
    assert mo.tolist() == [0, 5, 6] and mem[go[0]:go[1]].tolist() == [0, 3, 6]


def test_users_do_not_merge():
    off = np.array([0, 3, 6], np.int64)
    ids = np.array([1, 2, 4, 4, 2, 1], np.int64)           # 4 at rows 2 and 3, different users
    mo, _, _ = litm.plan(ids, off, 3)
    assert mo.tolist() == [0, 3, 6]


def test_merge_sums():
    rng = np.random.default_rng(9)
    ids, off = random_case(rng, n_users=4, alphabet=4)
    X = rng.standard_normal((int(off[-1]), 8))
    mo, go, mem = litm.plan(ids, off, 3)
    Y = litm.merge(X, go, mem)
    for u in range(len(off) - 1):                           # per-user column sums are preserved
        np.testing.assert_allclose(Y[mo[u]:mo[u + 1]].sum(0), X[off[u]:off[u + 1]].sum(0), rtol=1e-12, atol=1e-12)
    ident = np.arange(len(X) + 1)
    assert np.array_equal(litm.merge(X, ident, np.arange(len(X))), X)
    for g in range(len(go) - 1):                            # a merged row is its members' sum
        np.testing.assert_allclose(Y[g], X[mem[go[g]:go[g + 1]]].sum(0), rtol=1e-12)


def test_planted_mistakes_are_caught(monkeypatch):
    real = litm.group_roots

    def anchored(item_id, hist_off, T):      # distance to the group's first token instead of chaining
        root = np.arange(len(item_id), dtype=np.int64)
        for u in range(len(hist_off) - 1):
            a, b = int(hist_off[u]), int(hist_off[u + 1])
            for p in range(a, b):
                for q in range(p - 1, max(a, p - T) - 1, -1):
                    if item_id[q] == item_id[p] and p - root[q] <= T:
                        root[p] = root[q]
                        break
        return root

    def across_users(item_id, hist_off, T):  # ignores user boundaries
        return real(item_id, np.array([0, hist_off[-1]]), T)

    def strict(item_id, hist_off, T):        # gap < T instead of <= T
        return real(item_id, hist_off, T - 1)

    for fn in (anchored, across_users, strict):
        monkeypatch.setattr(litm, "group_roots", fn)
        with pytest.raises(AssertionError):
            test_roots_match_union_find(3)
            test_special_cases()
            test_users_do_not_merge()
        monkeypatch.undo()
