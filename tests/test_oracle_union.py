"""Pins for the oracle's expert union (CPU only)."""

import itertools

import numpy as np

from oracle.union import expert_union


def _check(ids):
    ids = np.asarray(ids)
    R, k = ids.shape
    flat = ids.reshape(-1).tolist()
    union_ids, U, s2u, mask = expert_union(ids)
    ref = list(dict.fromkeys(flat))             # insertion-ordered dedup
    assert union_ids.tolist() == ref
    assert U == len(set(flat))
    assert k <= U <= min(k * R, max(flat) + 1)
    for t, e in enumerate(flat):
        assert union_ids[s2u[t]] == e
    for u, e in enumerate(ref):
        rows = {t // k for t, v in enumerate(flat) if v == e}
        assert int(mask[u]) == sum(1 << r for r in rows)


def test_union_exhaustive_tiny():
    n = 0
    for E in range(1, 6):
        for k in range(1, min(E, 3) + 1):
            row_choices = list(itertools.permutations(range(E), k))
            for R in range(1, 4):
                if len(row_choices) ** R > 4000:
                    combos = [tuple(row_choices[i] for i in np.random.default_rng(E * 100 + k * 10 + R)
                                    .integers(0, len(row_choices), R)) for _ in range(400)]
                else:
                    combos = itertools.product(row_choices, repeat=R)
                for rows in combos:
                    _check(np.array(rows))
                    n += 1
    assert n > 5000


def test_union_extremes():
    k = 8
    # all rows identical: U = k
    ids = np.tile(np.arange(k), (8, 1))
    u, U, s2u, mask = expert_union(ids)
    assert U == k and np.all(mask == 0xFF) and s2u.tolist() == list(range(k)) * 8
    # all distinct: U = 64 = k * rows (the one-block maximum)
    ids = np.arange(64).reshape(8, 8)
    u, U, s2u, mask = expert_union(ids)
    assert U == 64 and s2u.tolist() == list(range(64))
    assert [int(m) for m in mask] == [1 << (t // 8) for t in range(64)]
    # single row: union is the row itself, in slot order
    u, U, _, _ = expert_union(np.array([[5, 3, 9]]))
    assert u.tolist() == [5, 3, 9]


def test_union_random_large():
    rng = np.random.default_rng(21)
    for _ in range(300):
        E = int(rng.integers(8, 300))
        k = int(rng.integers(1, 9))
        R = int(rng.integers(1, 64 // k + 1))
        R = min(R, 8)
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(R)])
        _check(ids)


def test_union_past_64_ids():
    # 65..128 ids (up to 16 rows): the definition does not change with the
    # number of ids; checked against dict.fromkeys with ids repeated across the
    # 64th slot
    rng = np.random.default_rng(22)
    for _ in range(300):
        k = int(rng.integers(1, 17))
        R = int(rng.integers(max(1, 65 // k), 128 // k + 1)) if 128 // k >= 1 else 1
        R = max(1, min(R, 16))
        pool = int(rng.integers(k, 4 * k + 1))
        ids = np.stack([rng.choice(pool, size=k, replace=False) for _ in range(R)])
        _check(ids)
    _check(np.arange(128).reshape(16, 8))
    _check(np.tile(np.arange(8), (16, 1)))


# ---------------------------------------------------------------- one rank's share (expert parallel)
from oracle.union import expert_union_local  # noqa: E402


def _check_local(ids, lo, hi):
    ids = np.asarray(ids)
    R, k = ids.shape
    flat = ids.reshape(-1).tolist()
    u, U, s2u, mask = expert_union_local(ids, lo, hi)
    ref = list(dict.fromkeys(e for e in flat if lo <= e < hi))   # insertion-ordered dedup of the local ids
    assert u.tolist() == ref and U == len(ref)
    for t, e in enumerate(flat):
        if lo <= e < hi:
            assert u[s2u[t]] == e
        else:
            assert s2u[t] == -1
    for i, e in enumerate(ref):
        assert int(mask[i]) == sum(1 << (t // k) for t, v in enumerate(flat) if v == e)


def test_local_union_exhaustive_tiny():
    n = 0
    for E in range(1, 6):
        for k in range(1, min(E, 3) + 1):
            row_choices = list(itertools.permutations(range(E), k))
            for R in range(1, 3):
                for rows in itertools.product(row_choices, repeat=R):
                    for lo in range(E + 1):
                        for hi in range(lo, E + 1):
                            _check_local(np.array(rows), lo, hi)
                            n += 1
    assert n > 5000


def test_local_unions_partition_the_union():
    rng = np.random.default_rng(5)
    for _ in range(200):
        E = int(rng.integers(8, 300))
        k = int(rng.integers(1, 9))
        R = min(8, int(rng.integers(1, 64 // k + 1)))
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(R)])
        gu, GU, gs2u, gmask = expert_union(ids)
        # the whole range is the union itself
        lu, lU, ls2u, lmask = expert_union_local(ids, 0, E)
        assert lU == GU and np.array_equal(lu, gu) and np.array_equal(ls2u, gs2u) and np.array_equal(lmask, gmask)
        # G contiguous ranges: disjoint local unions that cover the union, each slot local to one rank
        G = int(rng.integers(2, 9))
        cuts = [0] + sorted(rng.choice(np.arange(1, E), size=min(G - 1, E - 1), replace=False).tolist()) + [E]
        parts = [expert_union_local(ids, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
        assert sum(p[1] for p in parts) == GU
        assert set().union(*[set(p[0].tolist()) for p in parts]) == set(gu.tolist())
        owners = np.sum([p[2] >= 0 for p in parts], axis=0)
        assert np.all(owners == 1)
