"""Pins of the permutation oracle (no GPU): a literal counting loop, the
properties of a stable expert sort, and the permuted rows."""
import numpy as np
import pytest

from oracle.permute import permute_rows, route_permutation


def literal(ids, E):
    """Walk the expanded slots in order with one running counter per expert."""
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    counts = [0] * E
    for v in flat:
        if 0 <= v < E:
            counts[v] += 1
    start = [0] * (E + 1)
    for e in range(E):
        start[e + 1] = start[e] + counts[e]
    nxt = start[:E]
    perm = []
    for v in flat:
        if 0 <= v < E:
            perm.append(nxt[v])
            nxt[v] += 1
        else:
            perm.append(-1)
    return start, perm


@pytest.mark.parametrize("T,k,E,seed", [(7, 3, 5, 0), (64, 8, 16, 1), (33, 1, 4, 2),
                                        (50, 6, 300, 3)])
def test_literal_counting(T, k, E, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(-2, E + 2, size=(T, k))  # includes ids not routed here
    m, perm, inv = route_permutation(ids, E)
    start, lp = literal(ids, E)
    assert m.tolist() == start and perm.tolist() == lp


def test_stable_sort_properties():
    rng = np.random.default_rng(5)
    T, k, E = 200, 4, 12
    ids = rng.integers(0, E, size=(T, k))
    m, perm, inv = route_permutation(ids, E)
    flat = ids.reshape(-1)
    assert sorted(perm.tolist()) == list(range(T * k))        # a bijection
    assert np.array_equal(perm[inv], np.arange(T * k))        # inverse map
    for e in range(E):
        xs = inv[m[e]:m[e + 1]]
        assert (flat[xs] == e).all() and (np.diff(xs) > 0).all()  # grouped and stable
    assert (np.diff(m) >= 0).all() and m[-1] == T * k


def test_permute_rows():
    rng = np.random.default_rng(6)
    T, k, E, H = 9, 2, 3, 5
    ids = rng.integers(0, E, size=(T, k))
    ids[4, 1] = E  # not routed here
    x = rng.standard_normal((T, H))
    m, perm, inv = route_permutation(ids, E)
    out = permute_rows(x, perm, k, np.full((T * k, H), 7.0))
    for p in range(m[-1]):
        assert np.array_equal(out[p], x[inv[p] // k])
    assert (out[m[-1]:] == 7.0).all()  # rows no slot maps to keep their values
