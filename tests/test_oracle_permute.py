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


def test_hand_worked_example():
    """Three tokens, top_k=2, E=3; slot 3's id 5 is not an expert held here.
    Slots by expert, in slot order: e0 <- {1, 4}; e1 <- {0, 5}; e2 <- {2}."""
    ids = np.array([[1, 0], [2, 5], [0, 1]])
    m, perm, inv = route_permutation(ids, 3)
    assert m.tolist() == [0, 2, 4, 5]
    assert perm.tolist() == [2, 0, 4, -1, 1, 3]
    assert inv.tolist() == [1, 4, 0, 5, 2, -1]
    out = permute_rows(np.array([[10.0], [20.0], [30.0]]), perm, 2, np.zeros((6, 1)))
    assert out[:, 0].tolist() == [10.0, 30.0, 10.0, 30.0, 20.0, 0.0]


def test_one_expert_is_the_identity():
    ids = np.zeros((17, 1), dtype=np.int64)
    m, perm, inv = route_permutation(ids, 1)
    assert m.tolist() == [0, 17]
    assert perm.tolist() == list(range(17)) and inv.tolist() == list(range(17))
