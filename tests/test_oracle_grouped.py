"""Pins of the grouped-GEMM oracle (no GPU): brute force, library special
cases and an exact integer probe."""
import numpy as np
import torch

import synth
from oracle import formats as F
from oracle.grouped_mm import grouped_mm, grouped_mm_rows
from tests.parity import bits16


def _rand_bits(rng, shape, std=1.0):
    x = (rng.standard_normal(shape) * std).astype(np.float32)
    return F.f64_to_bf16_bits(x.astype(np.float64))


def test_brute_force_tiny_ragged():
    rng = np.random.default_rng(1)
    counts = [2, 0, 3, 1]
    k, n = 5, 7                    # n != k so a transposed operand cannot pass
    cum = sum(counts)
    a = _rand_bits(rng, (cum + 2, k))            # two trailing rows not in any group
    b = _rand_bits(rng, (len(counts), n, k))
    m_indptr = np.concatenate([[0], np.cumsum(counts)])
    out, written = grouped_mm(a, b, m_indptr)
    A, B = F.bf16_to_f64(a), F.bf16_to_f64(b)
    for row in range(cum):
        e = next(i for i in range(len(counts)) if m_indptr[i] <= row < m_indptr[i + 1])
        for col in range(n):
            s = 0.0
            for kk in range(k):
                s += A[row, kk] * B[e, col, kk]
            assert abs(out[row, col] - s) <= 1e-12 * (1 + abs(s))
    assert written[:cum].all() and not written[cum:].any()
    assert not out[cum:].any()


def test_single_expert_is_matmul():
    rng = np.random.default_rng(2)
    a = _rand_bits(rng, (9, 16))
    b = _rand_bits(rng, (1, 12, 16))
    out, _ = grouped_mm(a, b, np.array([0, 9]))
    assert np.allclose(out, np.matmul(F.bf16_to_f64(a), F.bf16_to_f64(b)[0].T), rtol=1e-13,
                       atol=1e-13)


def test_uniform_groups_is_batched_matmul():
    rng = np.random.default_rng(3)
    E, tpe, k, n = 4, 3, 8, 6
    a = _rand_bits(rng, (E * tpe, k))
    b = _rand_bits(rng, (E, n, k))
    out, _ = grouped_mm(a, b, np.arange(E + 1) * tpe)
    ref = np.einsum("etk,enk->etn", F.bf16_to_f64(a).reshape(E, tpe, k), F.bf16_to_f64(b))
    assert np.allclose(out, ref.reshape(E * tpe, n), rtol=1e-13, atol=1e-13)


def test_integer_probe_is_exact():
    case = synth.grouped_int_probe(counts=(0, 1, 3, 0, 2), n=6, k=5)
    a = bits16(case.a)
    b = bits16(case.b)
    mi = case.m_indptr.numpy()
    out, written = grouped_mm(a, b, mi)
    A = case.a.to(torch.int64).numpy()
    B = case.b.to(torch.int64).numpy()
    for e in range(len(mi) - 1):
        for row in range(mi[e], mi[e + 1]):
            for col in range(6):
                assert out[row, col] == int(sum(int(A[row, kk]) * int(B[e, col, kk])
                                                for kk in range(5)))
    assert written.all()


def test_selected_rows_match_full():
    rng = np.random.default_rng(4)
    counts = [3, 0, 4, 2]
    a = _rand_bits(rng, (9, 8))
    b = _rand_bits(rng, (4, 6, 8))
    mi = np.concatenate([[0], np.cumsum(counts)])
    full, _ = grouped_mm(a, b, mi)
    rows = [0, 3, 6, 8]
    cols = [1, 4]
    sel = grouped_mm_rows(a[rows], lambda e, c: b[e][c], mi, rows, cols)
    assert np.array_equal(sel, full[np.ix_(rows, cols)])


def test_fp16_inputs_decode_as_fp16():
    # small integers are exact in both types: the fp16 reading of the fp16 bits
    # and the bf16 reading of the bf16 bits of the same values agree
    from oracle.formats import f64_to_bf16_bits, f64_to_f16_bits
    rng = np.random.default_rng(3)
    a = rng.integers(-4, 5, (20, 32)).astype(np.float64)
    b = rng.integers(-4, 5, (3, 16, 32)).astype(np.float64)
    mi = np.array([0, 7, 7, 20])
    o16, w16 = grouped_mm(f64_to_f16_bits(a), f64_to_f16_bits(b), mi, "f16")
    ob, wb = grouped_mm(f64_to_bf16_bits(a), f64_to_bf16_bits(b), mi)
    assert np.array_equal(o16, ob) and np.array_equal(w16, wb)
    # a value bf16 cannot hold: 1 + 2**-10 is exact in fp16 only
    one = f64_to_f16_bits(np.array([[1 + 2.0 ** -10]]))
    o, _ = grouped_mm(one, one.reshape(1, 1, 1), np.array([0, 1]), "f16")
    assert o[0, 0] == (1 + 2.0 ** -10) ** 2
