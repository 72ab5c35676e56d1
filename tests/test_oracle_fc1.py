"""Pins of the FC1 SwiGLU oracle (no GPU): a literal per-element loop, closed
forms of SiLU, the library logistic function, the clamp and the additive
FC1 delta."""
import math

import numpy as np
from scipy.special import expit

from oracle.fc1 import grouped_mm_swiglu, swiglu
from oracle.formats import bf16_to_f64, f64_to_bf16_bits


def ints_bf16(rng, shape, lo=-3, hi=3):
    return f64_to_bf16_bits(rng.integers(lo, hi + 1, shape).astype(np.float64))


def test_literal_loop():
    rng = np.random.default_rng(0)
    counts, inter, k = (2, 0, 3), 3, 8
    mi = np.concatenate([[0], np.cumsum(counts)])
    a = ints_bf16(rng, (5, k))
    b = ints_bf16(rng, (3, 2 * inter, k))
    alpha = np.array([1.0, 0.5, 1.702], dtype=np.float32)
    beta = np.array([0.0, 1.0, 1.0], dtype=np.float32)
    limit = np.array([7.0, 2.0, 3.5], dtype=np.float32)
    out, written = grouped_mm_swiglu(a, b, mi, alpha=alpha, beta=beta, limit=limit)
    A, B = bf16_to_f64(a), bf16_to_f64(b)
    for e in range(3):
        for r in range(mi[e], mi[e + 1]):
            for c in range(inter):
                hg = sum(A[r, kk] * B[e, c, kk] for kk in range(k))
                hu = sum(A[r, kk] * B[e, inter + c, kk] for kk in range(k))
                g = min(hg, float(limit[e]))
                u = max(-float(limit[e]), min(hu, float(limit[e])))
                want = g / (1.0 + math.exp(-float(alpha[e]) * g)) * (u + float(beta[e]))
                assert abs(out[r, c] - want) <= 1e-14 * max(1.0, abs(want)), (e, r, c)
    assert written.all()


def test_silu_closed_forms_and_library_logistic():
    x = np.linspace(-30, 30, 601)
    one = np.ones_like(x)
    s = swiglu(x, one)
    assert s[300] == 0.0                                      # silu(0) = 0
    assert np.allclose(s - swiglu(-x, one), x, rtol=0, atol=1e-12)  # silu(x) - silu(-x) = x
    assert np.allclose(s, x * expit(x), rtol=1e-15, atol=0)   # the library logistic
    assert abs(swiglu(np.array([-800.0]), np.array([1.0]))[0]) == 0.0   # no overflow
    assert swiglu(np.array([800.0]), np.array([2.0]))[0] == 1600.0


def test_defaults_are_plain_swiglu_and_numpy_product():
    rng = np.random.default_rng(1)
    a = f64_to_bf16_bits(rng.standard_normal((40, 64)))
    b = f64_to_bf16_bits(rng.standard_normal((1, 32, 64)) / 8)
    out, _ = grouped_mm_swiglu(a, b, np.array([0, 40]))
    h = bf16_to_f64(a) @ bf16_to_f64(b)[0].T
    assert np.allclose(out, h[:, :16] * expit(h[:, :16]) * h[:, 16:], rtol=1e-13, atol=1e-15)


def test_clamp_and_delta():
    g = np.array([-10.0, 0.5, 10.0])
    u = np.array([-10.0, 0.5, 10.0])
    got = swiglu(g, u, alpha=2.0, beta=1.0, limit=3.0)
    want = np.array([-10.0 * expit(-20.0) * (-3.0 + 1.0), 0.5 * expit(1.0) * 1.5,
                     3.0 * expit(6.0) * (3.0 + 1.0)])
    assert np.allclose(got, want, rtol=1e-15, atol=0)
    # a delta that cancels h exactly leaves g = u = 0, so out = 0 * sigmoid(0) * beta = 0
    rng = np.random.default_rng(2)
    a = ints_bf16(rng, (6, 16))
    b = ints_bf16(rng, (2, 8, 16))
    mi = np.array([0, 4, 6])
    h = np.concatenate([bf16_to_f64(a[:4]) @ bf16_to_f64(b[0]).T,
                        bf16_to_f64(a[4:]) @ bf16_to_f64(b[1]).T])
    delta = f64_to_bf16_bits(-h)  # small integers: exact in bf16
    out, _ = grouped_mm_swiglu(a, b, mi, delta_bits=delta,
                               beta=np.array([1.5, -2.0], dtype=np.float32))
    assert (out == 0).all()
