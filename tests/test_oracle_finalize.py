"""Pins of the MoE finalize oracle (no GPU): literal loops, the top_k=1
identity case, linearity in the weights, fp32 and bf16 row paths."""
import numpy as np
import torch

import synth
from oracle import formats as F
from oracle.finalize import moe_finalize
from tests.parity import bits16


def tiny(seed=3, T=7, k=3, rows=25, H=12):
    g = synth.gen(seed)
    fc2 = synth.bf16_normal((rows, H), 1.0, g)
    perm = torch.randperm(rows, generator=g)[:T * k].to(torch.int32)
    perm[[1, 5, 9]] = -1          # not routed here
    perm[11] = rows + 4           # past padded_rows: not routed here either
    w = synth.inputs.softmax_weights(T, k, g)
    delta = np.random.default_rng(seed).standard_normal((T, H))
    return fc2, perm, w, delta


def literal(fc2, perm, w, delta):
    """The combine with Python floats and explicit loops."""
    x = F.bf16_to_f64(bits16(fc2))
    T, k = w.shape
    rows, H = x.shape
    out = [[float(delta[t][h]) for h in range(H)] for t in range(T)]
    for t in range(T):
        for j in range(k):
            p = int(perm[t * k + j])
            if 0 <= p < rows:
                for h in range(H):
                    out[t][h] += float(w[t, j]) * float(x[p, h])
    return np.array(out)


def test_literal_loops():
    fc2, perm, w, delta = tiny()
    ours = moe_finalize(bits16(fc2), "bf16", perm.numpy(), w.numpy(), delta)
    assert np.allclose(ours, literal(fc2, perm, w, delta), rtol=1e-13, atol=1e-13)


def test_top1_identity_is_the_rows_plus_delta():
    g = synth.gen(4)
    fc2 = synth.bf16_normal((9, 16), 1.0, g)
    delta = np.arange(9 * 16, dtype=np.float64).reshape(9, 16) / 7.0
    ours = moe_finalize(bits16(fc2), "bf16", np.arange(9), np.ones((9, 1), np.float32), delta)
    assert np.array_equal(ours, F.bf16_to_f64(bits16(fc2)) + delta)


def test_linear_in_the_weights_and_skips_unrouted_slots():
    fc2, perm, w, delta = tiny(5)
    z = np.zeros_like(delta)
    one = moe_finalize(bits16(fc2), "bf16", perm.numpy(), w.numpy(), z)
    two = moe_finalize(bits16(fc2), "bf16", perm.numpy(), 2 * w.numpy(), z)
    assert np.array_equal(2 * one, two)
    none = moe_finalize(bits16(fc2), "bf16", np.full(perm.numel(), -1), w.numpy(), delta)
    assert np.array_equal(none, delta)


def test_fp32_rows_equal_bf16_rows_of_the_same_values():
    fc2, perm, w, delta = tiny(6)
    a = moe_finalize(bits16(fc2), "bf16", perm.numpy(), w.numpy(), delta)
    b = moe_finalize(fc2.float().numpy(), "f32", perm.numpy(), w.numpy(), delta)
    assert np.array_equal(a, b)
    h = moe_finalize(bits16(fc2.half()), "f16", perm.numpy(), w.numpy(), delta)
    assert np.allclose(h, a, rtol=1e-3, atol=1e-3)


def test_token_subset_equals_rows_of_the_whole():
    """``tokens=`` (used by the sampled GPU tests) returns the rows of the
    all-token combine and of the literal loops, in the order asked."""
    fc2, perm, w, delta = tiny(7)
    full = moe_finalize(bits16(fc2), "bf16", perm.numpy(), w.numpy(), delta)
    lit = literal(fc2, perm, w, delta)
    S = [6, 2, 2, 0]
    sub = moe_finalize(bits16(fc2), "bf16", perm.numpy(), w.numpy(), delta[S], tokens=S)
    assert np.array_equal(sub, full[S])
    assert np.allclose(sub, lit[S], rtol=1e-13, atol=1e-13)
