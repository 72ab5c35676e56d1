"""Pins of the fold oracle against IEEE float32 arithmetic done by numpy and
torch (no GPU)."""
import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle.fold import fold, fold_ratio, prepare_host_check


def lib_fold(lb_bits, s, alpha):
    """numpy float32 division and product, torch's float32 -> bf16 cast."""
    with np.errstate(all="ignore"):
        ratio = np.float32(s) / np.float32(alpha)
        prod = F.bf16_to_f64(lb_bits).astype(np.float32) * ratio
    t = torch.from_numpy(np.asarray(prod, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def rand_bf16(rng, n, std):
    return F.f64_to_bf16_bits(rng.standard_normal(n) * std)


@pytest.mark.parametrize("s,alpha", [(0.5, 0.01), (2.0, 3.0), (1e-3, 7.77), (123.4, 0.056),
                                     (-0.75, 0.3), (1.0, 1.0)])
def test_fold_matches_float32_library(s, alpha):
    rng = np.random.default_rng(5)
    lb = rand_bf16(rng, 50_000, 0.02)
    bits, zero = fold(lb, s, alpha)
    assert np.array_equal(bits, lib_fold(lb, s, alpha))
    assert not zero


def test_ratio_is_correctly_rounded_division():
    rng = np.random.default_rng(6)
    s = rng.standard_normal(20000).astype(np.float32) * np.float32(10) ** rng.integers(
        -30, 30, 20000).astype(np.float32)
    a = rng.standard_normal(20000).astype(np.float32) * np.float32(10) ** rng.integers(
        -30, 30, 20000).astype(np.float32)
    ours = np.array([fold_ratio(x, y) for x, y in zip(s, a)], dtype=np.float32)
    with np.errstate(all="ignore"):
        lib = s / a
    same = (ours.view(np.uint32) == lib.view(np.uint32)) | (np.isnan(ours) & np.isnan(lib))
    assert same.all()


def test_fold_edge_cases():
    all_bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = all_bits[np.isfinite(F.bf16_to_f64(all_bits))]
    for s, alpha in [(1e-38, 1.0),      # products deep in the subnormal range
                     (3.0e38, 0.5),     # ratio overflows -> Inf products
                     (1.0, 3.0),        # inexact ratio, many RNE decisions
                     (1.0 + 2 ** -23, 1.0)]:
        bits, _ = fold(finite, s, alpha)
        lib = lib_fold(finite, s, alpha)
        same = (bits == lib) | (np.isnan(F.bf16_to_f64(bits)) & np.isnan(F.bf16_to_f64(lib)))
        assert same.all(), (s, alpha)


def test_fold_tie_rounding():
    # lora_b = 1 + 2**-7 (bf16), ratio = 1 + 2**-8 exactly: product 1 + 3*2**-8 + 2**-15
    # -> rounds up; ratio 1 + 2**-9 gives 1 + 2**-7 + 2**-9 + 2**-16 -> stays
    lb = F.f64_to_bf16_bits(np.array([1 + 2 ** -7]))
    bits, _ = fold(lb, 1 + 2 ** -8, 1.0)
    assert int(bits[0]) == int(F.f64_to_bf16_bits(np.array([1 + 2 ** -6]))[0])
    # exact tie: lora_b = 1, ratio = 1 + 2**-8 -> 0x3F80 (even)
    bits, _ = fold(F.f64_to_bf16_bits(np.array([1.0])), 1 + 2 ** -8, 1.0)
    assert int(bits[0]) == 0x3F80


def test_zero_scale_flags_zero_adapter():
    lb = F.f64_to_bf16_bits(np.array([0.5, -0.25, 0.0]))
    for s in (0.0, -0.0):
        bits, zero = fold(lb, s, 0.01)
        assert zero
        assert not F.bf16_to_f64(bits).any()


def test_alpha_0_01_ratio_is_50():
    assert fold_ratio(0.5, 0.01) == np.float32(50.0)


def test_prepare_host_check():
    with pytest.raises(ValueError):
        prepare_host_check(0.5, 0.0)
    with pytest.raises(ValueError):
        prepare_host_check(1e30, 1e-30)
    prepare_host_check(0.0, 0.01)
