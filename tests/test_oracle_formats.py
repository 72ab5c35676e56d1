"""Pins of the oracle's number formats against library routines and the
formats' bit-field definitions (no GPU)."""
import numpy as np
import pytest
import torch

from oracle import formats as F


def test_bf16_decode_matches_torch_on_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = F.bf16_to_f64(bits)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    same = (ours == lib) | (np.isnan(ours) & np.isnan(lib))
    assert same.all()
    # signed zero preserved
    assert np.signbit(F.bf16_to_f64(np.array([0x8000], np.uint16)))[0]


def _torch_f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(x32.astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_rounding_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(0)
    # random bit patterns cover every binade including subnormals and large values
    pats = rng.integers(0, 1 << 32, 200_000, dtype=np.uint64).astype(np.uint32)
    x32 = pats.view(np.float32)
    x32 = x32[np.isfinite(x32)]
    ours = F.f64_to_bf16_bits(x32.astype(np.float64))
    lib = _torch_f32_to_bf16_bits(x32)
    assert np.array_equal(ours, lib)


@pytest.mark.parametrize("x,bits", [
    (1.0 + 2.0 ** -8, 0x3F80),                 # tie -> even (down)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),             # tie -> even (up)
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),    # just above the tie
    (-(1.0 + 2.0 ** -8), 0xBF80),
    (2.0 ** -133, 0x0001),                     # smallest subnormal
    (2.0 ** -134, 0x0000),                     # half of it: tie to even zero
    (1.5 * 2.0 ** -134, 0x0001),
    ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),    # largest finite
    (2.0 ** 128 - 2.0 ** 119, 0x7F80),         # halfway to 2**128: ties to even = Inf
    (2.0 ** 128 - 2.0 ** 119 - 2.0 ** 100, 0x7F7F),
    (float("inf"), 0x7F80),
    (float("-inf"), 0xFF80),
    (-0.0, 0x8000),
    (float("nan"), 0x7FC0),
])
def test_bf16_rounding_hand_cases(x, bits):
    assert int(F.f64_to_bf16_bits(np.array([x]))[0]) == bits


def test_e2m1_from_bitfields():
    # sign | 2-bit exponent (bias 1) | 1-bit mantissa; exponent 0 is subnormal
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        want = -mag if s else mag
        got = float(F.e2m1_to_f64(np.array([c]))[0])
        assert got == want and np.signbit(got) == bool(s)


def test_ue4m3_matches_torch_float8_e4m3fn():
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(F.ue4m3_to_f64(codes), lib)
    assert np.isnan(F.ue4m3_to_f64(np.array([0x7F])))[0]
    assert np.isnan(F.ue4m3_to_f64(np.array([0x80])))[0]
    # the generator's scale range 0x28..0x48 is exactly [0.25, 4]
    assert F.ue4m3_to_f64(np.array([0x28]))[0] == 0.25
    assert F.ue4m3_to_f64(np.array([0x48]))[0] == 4.0
    assert F.ue4m3_to_f64(np.array([0x38]))[0] == 1.0


def test_e2m1_times_ue4m3_is_exact_in_bf16():
    """Every product of an E2M1 value and a finite UE4M3 scale is a bf16
    number (at most 6 significant bits, range 2**-10 .. 2688)."""
    v = F.e2m1_to_f64(np.arange(16))
    s = F.ue4m3_to_f64(np.arange(0x7F))
    prod = (v[:, None] * s[None, :]).ravel()
    back = F.bf16_to_f64(F.f64_to_bf16_bits(prod))
    assert np.array_equal(back, prod)


def test_f16_decode_matches_numpy_on_all_patterns():
    from oracle.formats import f16_to_f64
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    want = bits.view(np.float16).astype(np.float64)
    got = f16_to_f64(bits)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_f16_rounding_matches_numpy_and_hand_cases():
    from oracle.formats import f64_to_f16_bits
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(0, 1, 20000), rng.normal(0, 1e4, 5000),
                        rng.normal(0, 1e-6, 5000), [0.0, -0.0, 65504.0, 65520.0, 1e6, -1e6]])
    want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(f64_to_f16_bits(x), want)
    # ties to even: 1 + 2**-11 lies halfway between 1 and 1 + 2**-10 -> 1 (even)
    assert f64_to_f16_bits(np.array([1 + 2.0 ** -11]))[0] == 0x3C00
    # 1 + 3*2**-11 lies halfway between 1 + 2**-10 and 1 + 2**-9 -> the even one
    assert f64_to_f16_bits(np.array([1 + 3 * 2.0 ** -11]))[0] == 0x3C02
    # smallest subnormal and the halfway point below it
    assert f64_to_f16_bits(np.array([2.0 ** -24]))[0] == 0x0001
    assert f64_to_f16_bits(np.array([2.0 ** -25]))[0] == 0x0000
    assert f64_to_f16_bits(np.array([np.nan]))[0] == 0x7E00
