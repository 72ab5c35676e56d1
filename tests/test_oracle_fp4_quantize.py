"""Pins of the NVFP4 quantisation oracle (no GPU): its two roundings against
torch's own float8_e4m3fn conversion and a hand table, fixed points of
quantise(dequantise(.)), the error bound, scale and sign symmetries, the
special blocks and the 128x4 placement."""
import numpy as np
import pytest
import torch

from oracle import fp4_quantize as Q
from oracle.formats import E2M1_MAGNITUDES, ue4m3_to_f64
from oracle.nvfp4 import dequant, sf_offset


def test_ue4m3_rounding_matches_torch_float8_e4m3fn():
    """Every finite UE4M3 value, every midpoint between neighbours (a tie) and
    random fp32 values in [0, 448]: nearest with ties to even, as torch's
    RNE conversion to float8_e4m3fn does."""
    vals = ue4m3_to_f64(np.arange(0x7F))
    mids = (vals[:-1] + vals[1:]) / 2          # exact in fp32
    rng = np.random.default_rng(0)
    rnd = np.concatenate([rng.uniform(0, 448, 20000), np.exp(rng.uniform(-12, 6, 20000))])
    xs = np.concatenate([vals, mids, rnd[rnd <= 448]]).astype(np.float32)
    ours = np.array([Q.ue4m3_round(np.float32(v)) for v in xs], dtype=np.uint8)
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    # ties really are ties: each midpoint lands on the even code of its pair
    tie = np.array([Q.ue4m3_round(np.float32(m)) for m in mids])
    assert np.all(tie % 2 == 0)


def test_ue4m3_saturates():
    for v in [448.0, 449.0, 463.99, 464.0, 480.0, 1e30, np.inf]:
        assert Q.ue4m3_round(np.float32(v)) == 0x7E
    assert Q.ue4m3_round(np.float32(0.0)) == 0
    assert Q.ue4m3_round(np.float32(2.0 ** -10)) == 0      # tie between 0 and 2^-9: even (0)
    assert Q.ue4m3_round(np.float32(3 * 2.0 ** -10)) == 2  # tie between 1 and 2 (x 2^-9): even


def test_e2m1_rounding_hand_table():
    table = [  # (value, code): exact values, midpoints (ties to the even code), between, above
        (0.0, 0), (0.5, 1), (1.0, 2), (1.5, 3), (2.0, 4), (3.0, 5), (4.0, 6), (6.0, 7),
        (0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),
        (0.2499, 0), (0.2501, 1), (0.7499, 1), (1.2501, 3), (1.7499, 3), (2.5001, 5),
        (3.4999, 5), (4.9999, 6), (5.0001, 7), (6.5, 7), (1e9, 7)]
    for v, code in table:
        assert Q.e2m1_round(np.float32(v)) == code, v
        assert Q.e2m1_round(np.float32(-v)) == code | 8, -v
    assert Q.e2m1_round(np.float32(-0.0)) == 8


def _fixed_point_case(rng, rows, K, g):
    """Codes and scale codes whose dequantised values, divided by a power-of-
    two g, quantise back to themselves: every block holds a +-6 (the block
    maximum maps onto 6 exactly) and a scale that keeps amax * g / 6 exact."""
    codes = rng.integers(0, 16, (rows, K)).astype(np.uint8)
    for r in range(rows):
        for b in range(K // 16):
            codes[r, 16 * b + rng.integers(16)] = rng.choice([7, 15])
    scodes = rng.integers(1, 0x7F, (rows, K // 16)).astype(np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    sf = Q.place_scales(scodes, rows, K)
    x = (dequant(packed, sf, K) / g).astype(np.float32)
    assert np.array_equal(x.astype(np.float64) * g, dequant(packed, sf, K))  # exact
    return packed, scodes, sf, x


@pytest.mark.parametrize("g", [1.0, 2.0 ** 10, 2.0 ** -7])
def test_quantize_of_dequantized_is_a_fixed_point(g):
    rng = np.random.default_rng(int(np.log2(g)) + 50)
    packed, scodes, sf, x = _fixed_point_case(rng, 5, 64, g)
    c2, s2 = Q.quantize_rows(x, np.float32(g))
    assert np.array_equal(s2, scodes)
    # +0 and -0 codes both dequantise to 0 and come back as the sign of x
    same = np.where((packed & 7) == 0, packed & 0x88, packed)
    got = np.where((c2 & 7) == 0, c2 & 0x88, c2)
    assert np.array_equal(got & 0x77, same & 0x77)
    nz_lo, nz_hi = (packed & 7) != 0, (packed & 0x70) != 0
    assert np.array_equal((c2 & 0x8)[nz_lo], (packed & 0x8)[nz_lo])
    assert np.array_equal((c2 & 0x80)[nz_hi], (packed & 0x80)[nz_hi])


def test_error_bound_on_normal_data():
    """|dequant/g - x| <= S/g per element (S the block's decoded scale): the
    E2M1 grid spacing is at most 2 below 6, and the scale's rounding pushes the
    block maximum at most 6 * 2^-4 past 6."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((7, 256)) * np.exp(rng.uniform(-3, 3, (7, 1)))).astype(np.float32)
    g = np.float32(448.0 * 6.0 / np.abs(x).max())
    codes, sf = Q.fp4_quantize(x, g)
    back = dequant(codes, sf, 256) / float(g)
    rows = np.arange(7)
    S = ue4m3_to_f64(sf[sf_offset(rows[:, None], np.arange(16)[None, :], 256)])
    bound = np.repeat(S, 16, axis=1) / float(g)
    assert np.all(np.abs(back - x) <= bound)
    # and the quantisation is not trivially coarse: relative rms error < 10%
    assert np.sqrt(np.mean((back - x) ** 2)) < 0.1 * np.sqrt(np.mean(x.astype(np.float64) ** 2))


def test_power_of_two_rescaling_and_sign_symmetry():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 64)).astype(np.float32)
    x[0, 5] = 0.0
    g = np.float32(37.0)
    c0, s0 = Q.quantize_rows(x, g)
    c1, s1 = Q.quantize_rows(x * np.float32(8.0), g / np.float32(8.0))
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1)
    cn, sn = Q.quantize_rows(-x, g)
    assert np.array_equal(sn, s0)
    assert np.array_equal(cn, c0 ^ 0x88)


def test_special_blocks():
    g = np.float32(1.0)
    c, s = Q.quantize_block(np.zeros(16, np.float32), g)
    assert s == 0 and c == [0] * 16
    neg0 = np.full(16, -0.0, np.float32)
    c, s = Q.quantize_block(neg0, g)
    assert s == 0 and c == [8] * 16
    # tiny block: the scale underflows to 0, every code is a signed zero
    c, s = Q.quantize_block(np.array([1e-30, -1e-30] * 8, np.float32), g)
    assert s == 0 and c == [0, 8] * 8
    # a huge global scale saturates the scale at 448; elements then saturate at 6
    c, s = Q.quantize_block(np.array([1.0] + [0.0] * 15, np.float32), np.float32(1e6))
    assert s == 0x7E and c[0] == 7
    # one block does not see its neighbours
    x = np.random.default_rng(5).standard_normal((1, 32)).astype(np.float32)
    a, sa = Q.quantize_rows(x, g)
    x2 = x.copy()
    x2[0, 16:] *= 100
    b, sb = Q.quantize_rows(x2, g)
    assert np.array_equal(a[0, :8], b[0, :8]) and sa[0, 0] == sb[0, 0]


def test_placement_and_padding():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((130, 64)).astype(np.float32)
    codes, sf = Q.fp4_quantize(x, np.float32(10.0))
    _, scodes = Q.quantize_rows(x, np.float32(10.0))
    assert sf.size == 2 * 1 * 512
    for r, c in [(0, 0), (33, 2), (129, 3), (127, 1)]:
        assert sf[sf_offset(r, c, 64)] == scodes[r, c]
    used = np.zeros(sf.size, bool)
    used[sf_offset(np.arange(130)[:, None], np.arange(4)[None, :], 64)] = True
    assert used.sum() == 130 * 4 and not sf[~used].any()  # padding rows are zero
    # and the nibble order: element 2i low, 2i+1 high
    c16, _ = Q.quantize_rows(x[:1, :16], np.float32(10.0))
    single = [Q.quantize_block(x[0, :16], np.float32(10.0))[0]]
    assert c16[0, 0] == single[0][0] | (single[0][1] << 4)
    assert E2M1_MAGNITUDES[7] == 6.0
