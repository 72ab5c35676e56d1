"""Pins of the NVFP4 + LoRA oracle (no GPU)."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import nvfp4 as N
from oracle.fold import fold
from tests.parity import bits16


def _sf_offset_by_reshape(rows: int, k: int) -> np.ndarray:
    """Second, independent coding of the 128x4 tiling: lay the logical
    [rows_pad, cols_pad] index grid out as
    [row_block, col_block, 32, 4 (row quarter), 4 (col)] and read where each
    logical (row, col) lands."""
    cols = -(-k // 16)
    rp, cp = -(-rows // 128) * 128, -(-cols // 4) * 4
    logical = np.arange(rp * cp).reshape(rp, cp)            # value = row*cp + col
    t = logical.reshape(rp // 128, 4, 32, cp // 4, 4)       # [rb, quarter, r32, cb, c4]
    phys = t.transpose(0, 3, 2, 1, 4).reshape(-1)           # physical order
    where = np.empty(rp * cp, dtype=np.int64)
    where[phys] = np.arange(rp * cp)
    return where.reshape(rp, cp)


@pytest.mark.parametrize("rows,k", [(128, 256), (300, 512), (4096, 8192), (1, 64), (129, 320)])
def test_sf_offset_two_codings_agree(rows, k):
    where = _sf_offset_by_reshape(rows, k)
    r = np.arange(where.shape[0])[:, None]
    c = np.arange(where.shape[1])[None, :]
    assert np.array_equal(N.sf_offset(r, c, k), where)


def test_sf_offset_hand_worked():
    # k=256 -> 16 scale columns -> 4 column tiles per row block
    assert N.sf_offset(33, 5, 256) == (0 * 4 + 1) * 512 + 1 * 16 + 1 * 4 + 1
    assert N.sf_offset(200, 7, 256) == (1 * 4 + 1) * 512 + 8 * 16 + 2 * 4 + 3
    assert N.sf_offset(0, 0, 8192) == 0
    assert N.sf_offset(127, 3, 8192) == 31 * 16 + 3 * 4 + 3
    # buffer size agrees with the generator's
    assert N.sf_offset(4095, 511, 8192) + 1 == synth.sf_buffer_bytes(4096, 8192)


def test_dequant_elementwise_literal():
    rng = np.random.default_rng(3)
    rows, k = 130, 64
    packed = rng.integers(0, 256, (rows, k // 2), dtype=np.uint8)
    sf = rng.integers(0x01, 0x7F, synth.sf_buffer_bytes(rows, k), dtype=np.uint8)
    deq = N.dequant(packed, sf, k)
    for r in [0, 1, 31, 32, 127, 128, 129]:
        for kk in range(k):
            byte = int(packed[r, kk // 2])
            code = byte & 0xF if kk % 2 == 0 else byte >> 4
            s = F.ue4m3_to_f64(sf[N.sf_offset(r, kk // 16, k)])
            assert deq[r, kk] == F.e2m1_to_f64(code) * s


def test_exact_probe_matches_fraction_brute_force():
    case = synth.nvfp4_probe("exact", M=6, N=5, K=64)
    base = N.base_product(case.a.numpy(), case.b.numpy(), case.a_sf.numpy(), case.b_sf.numpy(),
                          case.K)
    qa = N.unpack_codes(case.a.numpy())
    qb = N.unpack_codes(case.b.numpy())
    for m in range(6):
        for n in range(5):
            s = sum(Fraction(float(F.e2m1_to_f64(qa[m, kk]))) * Fraction(float(F.e2m1_to_f64(qb[n, kk])))
                    for kk in range(64))
            assert Fraction(float(base[m, n])) == s


def test_identity_probe_returns_dequantised_a():
    case = synth.nvfp4_probe("identity", M=16, N=64, K=64)
    base = N.base_product(case.a.numpy(), case.b.numpy(), case.a_sf.numpy(), case.b_sf.numpy(),
                          case.K)
    assert np.array_equal(base, N.dequant(case.a.numpy(), case.a_sf.numpy(), case.K))


def test_lora_only_probe_is_lora_plus_bias():
    case = synth.nvfp4_probe("lora_only", M=8, N=32, K=64)
    base = N.base_product(case.a.numpy(), case.b.numpy(), case.a_sf.numpy(), case.b_sf.numpy(),
                          case.K)
    assert not base.any()
    out = N.mm_nvfp4_raw(base, 0.01, bits16(case.d), bits16(case.lora_b), 0.5, bits16(case.bias))
    D = F.bf16_to_f64(bits16(case.d))
    LB = F.bf16_to_f64(bits16(case.lora_b))
    ref = np.float32(0.5) * np.einsum("mr,nr->mn", D, LB) + F.bf16_to_f64(bits16(case.bias))
    assert np.allclose(out, ref, rtol=1e-13, atol=1e-15)


def test_zero_adapter_forms_equal_off():
    case = synth.nvfp4_lora_case(seed=11, M=32, N=64, K=256)
    base = N.base_product(case.a.numpy(), case.b.numpy(), case.a_sf.numpy(), case.b_sf.numpy(),
                          case.K)
    bias = bits16(case.bias)
    off = N.mm_nvfp4_off(base, 0.01, bias)
    assert np.array_equal(N.mm_nvfp4_raw(base, 0.01, bits16(case.d), bits16(case.lora_b), 0.0,
                                         bias), off)
    fb, zero = fold(bits16(case.lora_b), 0.0, 0.01)
    assert zero
    assert np.array_equal(N.mm_nvfp4_prepared(base, 0.01, bits16(case.d), fb, zero, bias), off)


def test_prepared_equals_raw_when_the_fold_is_exact():
    """With lora_scale/alpha a power of two the fold is exact, so the two
    adapter forms compute the same number."""
    case = synth.nvfp4_lora_case(seed=12, M=16, N=32, K=256, alpha=0.5, lora_scale=0.25)
    base = N.base_product(case.a.numpy(), case.b.numpy(), case.a_sf.numpy(), case.b_sf.numpy(),
                          case.K)
    fb, zero = fold(bits16(case.lora_b), 0.25, 0.5)
    assert np.array_equal(F.bf16_to_f64(fb), F.bf16_to_f64(bits16(case.lora_b)) * 0.5)
    raw = N.mm_nvfp4_raw(base, 0.5, bits16(case.d), bits16(case.lora_b), 0.25, bits16(case.bias))
    prep = N.mm_nvfp4_prepared(base, 0.5, bits16(case.d), fb, zero, bits16(case.bias))
    assert np.allclose(raw, prep, rtol=1e-14, atol=1e-14)


def test_uniform_unit_scales_is_plain_matmul():
    case = synth.nvfp4_probe("exact", M=20, N=24, K=128)
    A = F.e2m1_to_f64(N.unpack_codes(case.a.numpy()))
    B = F.e2m1_to_f64(N.unpack_codes(case.b.numpy()))
    base = N.base_product(case.a.numpy(), case.b.numpy(), case.a_sf.numpy(), case.b_sf.numpy(),
                          case.K)
    assert np.array_equal(base, np.matmul(A, B.T))


def test_scales_enter_per_block_and_per_row():
    """Doubling one row's scale byte exponent for one K block doubles exactly
    that block's contribution for that row only."""
    case = synth.nvfp4_lora_case(seed=13, M=4, N=3, K=64)
    a, b, asf, bsf = (case.a.numpy(), case.b.numpy(), case.a_sf.numpy().copy(),
                      case.b_sf.numpy())
    base0 = N.base_product(a, b, asf, bsf, 64)
    off = N.sf_offset(2, 1, 64)
    asf[off] += 8                        # exponent + 1 => value x2 (stays < 0x7F)
    base1 = N.base_product(a, b, asf, bsf, 64)
    da = N.dequant(a, case.a_sf.numpy(), 64)
    db = N.dequant(b, bsf, 64)
    blk = slice(16, 32)
    want = base0.copy()
    want[2] += da[2, blk] @ db[:, blk].T
    assert np.allclose(base1, want, rtol=1e-14, atol=0)
