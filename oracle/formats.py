"""Number formats used by the pages, decoded exactly into float64.

- bf16: the 16 high bits of an IEEE binary32.
- fp16: IEEE binary16 (1 sign, 5 exponent bits with bias 15, 10 mantissa
  bits; subnormals at exponent 0) -- the other input and output type the
  grouped_mm_bf16 page lists.
- E2M1 (the NVFP4 element code; ``flashinfer.gemm.mm_nvfp4_lora``,
  parameters a and b, stores two such codes in each byte): 1 sign,
  2 exponent (bias 1), 1 mantissa bit; magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
  The pages only name the format; the values follow the OCP microscaling
  definition.
- UE4M3 (the NVFP4 block scale; same page, parameters a_sf and b_sf: one
  scale for every 16 consecutive elements along K): an E4M3 byte (4 exponent
  bits, bias 7, 3 mantissa bits, subnormal at exponent 0, 0x7F = NaN) whose
  sign bit is zero.

All decoders are exact: every value of these formats is a float64.
"""
from __future__ import annotations

import numpy as np

# E2M1 magnitudes indexed by the low three bits of the code.
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to bf16 once, to nearest with ties to even.

    Written from the definition: find the spacing of bf16 numbers in the
    binade of |x| (8 significant bits; subnormal spacing 2**-133), round the
    quotient to an integer with ties to even (``np.rint``), and rebuild the
    value.  Overflow past the largest finite bf16 gives +-Inf, NaN gives the
    canonical quiet NaN 0x7FC0.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    finite = np.isfinite(x)
    axf = np.where(finite, ax, 0.0)
    _, e = np.frexp(axf)                       # axf = m * 2**e, m in [0.5, 1)
    q = np.maximum(e - 8, -133)                # exponent of one unit in the last place
    y = np.ldexp(np.rint(np.ldexp(axf, -q)), q)
    max_finite = (2.0 - 2.0 ** -7) * 2.0 ** 127
    overflow = y > max_finite
    y = np.where(overflow, 0.0, y)
    bits = (y.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(overflow | (np.isinf(x)), np.uint16(0x7F80), bits)
    bits = bits | (np.signbit(x).astype(np.uint16) << np.uint16(15))
    bits = np.where(np.isnan(x), np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


def f16_to_f64(bits) -> np.ndarray:
    """fp16 bit patterns (uint16) -> float64, from the field definition."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(u >> 15, -1.0, 1.0)
    E = (u >> 10) & 0x1F
    M = u & 0x3FF
    mag = np.where(E == 0, M * 2.0 ** -24, (1.0 + M / 1024.0) * np.ldexp(1.0, E - 15))
    val = sign * mag
    val = np.where((E == 31) & (M == 0), sign * np.inf, val)
    return np.where((E == 31) & (M != 0), np.nan, val)


def f64_to_f16_bits(x) -> np.ndarray:
    """Round float64 values to fp16 once, to nearest with ties to even.

    Same construction as :func:`f64_to_bf16_bits`: 11 significant bits,
    subnormal spacing 2**-24, overflow past 65504 gives +-Inf, NaN gives
    0x7E00.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    finite = np.isfinite(x)
    axf = np.where(finite, ax, 0.0)
    _, e = np.frexp(axf)
    q = np.maximum(e - 11, -24)
    y = np.ldexp(np.rint(np.ldexp(axf, -q)), q)
    overflow = y > 65504.0
    y = np.where(overflow, 0.0, y)
    # y is now an exact fp16 magnitude: encode its fields
    _, ey = np.frexp(np.where(y > 0, y, 1.0))
    normal = y >= 2.0 ** -14
    E = np.where(normal, ey - 1 + 15, 0)
    M = np.where(normal, np.ldexp(y, -(ey - 1)) * 1024.0 - 1024.0, y * 2.0 ** 24)
    bits = ((E.astype(np.int64) << 10) | np.rint(M).astype(np.int64)).astype(np.uint16)
    bits = np.where(y == 0, np.uint16(0), bits)
    bits = np.where(overflow | np.isinf(x), np.uint16(0x7C00), bits)
    bits = bits | (np.signbit(x).astype(np.uint16) << np.uint16(15))
    bits = np.where(np.isnan(x), np.uint16(0x7E00), bits)
    return bits.astype(np.uint16)


def to_f64(bits, dtype: str) -> np.ndarray:
    """Decode 16-bit patterns of the named type ("bf16" or "f16")."""
    if dtype == "bf16":
        return bf16_to_f64(bits)
    if dtype == "f16":
        return f16_to_f64(bits)
    raise ValueError(dtype)


def e2m1_to_f64(codes) -> np.ndarray:
    """E2M1 codes (low 4 bits used) -> float64; code 8 is -0."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where(c & 8, -mag, mag)


def ue4m3_to_f64(codes) -> np.ndarray:
    """UE4M3 scale bytes -> float64.

    Exponent field ``E = u >> 3`` and mantissa ``M = u & 7``: subnormal
    ``M * 2**-9`` when E == 0, else ``(1 + M/8) * 2**(E-7)``.  0x7F is NaN;
    bytes with the sign bit set are not UE4M3 and decode to NaN here.
    """
    u = np.asarray(codes).astype(np.int64)
    E = (u >> 3) & 0xF
    M = u & 7
    val = np.where(E == 0, M * 2.0 ** -9, (1.0 + M / 8.0) * np.ldexp(1.0, E - 7))
    bad = (u == 0x7F) | (u >= 0x80)
    return np.where(bad, np.nan, val)
