"""NVFP4 quantisation: a real matrix -> E2M1 codes and UE4M3 block scales.

TEST INFRASTRUCTURE ONLY (see the package docstring).

``flashinfer.gemm.mm_nvfp4_lora`` (the paragraph after the formula) takes its
operands as the output of ``fp4_quantize()``: E2M1 codes, a pair in each
byte, and one UE4M3 scale for every 16 elements along K in the 128x4 layout;
its ``alpha`` parameter is ``alpha_base / (a_global_scale * b_global_scale)``,
so the quantised operand stands for the matrix multiplied by a per-tensor
global scale ``g``.  The pages name the producer but do not spell out its
steps.  Reading taken here (the usual NVFP4 recipe, every arithmetic step in
IEEE fp32 with round-to-nearest-even, so that both implementations decide
every code in the same precision):

for each row and each block of 16 consecutive elements ``x_i`` along K:
  1. ``amax = max_i |x_i|``;
  2. ``s = fl32(fl32(amax * g) / 6)`` -- the scale that maps the block's
     largest magnitude onto 6, the largest E2M1 magnitude;
  3. ``sf`` = the UE4M3 code nearest to ``s`` (ties to the even code, i.e.
     mantissa bit 0 clear); anything at or above 448 saturates to 0x7E (448);
     ``S`` = its value;
  4. ``r = fl32(g / S)``, or 0 when ``S == 0``;
  5. each element: ``t = fl32(x_i * r)``, code = the E2M1 value nearest to
     ``|t|`` (ties to the even code), magnitudes above 6 saturate to 6, the
     sign bit is the sign of ``t`` (so ``-0`` gives code 8).

Layout: codes ``[rows, K/2]`` with element ``2i`` in the low nibble; scales
in the 128x4 tiling of :mod:`oracle.nvfp4` with every padding byte (rows past
the last, up to the multiple of 128) zero.  ``dequant(codes, sf) / g``
approximates the input: per element the error is at most ``S / g`` (checked
in the tests).
"""
from __future__ import annotations

import numpy as np

from .formats import E2M1_MAGNITUDES, ue4m3_to_f64
from .nvfp4 import sf_offset

# every finite UE4M3 value, ascending with the code (codes 0x00 .. 0x7E)
_UE4M3_VALUES = ue4m3_to_f64(np.arange(0x7F))
UE4M3_MAX_CODE = 0x7E


def nearest_code(v: float, table: np.ndarray) -> int:
    """Index of the entry of the ascending ``table`` nearest to ``v >= 0``;
    on a tie the even index; past the last entry the last index."""
    if v >= table[-1]:
        return len(table) - 1
    hi = int(np.searchsorted(table, v, side="left"))  # table[hi-1] < v <= table[hi]
    if hi == 0:
        return 0
    lo = hi - 1
    dl, dh = v - table[lo], table[hi] - v
    if dl < dh:
        return lo
    if dh < dl:
        return hi
    return lo if lo % 2 == 0 else hi


def ue4m3_round(s: np.float32) -> int:
    """Step 3: fp32 ``s >= 0`` -> UE4M3 code (nearest, ties even, saturating)."""
    return nearest_code(float(s), _UE4M3_VALUES)


def e2m1_round(t: np.float32) -> int:
    """Step 5: fp32 ``t`` -> E2M1 code (nearest magnitude, ties even,
    saturating at 6; sign bit from the sign of ``t``)."""
    mag = nearest_code(abs(float(t)), E2M1_MAGNITUDES)
    return mag | (8 if np.signbit(t) else 0)


def quantize_block(x16: np.ndarray, g: np.float32):
    """One block of 16 fp32 values: ``(codes[16], scale code)``."""
    x16 = np.asarray(x16, dtype=np.float32)
    g = np.float32(g)
    amax = np.float32(np.max(np.abs(x16)))
    s = np.float32(np.float32(amax * g) / np.float32(6.0))
    sf = ue4m3_round(s)
    S = np.float32(_UE4M3_VALUES[sf])
    r = np.float32(g / S) if S != 0 else np.float32(0.0)
    codes = [e2m1_round(np.float32(xi * r)) for xi in x16]
    return codes, sf


def quantize_rows(x: np.ndarray, g):
    """Rows of ``x`` (float32-representable values ``[n, K]``) quantised with
    global scale ``g``: ``(codes uint8 [n, K/2], scale codes uint8 [n, K/16])``
    -- the scales in plain row order, before the 128x4 placement."""
    x = np.asarray(x, dtype=np.float32)
    n, K = x.shape
    assert K % 16 == 0
    codes = np.zeros((n, K // 2), dtype=np.uint8)
    scodes = np.zeros((n, K // 16), dtype=np.uint8)
    for r in range(n):
        for b in range(K // 16):
            c, s = quantize_block(x[r, 16 * b:16 * b + 16], g)
            scodes[r, b] = s
            for i in range(0, 16, 2):
                codes[r, 8 * b + i // 2] = c[i] | (c[i + 1] << 4)
    return codes, scodes


def place_scales(scodes: np.ndarray, rows: int, K: int) -> np.ndarray:
    """Scale codes ``[rows, K/16]`` placed in the 128x4 tiled buffer (rows
    padded to 128, padding bytes zero)."""
    nblk = K // 16
    n_col_tiles = -(-nblk // 4)
    sf = np.zeros((-(-rows // 128)) * n_col_tiles * 512, dtype=np.uint8)
    r = np.arange(rows)[:, None]
    c = np.arange(nblk)[None, :]
    sf[sf_offset(r, c, K)] = scodes
    return sf


def fp4_quantize(x: np.ndarray, g):
    """Quantise ``x`` (float32-representable values ``[rows, K]``) with global
    scale ``g``.  Returns ``(codes uint8 [rows, K/2], sf uint8 [padded])``."""
    x = np.asarray(x, dtype=np.float32)
    codes, scodes = quantize_rows(x, g)
    return codes, place_scales(scodes, x.shape[0], x.shape[1])
