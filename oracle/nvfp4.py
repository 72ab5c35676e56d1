"""NVFP4 base GEMM with a BF16 LoRA correction.

Follows ``flashinfer.gemm.mm_nvfp4_lora`` (the formula, the raw-path and
prepared-path bullets and the parameter list):

    out = alpha * (dequant(a) @ dequant(b)^T) + lora_scale * (d @ lora_b^T) [+ bias]

- ``a`` is uint8 ``[M, K/2]``, ``b`` uint8 ``[N, K/2]``: E2M1 codes, a pair in each
  byte, row-major;
- ``a_sf`` / ``b_sf``: one UE4M3 scale per 16 elements along K, in the
  128x4-tiled layout with rows padded to 128;
- ``alpha``: element 0 of an fp32 tensor; ``lora_scale``: fp32 scalar;
- raw path: ``d`` and ``lora_b`` used as given, ``alpha`` and ``lora_scale``
  independent; prepared path: ``alpha * (base + d @ b_folded^T)``;
  adapter off (no adapter, ``lora_scale`` None or 0, or a prepared adapter of
  scale 0): ``alpha * base`` -- all plus bias, rounded once by the GPU.

Two layout conventions are named on the page but not defined there; this
module takes the public convention for both (**parity unpinned** by the
pages):
- nibble order: element ``2i`` is the LOW nibble of byte ``i`` of a row,
  element ``2i+1`` the high nibble;
- 128x4 scale tiling: rows are grouped in blocks of 128 and scale columns in
  blocks of 4; each 128x4 block is a 512-byte tile, tiles ordered row-block
  major; inside a tile row ``r`` and column ``c`` sit at byte
  ``(r % 32) * 16 + ((r % 128) // 32) * 4 + (c % 4)``.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64, e2m1_to_f64, ue4m3_to_f64

SF_VEC = 16  # elements per scale along K


def sf_offset(row, col, k: int):
    """Byte offset of the scale of (row, scale column col) in the 128x4
    tiled buffer of a matrix with ``k`` elements per row."""
    row = np.asarray(row, dtype=np.int64)
    col = np.asarray(col, dtype=np.int64)
    n_cols = -(-k // SF_VEC)            # ceil(k / 16) scale columns
    n_col_tiles = -(-n_cols // 4)       # ceil(n_cols / 4) tiles per row block
    tile = (row // 128) * n_col_tiles + col // 4
    return tile * 512 + (row % 32) * 16 + ((row % 128) // 32) * 4 + (col % 4)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """uint8 ``[rows, K/2]`` -> E2M1 codes ``[rows, K]`` (low nibble first)."""
    p = np.asarray(packed, dtype=np.uint8)
    codes = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    codes[:, 0::2] = p & 0xF
    codes[:, 1::2] = p >> 4
    return codes


def scales(sf: np.ndarray, rows, k: int) -> np.ndarray:
    """UE4M3 scale values ``[len(rows), k/16]`` for the given row indices."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.arange(k // SF_VEC, dtype=np.int64)
    off = sf_offset(rows[:, None], cols[None, :], k)
    return ue4m3_to_f64(np.asarray(sf, dtype=np.uint8).reshape(-1)[off])


def dequant(packed: np.ndarray, sf: np.ndarray, k: int, rows=None) -> np.ndarray:
    """float64 ``[rows, k]``: E2M1 value times its block's UE4M3 scale.

    ``packed`` holds the selected rows' codes (all rows when ``rows`` is
    None); ``rows`` are their indices in the full matrix (they select the
    scales).  The products are exact (at most 6 significant bits).
    """
    packed = np.asarray(packed, dtype=np.uint8)
    if rows is None:
        rows = np.arange(packed.shape[0])
    vals = e2m1_to_f64(unpack_codes(packed))
    s = scales(sf, rows, k)
    return vals * np.repeat(s, SF_VEC, axis=1)


def base_product(a, b, a_sf, b_sf, k: int, a_rows=None, b_rows=None) -> np.ndarray:
    """``dequant(a) @ dequant(b)^T`` in float64."""
    return dequant(a, a_sf, k, a_rows) @ dequant(b, b_sf, k, b_rows).T


def lora_term(d_bits, lora_b_bits) -> np.ndarray:
    """``d @ lora_b^T`` in float64 (``d`` [M, r], ``lora_b`` [N, r] bf16)."""
    return bf16_to_f64(d_bits) @ bf16_to_f64(lora_b_bits).T


def _bias_row(bias_bits, n):
    return np.zeros(n) if bias_bits is None else bf16_to_f64(bias_bits)


def mm_nvfp4_off(base, alpha, bias_bits=None) -> np.ndarray:
    """Adapter-off output: ``alpha * base + bias``."""
    a = float(np.float32(alpha))
    return a * base + _bias_row(bias_bits, base.shape[1])[None, :]


def mm_nvfp4_raw(base, alpha, d_bits, lora_b_bits, lora_scale, bias_bits=None) -> np.ndarray:
    """Raw path: ``alpha * base + lora_scale * (d @ lora_b^T) + bias``.  A zero
    scale is the adapter-off output."""
    a = float(np.float32(alpha))
    s = float(np.float32(lora_scale))
    out = a * base + _bias_row(bias_bits, base.shape[1])[None, :]
    if s != 0.0:
        out = out + s * lora_term(d_bits, lora_b_bits)
    return out


def mm_nvfp4_prepared(base, alpha, d_bits, b_folded_bits, zero_adapter: bool,
                      bias_bits=None) -> np.ndarray:
    """Prepared path: ``alpha * (base + d @ b_folded^T) + bias``; a prepared
    adapter of scale 0 is the adapter-off output."""
    a = float(np.float32(alpha))
    if zero_adapter:
        return mm_nvfp4_off(base, alpha, bias_bits)
    return a * (base + lora_term(d_bits, b_folded_bits)) + _bias_row(bias_bits,
                                                                     base.shape[1])[None, :]
