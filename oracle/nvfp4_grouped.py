"""NVFP4 block-scaled grouped GEMM: ragged per-expert products with FP4
expert weights.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Joins two pages' definitions:
- the ragged walk of ``flashinfer.grouped_mm.grouped_mm_bf16`` (formula):
  ``out[m_indptr[e]:m_indptr[e+1]] = a[...] @ b[e]^T`` for every expert;
- the NVFP4 operand format of ``flashinfer.gemm.mm_nvfp4_lora`` (parameters
  a, b, a_sf, b_sf, alpha): E2M1 codes two per byte, one UE4M3 scale per 16
  elements along K in the 128x4 layout, ``alpha`` the base scale applied to
  the fp32 product -- the weight format the FP4 fused-MoE page names for its
  expert weights (``prims_ts_fp4_block_scale_moe``, parameters
  ``gemm1_weights`` / ``gemm2_weights`` and their scales, and the per-expert
  output scales).

Readings (each listed with its reason in the design notes):
- ``a`` uint8 ``[cum_m, K/2]`` with ONE scale buffer over all ``cum_m`` rows
  (rows padded to 128): the activations are quantised as one matrix;
- ``b`` uint8 ``[E, N, K/2]``; ``b_sf`` holds E consecutive scale buffers,
  each the 128x4 layout of that expert's ``[N, K/16]`` scales;
- ``alpha`` fp32 ``[E]``, one base scale per expert (the per-expert output
  scale of the fused-MoE page): ``out = alpha[e] * (dequant(a) @ dequant(b[e])^T)``;
- the value is exact (float64); the GPU rounds it once.  Rows outside
  ``[m_indptr[0], m_indptr[E])`` are not written.
"""
from __future__ import annotations

import numpy as np

from .nvfp4 import base_product


def expert_sf_bytes(n: int, k: int) -> int:
    """Bytes of one expert's 128x4 scale buffer for ``[n, k/16]`` scales."""
    cols = -(-k // 16)
    return (-(-n // 128)) * (-(-cols // 4)) * 512


def grouped_mm_nvfp4(a, a_sf, b, b_sf, alpha, m_indptr, k: int):
    """Return ``(out, written)``: float64 ``[cum_m, N]`` and a bool row mask."""
    a = np.asarray(a, dtype=np.uint8)
    b = np.asarray(b, dtype=np.uint8)
    E, n, _ = b.shape
    m_indptr = np.asarray(m_indptr, dtype=np.int64)
    alpha = np.asarray(alpha, dtype=np.float32).astype(np.float64).reshape(-1)
    assert m_indptr.shape == (E + 1,) and alpha.shape == (E,)
    per = expert_sf_bytes(n, k)
    b_sf = np.asarray(b_sf, dtype=np.uint8).reshape(-1)
    out = np.zeros((a.shape[0], n), dtype=np.float64)
    written = np.zeros(a.shape[0], dtype=bool)
    for e in range(E):
        s, t = int(m_indptr[e]), int(m_indptr[e + 1])
        if t <= s:
            continue
        rows = np.arange(s, t)
        prod = base_product(a[s:t], b[e], a_sf, b_sf[e * per:(e + 1) * per], k, a_rows=rows)
        out[s:t] = alpha[e] * prod
        written[s:t] = True
    return out, written


def grouped_mm_nvfp4_rows(a_rows, a_sf, b_codes_of, b_sf, alpha, m_indptr, k: int, n: int,
                          rows, cols):
    """float64 ``[len(rows), len(cols)]``: the same values at sampled rows
    (each inside some group) and columns, one row at a time.

    ``a_rows`` holds the codes of the sampled rows ``[len(rows), K/2]``;
    ``b_codes_of(e)`` returns expert ``e``'s codes at ``cols`` ``[len(cols), K/2]``
    (so a large ``b`` need not be copied whole).
    """
    a_rows = np.asarray(a_rows, dtype=np.uint8)
    m_indptr = np.asarray(m_indptr, dtype=np.int64)
    alpha = np.asarray(alpha, dtype=np.float32).astype(np.float64).reshape(-1)
    E = m_indptr.size - 1
    per = expert_sf_bytes(n, k)
    b_sf = np.asarray(b_sf, dtype=np.uint8).reshape(-1)
    cols = np.asarray(cols, dtype=np.int64)
    out = np.empty((len(rows), len(cols)), dtype=np.float64)
    for i, r in enumerate(rows):
        e = int(np.searchsorted(m_indptr, r, side="right")) - 1
        assert 0 <= e < E and m_indptr[e] <= r < m_indptr[e + 1]
        prod = base_product(a_rows[i:i + 1], np.asarray(b_codes_of(e), dtype=np.uint8), a_sf,
                            b_sf[e * per:(e + 1) * per], k, a_rows=[r], b_rows=cols)
        out[i] = alpha[e] * prod[0]
    return out
