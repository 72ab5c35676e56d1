"""Ragged per-expert grouped GEMM.

Follows ``flashinfer.grouped_mm.grouped_mm_bf16`` (the formula and the
parameter list): for every expert ``e`` with ``start, end = m_indptr[e],
m_indptr[e+1]``, ``out[start:end] = a[start:end] @ b[e]^T``; ``a`` is
``(cum_m, k)``, ``b`` is ``(batch_size, n, k)``, ``m_indptr`` holds cumulative
token counts.

Readings where the page is silent:
- the output has ``a.shape[0]`` rows; rows outside
  ``[m_indptr[0], m_indptr[-1])`` are not defined by the formula and are
  reported as not written;
- the value is the exact product of the bf16 (or fp16) inputs, computed in
  float64; the GPU rounds it once to the output dtype.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64, to_f64


def grouped_mm(a_bits: np.ndarray, b_bits: np.ndarray, m_indptr: np.ndarray,
               dtype: str = "bf16"):
    """Return ``(out, written)``: float64 ``[cum_m, n]`` and a bool row mask.

    ``a_bits`` uint16 ``[cum_m, k]``, ``b_bits`` uint16 ``[E, n, k]`` (bit
    patterns of ``dtype``, "bf16" or "f16"), ``m_indptr`` int ``[E+1]``
    (non-decreasing).
    """
    A = to_f64(a_bits, dtype)
    B = to_f64(b_bits, dtype)
    m_indptr = np.asarray(m_indptr, dtype=np.int64)
    cum_m = A.shape[0]
    E, n, k = B.shape
    assert A.shape[1] == k and m_indptr.shape == (E + 1,)
    out = np.zeros((cum_m, n), dtype=np.float64)
    written = np.zeros(cum_m, dtype=bool)
    for e in range(E):
        s, t = int(m_indptr[e]), int(m_indptr[e + 1])
        if t <= s:
            continue
        out[s:t] = A[s:t] @ B[e].T
        written[s:t] = True
    return out, written


def expert_of_row(m_indptr: np.ndarray, row: int) -> int:
    """The expert whose range ``[m_indptr[e], m_indptr[e+1])`` holds ``row``."""
    m_indptr = np.asarray(m_indptr, dtype=np.int64)
    e = int(np.searchsorted(m_indptr, row, side="right") - 1)
    assert 0 <= e < m_indptr.size - 1 and m_indptr[e] <= row < m_indptr[e + 1]
    return e


def grouped_mm_rows(a_rows_bits: np.ndarray, b_rows_of_expert, m_indptr: np.ndarray, rows,
                    cols=None):
    """Selected output elements, one row at a time, for full-size checks.

    ``a_rows_bits[i]`` is row ``rows[i]`` of ``a``; ``b_rows_of_expert(e, cols)``
    returns the uint16 rows ``b[e, cols, :]`` (all rows when cols is None).
    """
    res = []
    for i, r in enumerate(rows):
        e = expert_of_row(m_indptr, int(r))
        Bsel = bf16_to_f64(b_rows_of_expert(e, cols))
        res.append(Bsel @ bf16_to_f64(a_rows_bits[i]))
    return np.stack(res)
