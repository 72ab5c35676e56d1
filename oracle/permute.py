"""Routing output -> expert-sorted permutation, and the permuted rows.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows ``flashinfer.fused_moe.bgmv_moe_gemm2_lora_delta`` (parameter
``expanded_idx_to_permuted_idx``: entry ``token*top_k + slot`` holds that
slot's row in the permuted buffer, or a negative value when the slot is
inactive) and
``flashinfer.grouped_mm.grouped_mm_bf16`` (parameter ``m_indptr``: cumulative
row counts of the groups, one group per expert).

Readings (each listed with its reason in the design notes):
- the permuted order is a stable sort of the expanded slots by expert id:
  expert ``e``'s rows are ``m_indptr[e] .. m_indptr[e+1]-1`` and inside an
  expert the slots keep their expanded order;
- a slot whose expert id lies outside ``[0, num_experts)`` is not routed here:
  its entry is -1 and it takes no row;
- the permuted rows are the token rows: row ``perm[t*top_k + j]`` of the
  permuted matrix is row ``t`` of the token matrix (rows no slot maps to are
  left as they were).
"""
from __future__ import annotations

import numpy as np


def route_permutation(topk_ids, num_experts: int):
    """``(m_indptr [E+1], perm [T*k], inverse [T*k])`` as int64 arrays.

    ``inverse[p]`` is the expanded index at permuted row ``p`` for
    ``p < m_indptr[E]`` and -1 after.  A stable sort (a library primitive)
    and counts, as the reading states.
    """
    flat = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    valid = (flat >= 0) & (flat < num_experts)
    idx = np.nonzero(valid)[0]
    order = idx[np.argsort(flat[idx], kind="stable")]
    perm = np.full(flat.size, -1, dtype=np.int64)
    perm[order] = np.arange(order.size)
    counts = np.bincount(flat[idx], minlength=num_experts)[:num_experts]
    m_indptr = np.zeros(num_experts + 1, dtype=np.int64)
    m_indptr[1:] = np.cumsum(counts)
    inverse = np.full(flat.size, -1, dtype=np.int64)
    inverse[:order.size] = order
    return m_indptr, perm, inverse


def permute_rows(x, perm, top_k: int, out):
    """``out[perm[t*top_k + j]] = x[t]`` for every slot with ``perm >= 0``
    (``out`` is modified and returned; ``perm`` entries past ``out`` skipped)."""
    x = np.asarray(x)
    perm = np.asarray(perm, dtype=np.int64).reshape(-1)
    for s, p in enumerate(perm):
        if 0 <= p < out.shape[0]:
            out[p] = x[s // top_k]
    return out
