"""MoE finalize (combine) with the FC2 LoRA delta added.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows ``flashinfer.fused_moe.bgmv_moe_gemm2_lora_delta`` (the description
and the return value): the delta is combined over the experts like the FC2
output and is added to the MoE output after the combine.  The combine itself
is the finalize step named on ``flashinfer.fused_moe.prims_ts_fp4_block_scale_moe``
(parameter ``do_finalize``): each token's output is the routing-weighted sum
of the FC2 rows of its routed slots.  Written out:

    moe_out[t] = sum_j w[t, j] * fc2[perm[t*top_k + j]] + delta[t]

with ``w = topk_weights`` and ``fc2`` the FC2 grouped-GEMM output in permuted
row order.

Readings (each listed with its reason in the design notes):
- a slot whose permuted row is negative or at least ``padded_rows`` is not
  routed to this rank and contributes nothing (the same slots the delta skips
  for that reason);
- ``delta`` is the exact delta of :mod:`oracle.lora_delta` (a token without
  adapter has a zero delta and still gets its combine);
- the value is exact (float64); the GPU rounds the whole sum once.
"""
from __future__ import annotations

import numpy as np

from .formats import to_f64


def fc2_rows_f64(fc2, dtype: str) -> np.ndarray:
    """FC2 rows as float64: ``fc2`` holds uint16 patterns of ``dtype`` ("bf16"
    or "f16") or float32 values (``dtype`` "f32")."""
    if dtype == "f32":
        return np.asarray(fc2, dtype=np.float32).astype(np.float64)
    return to_f64(np.asarray(fc2, dtype=np.uint16), dtype)


def moe_finalize(fc2, fc2_dtype: str, perm, topk_weights, delta, tokens=None) -> np.ndarray:
    """float64 ``[len(tokens), H]`` combined output (all tokens by default).

    ``fc2`` ``[padded_rows, H]`` (see :func:`fc2_rows_f64`), ``perm`` int
    ``[T*top_k]``, ``topk_weights`` float32 ``[T, top_k]``, ``delta`` float64
    ``[len(tokens), H]`` for the same tokens (zeros for no LoRA).
    """
    w = np.asarray(topk_weights, dtype=np.float32).astype(np.float64)
    T, top_k = w.shape
    perm = np.asarray(perm, dtype=np.int64).reshape(-1)
    rows = np.asarray(fc2)
    padded_rows, H = rows.shape
    tokens = list(range(T)) if tokens is None else list(tokens)
    out = np.array(delta, dtype=np.float64, copy=True).reshape(len(tokens), H)
    for i, t in enumerate(tokens):
        acc = np.zeros(H, dtype=np.float64)
        for j in range(top_k):
            p = int(perm[t * top_k + j])
            if p < 0 or p >= padded_rows:
                continue
            acc += w[t, j] * fc2_rows_f64(rows[p], fc2_dtype)
        out[i] += acc
    return out
