"""FC1 (gate/up) LoRA delta of a routed MoE.

TEST INFRASTRUCTURE ONLY (see the package docstring).

``flashinfer.fused_moe.bgmv_moe_gemm2_lora_delta`` (description) says that
the FC1 side runs with ``gemm1_lora_delta`` set, and the FP4 fused-MoE page
(``prims_ts_fp4_block_scale_moe``, parameters) takes FC1 as the gate/up
product of the permuted activations with ``gemm1_weights``.  Neither page
writes the FC1 delta out.  Reading taken here, the FC1 counterpart of the
FC2 formula on the delta page:

    delta1[p] = scale * B_up[l, e] @ (A_up[l, e] @ x[p])      p = perm[t*top_k + j]

for every slot ``(t, j)`` whose permuted row ``p`` lies in ``[0, padded_rows)``,
with ``e = topk_ids[t, j]``, ``l = lora_ids[t]`` and ``x[p]`` the permuted FC1
input row (the row the FC1 GEMM multiplies).  Unlike FC2 there is no routing
weight and no combine: each routed row gets its own delta, ``[2I]`` wide,
which the FC1 GEMM adds before its activation.  A slot whose token has no
adapter (``l < 0``) or whose expert lies outside ``[0, E)`` gets a +0 row.
Rows no slot points at are not written.

The pointer tables resolve the banks exactly as for the FC2 delta:
``A_up[l, e]`` is the ``[rank, hidden]`` block ``l * lora_stride_a`` elements
after byte address ``w_ptr_a[e]``, ``B_up[l, e]`` the ``[out_features, rank]``
block ``l * lora_stride_b`` elements after ``w_ptr_b[e]``.  The value is exact
(float64 from the 16-bit inputs); the GPU rounds it once.
"""
from __future__ import annotations

import numpy as np

from .formats import to_f64
from .lora_delta import Bank


def moe_fc1_lora_delta(act_bits, perm, bank_a: Bank, w_ptr_a, stride_a, bank_b: Bank, w_ptr_b,
                       stride_b, topk_ids, lora_ids, rank: int, out_features: int, scale: float,
                       num_experts: int, rows=None, lora_dtype: str = "bf16"):
    """Return ``(out, written)``: float64 ``[len(rows), out_features]`` and a
    bool mask of the rows some slot writes.  ``act_bits`` holds the permuted
    FC1 input ``[padded_rows, hidden]`` as ``lora_dtype`` patterns; ``rows``
    selects output rows (all ``padded_rows`` by default)."""
    act = np.asarray(act_bits, dtype=np.uint16)
    padded_rows, hidden = act.shape
    assert bank_a.dtype == lora_dtype and bank_b.dtype == lora_dtype, "one lora_dtype"
    perm = np.asarray(perm, dtype=np.int64).reshape(-1)
    topk_ids = np.asarray(topk_ids, dtype=np.int64)
    lora_ids = np.asarray(lora_ids, dtype=np.int64).reshape(-1)
    w_ptr_a = np.asarray(w_ptr_a, dtype=np.int64).reshape(-1)
    w_ptr_b = np.asarray(w_ptr_b, dtype=np.int64).reshape(-1)
    T, top_k = topk_ids.shape
    scale = float(np.float32(scale))
    rows = list(range(padded_rows)) if rows is None else [int(r) for r in rows]
    where = {r: i for i, r in enumerate(rows)}
    out = np.zeros((len(rows), out_features), dtype=np.float64)
    written = np.zeros(len(rows), dtype=bool)
    for t in range(T):
        l = int(lora_ids[t])
        for j in range(top_k):
            p = int(perm[t * top_k + j])
            if p < 0 or p >= padded_rows or p not in where:
                continue
            i = where[p]
            written[i] = True
            e = int(topk_ids[t, j])
            if l < 0 or e < 0 or e >= num_experts:
                out[i] = 0.0
                continue
            A_le = bank_a.block(w_ptr_a[e], l * int(stride_a), (rank, hidden))
            B_le = bank_b.block(w_ptr_b[e], l * int(stride_b), (out_features, rank))
            out[i] = scale * (B_le @ (A_le @ to_f64(act[p], lora_dtype)))
    return out, written
