"""FC2 (down-projection) LoRA delta of a routed MoE.

Follows ``flashinfer.fused_moe.bgmv_moe_gemm2_lora_delta`` (the formula and
the parameter list):

    delta[t] = scale * sum_j w[t, j] * ( B_down[l, e] @ (A_down[l, e] @ a[t, j]) )

with ``e = topk_ids[t, j]``, ``w = topk_weights``, ``l = lora_ids[t]``.

Readings of the page (each listed with its reason in the design notes):
- ``a[t, j]`` is row ``expanded_idx_to_permuted_idx[t*top_k + j]`` of the
  PERMUTED activation; a negative entry marks an inactive slot, skipped;
- ``lora_ids[t] < 0`` means no adapter: the token's delta is +0;
- ``A_down[l, e]`` is the ``[rank, I]`` block that starts ``l * lora_stride_a``
  elements after the byte address ``w_ptr_a[0, e]``; ``B_down[l, e]`` is the
  ``[H, rank]`` block ``l * lora_stride_b`` elements after ``w_ptr_b[0, e]``;
- ``lora_dtype`` (bf16 or fp16, as the parameter list allows) is the type of
  both the activation buffer and the LoRA banks;
- the value is exact (float64 from the bf16/fp16/fp32 inputs); the GPU rounds
  it once to ``out_dtype``.
"""
from __future__ import annotations

import numpy as np

from .formats import to_f64

BF16_BYTES = 2


class Bank:
    """A LoRA weight bank as the device sees it: a flat uint16 array of
    ``dtype`` ("bf16" or "f16") patterns that starts at byte address ``base``.
    Blocks are resolved from byte addresses plus element strides, exactly as
    the pointer tables do."""

    def __init__(self, flat_bits: np.ndarray, base: int, dtype: str = "bf16"):
        self.flat = np.asarray(flat_bits, dtype=np.uint16).reshape(-1)
        self.base = int(base)
        self.dtype = dtype

    def block(self, byte_addr: int, elem_offset: int, shape) -> np.ndarray:
        start_bytes = int(byte_addr) - self.base
        assert start_bytes % BF16_BYTES == 0 and start_bytes >= 0
        start = start_bytes // BF16_BYTES + int(elem_offset)
        count = int(np.prod(shape))
        assert start + count <= self.flat.size, "pointer/stride outside the bank"
        return to_f64(self.flat[start:start + count], self.dtype).reshape(shape)


def moe_fc2_lora_delta(act_bits, perm, bank_a: Bank, w_ptr_a, stride_a, bank_b: Bank, w_ptr_b,
                       stride_b, topk_ids, topk_weights, lora_ids, rank: int, hidden: int,
                       scale: float, tokens=None, lora_dtype: str = "bf16") -> np.ndarray:
    """float64 ``[len(tokens), H]`` delta (all tokens by default); ``act_bits``
    and both banks hold ``lora_dtype`` patterns.

    Vectorised per slot; the per-slot work is one ``[r, I] @ [I]`` product
    and one ``[H, r] @ [r]`` product exactly as the formula nests them.
    """
    act = act_bits  # uint16 [padded_rows, I]; rows decoded on demand
    assert bank_a.dtype == lora_dtype and bank_b.dtype == lora_dtype, "one lora_dtype"
    I = act.shape[1]
    perm = np.asarray(perm, dtype=np.int64).reshape(-1)
    topk_ids = np.asarray(topk_ids, dtype=np.int64)
    w = np.asarray(topk_weights, dtype=np.float32).astype(np.float64)
    lora_ids = np.asarray(lora_ids, dtype=np.int64).reshape(-1)
    w_ptr_a = np.asarray(w_ptr_a, dtype=np.int64).reshape(-1)
    w_ptr_b = np.asarray(w_ptr_b, dtype=np.int64).reshape(-1)
    T, top_k = topk_ids.shape
    scale = float(np.float32(scale))
    if tokens is None:
        tokens = range(T)
    tokens = list(tokens)
    out = np.zeros((len(tokens), hidden), dtype=np.float64)
    for i, t in enumerate(tokens):
        l = int(lora_ids[t])
        if l < 0:
            continue
        acc = np.zeros(hidden, dtype=np.float64)
        for j in range(top_k):
            p = int(perm[t * top_k + j])
            if p < 0:
                continue
            e = int(topk_ids[t, j])
            A_le = bank_a.block(w_ptr_a[e], l * int(stride_a), (rank, I))
            B_le = bank_b.block(w_ptr_b[e], l * int(stride_b), (hidden, rank))
            x = to_f64(act[p], lora_dtype)
            acc += w[t, j] * (B_le @ (A_le @ x))
        out[i] = scale * acc
    return out
