"""Pointer tables and bank layouts for the LoRA-delta tests.

``contiguous_tables`` addresses a plain ``[L, E, r, I]`` / ``[L, E, H, r]``
bank (adapter stride = one adapter's slab).  ``scattered_bank`` builds a bank
whose per-expert blocks sit in a shuffled order with a padded adapter stride,
so that a wrong pointer or stride computation reads the wrong numbers.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle.lora_delta import Bank
from tests.parity import bits16


def contiguous_tables(bank: torch.Tensor):
    """``(w_ptr int64 [1, E], stride_elems)`` for a contiguous [L, E, x, y] bank."""
    L, E, x, y = bank.shape
    base = bank.data_ptr()
    w_ptr = torch.tensor([[base + e * x * y * 2 for e in range(E)]], dtype=torch.int64)
    return w_ptr, E * x * y


def scattered_bank(bank: torch.Tensor, seed: int, pad: int = 40):
    """Copy ``bank`` [L, E, x, y] into a flat buffer where expert blocks are
    shuffled and each adapter slab is padded by ``pad`` elements.  Returns
    ``(flat, w_ptr [1, E], stride)``; the flat tensor lives on bank's device."""
    L, E, x, y = bank.shape
    blk = x * y
    stride = E * blk + pad
    pos = np.random.default_rng(seed).permutation(E)
    flat = torch.full((L * stride + pad,), float("nan"), dtype=bank.dtype, device=bank.device)
    for l in range(L):
        for e in range(E):
            off = l * stride + int(pos[e]) * blk
            flat[off:off + blk] = bank[l, e].reshape(-1)
    base = flat.data_ptr()
    w_ptr = torch.tensor([[base + int(pos[e]) * blk * 2 for e in range(E)]], dtype=torch.int64)
    return flat, w_ptr, stride


ORACLE_DTYPE = {torch.bfloat16: "bf16", torch.float16: "f16"}


def oracle_bank(t: torch.Tensor) -> Bank:
    return Bank(bits16(t.reshape(-1)), t.data_ptr(), ORACLE_DTYPE[t.dtype])
