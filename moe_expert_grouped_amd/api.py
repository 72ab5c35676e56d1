"""Torch-tensor front end of ``libmi_moe`` (argument marshalling only).

The functions mirror the pages' Python signatures:

- :func:`grouped_mm_bf16`            -- flashinfer.grouped_mm.grouped_mm_bf16
- :func:`bgmv_moe_gemm2_lora_delta`  -- flashinfer.fused_moe.bgmv_moe_gemm2_lora_delta
- :func:`mm_nvfp4_lora`              -- flashinfer.gemm.mm_nvfp4_lora
- :func:`prepare_nvfp4_lora_adapter` -- flashinfer.gemm.prepare_nvfp4_lora_adapter

Every computation happens in the HIP library; tensors only provide device
memory and the current stream.  Inputs must already live on the GPU.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib
from ._lib import MI_BF16, MI_F16, MI_F32, check

__all__ = [
    "grouped_mm_bf16",
    "grouped_mm_swiglu",
    "bgmv_moe_gemm2_lora_delta",
    "moe_finalize_lora",
    "moe_fc1_lora_delta",
    "moe_route_permutation",
    "moe_permute_rows",
    "route_workspace_bytes",
    "delta_workspace_bytes",
    "finalize_workspace_bytes",
    "fill_w_ptr",
    "mm_nvfp4_lora",
    "grouped_mm_nvfp4",
    "prepare_nvfp4_lora_adapter",
    "PreparedNvFp4LoraAdapter",
    "StaleAdapterError",
    "nvfp4_dequant",
    "fp4_quantize",
    "sf_bytes_needed",
]

_DT = {torch.bfloat16: MI_BF16, torch.float16: MI_F16, torch.float32: MI_F32}


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(dev: torch.device):
    return torch.cuda.current_stream(dev).cuda_stream


def _need_cuda(name, *tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name}: all tensors must be on the GPU")


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


# ---------------------------------------------------------------------------
# grouped GEMM
# ---------------------------------------------------------------------------

def grouped_mm_bf16(a: torch.Tensor, b: torch.Tensor, m_indptr: torch.Tensor,
                    out: torch.Tensor | None = None, out_dtype: torch.dtype = torch.bfloat16, *,
                    backend: str = "auto", tactic: int = -1) -> torch.Tensor:
    """``out[m_indptr[e]:m_indptr[e+1]] = a[...] @ b[e]^T`` for every expert.

    ``a`` bf16 ``(cum_m, k)``, ``b`` bf16 ``(batch, n, k)``, ``m_indptr`` int32
    ``(batch+1,)`` read on the device.  Rows outside
    ``[m_indptr[0], m_indptr[-1])`` of a caller-provided ``out`` are untouched
    (a fresh ``out`` is zero-filled there).  ``backend`` is accepted for
    signature compatibility; there is one program and ``tactic`` must be -1.
    """
    _need(tactic == -1, "grouped_mm_bf16: tactic must be -1 (single program)")
    _need(a.dtype in (torch.bfloat16, torch.float16) and b.dtype == a.dtype,
          "grouped_mm_bf16: a and b must both be bfloat16 or both float16")
    _need(a.dim() == 2 and b.dim() == 3 and b.shape[2] == a.shape[1],
          "grouped_mm_bf16: a must be (cum_m, k) and b (batch_size, n, k)")
    _need(m_indptr.dtype == torch.int32 and m_indptr.shape == (b.shape[0] + 1,),
          "grouped_mm_bf16: m_indptr must be int32 of shape (batch_size + 1,)")
    _need(out_dtype in (torch.bfloat16, torch.float32, torch.float16),
          "grouped_mm_bf16: out_dtype must be bfloat16, float16 or float32")
    _need_cuda("grouped_mm_bf16", a, b, m_indptr, out)
    a, b, m_indptr = a.contiguous(), b.contiguous(), m_indptr.contiguous()
    if out is None:
        out = torch.zeros((a.shape[0], b.shape[1]), dtype=out_dtype, device=a.device)
    _need(out.shape == (a.shape[0], b.shape[1]) and out.dtype == out_dtype and out.is_contiguous(),
          "grouped_mm_bf16: out must be a contiguous (cum_m, n) tensor of out_dtype")
    check(_lib.lib().mi_grouped_mm_bf16(_ptr(a), a.shape[0], a.shape[1], _DT[a.dtype], _ptr(b),
                                        b.shape[0], b.shape[1], _ptr(m_indptr), _ptr(out),
                                        _DT[out_dtype], _stream(a.device)))
    return out


# ---------------------------------------------------------------------------
# FC2 LoRA delta
# ---------------------------------------------------------------------------

def grouped_mm_swiglu(a: torch.Tensor, b: torch.Tensor, m_indptr: torch.Tensor, *,
                      fc1_delta: torch.Tensor | None = None,
                      gemm1_alpha: torch.Tensor | None = None,
                      gemm1_beta: torch.Tensor | None = None,
                      gemm1_clamp_limit: torch.Tensor | None = None,
                      out: torch.Tensor | None = None,
                      out_dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """FC1 of a routed MoE: ``h = a @ b[e]^T (+ fc1_delta)`` per expert's rows,
    then ``out = g * sigmoid(alpha*g) * (u + beta)`` with ``g`` the clamped gate
    half and ``u`` the clamped up half of ``h`` (plain SwiGLU by default).

    ``a`` bf16/fp16 ``(cum_m, k)``, ``b`` ``(batch, 2I, k)`` (gate rows, then
    up rows), ``fc1_delta`` bf16 ``(cum_m, 2I)``, ``gemm1_*`` fp32 ``(batch,)``.
    Returns ``(cum_m, I)``; rows outside the groups of a caller-provided ``out``
    are untouched (a fresh ``out`` is zero-filled there).
    """
    _need(a.dtype in (torch.bfloat16, torch.float16) and b.dtype == a.dtype,
          "grouped_mm_swiglu: a and b must both be bfloat16 or both float16")
    _need(a.dim() == 2 and b.dim() == 3 and b.shape[2] == a.shape[1] and b.shape[1] % 2 == 0,
          "grouped_mm_swiglu: a must be (cum_m, k) and b (batch_size, 2*I, k)")
    _need(m_indptr.dtype == torch.int32 and m_indptr.shape == (b.shape[0] + 1,),
          "grouped_mm_swiglu: m_indptr must be int32 of shape (batch_size + 1,)")
    _need(out_dtype in (torch.bfloat16, torch.float32, torch.float16),
          "grouped_mm_swiglu: out_dtype must be bfloat16, float16 or float32")
    E, two_i = b.shape[0], b.shape[1]
    for name, t in (("gemm1_alpha", gemm1_alpha), ("gemm1_beta", gemm1_beta),
                    ("gemm1_clamp_limit", gemm1_clamp_limit)):
        _need(t is None or (t.dtype == torch.float32 and t.numel() == E),
              f"grouped_mm_swiglu: {name} must be float32 with one value per expert")
    _need(fc1_delta is None or (fc1_delta.dtype == torch.bfloat16 and
                                fc1_delta.shape == (a.shape[0], two_i)),
          "grouped_mm_swiglu: fc1_delta must be bfloat16 (cum_m, 2*I)")
    _need_cuda("grouped_mm_swiglu", a, b, m_indptr, fc1_delta, gemm1_alpha, gemm1_beta,
               gemm1_clamp_limit, out)
    a, b, m_indptr = a.contiguous(), b.contiguous(), m_indptr.contiguous()
    opt = [None if t is None else t.contiguous()
           for t in (fc1_delta, gemm1_alpha, gemm1_beta, gemm1_clamp_limit)]
    if out is None:
        out = torch.zeros((a.shape[0], two_i // 2), dtype=out_dtype, device=a.device)
    _need(out.shape == (a.shape[0], two_i // 2) and out.dtype == out_dtype and
          out.is_contiguous(),
          "grouped_mm_swiglu: out must be a contiguous (cum_m, I) tensor of out_dtype")
    check(_lib.lib().mi_grouped_mm_swiglu(
        _ptr(a), a.shape[0], a.shape[1], _DT[a.dtype], _ptr(b), E, two_i // 2, _ptr(m_indptr),
        *(_ptr(t) for t in opt), _ptr(out), _DT[out_dtype], _stream(a.device)))
    return out


def fill_w_ptr(bank: torch.Tensor) -> torch.Tensor:
    """Base-pointer table ``[1, E]`` (int64 byte addresses) of a contiguous
    ``[L, E, x, y]`` LoRA bank: entry e addresses adapter 0's ``[x, y]`` block
    of expert e; adapter l is ``lora_stride = E*x*y`` elements further."""
    _need(bank.dim() == 4 and bank.is_contiguous(), "fill_w_ptr: bank must be contiguous [L, E, x, y]")
    L, E, x, y = bank.shape
    step = x * y * bank.element_size()
    return (bank.data_ptr() + torch.arange(E, dtype=torch.int64) * step).reshape(1, E).to(
        bank.device)


def delta_workspace_bytes(num_tokens, top_k, num_experts, num_adapters, rank) -> int:
    return int(_lib.lib().mi_moe_fc2_lora_delta_workspace_size(num_tokens, top_k, num_experts,
                                                               num_adapters, rank))


def finalize_workspace_bytes(num_tokens, top_k, num_experts, num_adapters, rank,
                             hidden_size) -> int:
    """Workspace of the two-pass finalize (the delta's plus an fp32 [T, H] delta)."""
    return int(_lib.lib().mi_moe_fc2_finalize_workspace_size(num_tokens, top_k, num_experts,
                                                             num_adapters, rank, hidden_size))


def bgmv_moe_gemm2_lora_delta(gemm1_activation_output: torch.Tensor,
                              expanded_idx_to_permuted_idx: torch.Tensor, w_ptr_a: torch.Tensor,
                              lora_stride_a: int, w_ptr_b: torch.Tensor, lora_stride_b: int,
                              topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                              lora_ids: torch.Tensor, rank: int, hidden_size: int, *,
                              num_adapters: int, lora_dtype: torch.dtype = torch.bfloat16,
                              scale: float = 1.0, out_dtype: torch.dtype = torch.bfloat16,
                              out: torch.Tensor | None = None,
                              workspace: torch.Tensor | None = None) -> torch.Tensor:
    """FC2 LoRA delta ``[T, H]`` to be added to the MoE output.

    ``num_adapters`` is the number of adapters in the banks (ids at or above
    it are treated as no adapter); the other arguments follow the page.
    """
    return _delta_call(None, gemm1_activation_output, expanded_idx_to_permuted_idx, w_ptr_a,
                       lora_stride_a, w_ptr_b, lora_stride_b, topk_ids, topk_weights, lora_ids,
                       rank, hidden_size, num_adapters, lora_dtype, scale, out_dtype, out,
                       workspace)


def moe_finalize_lora(fc2_out: torch.Tensor, gemm1_activation_output: torch.Tensor,
                      expanded_idx_to_permuted_idx: torch.Tensor, w_ptr_a: torch.Tensor,
                      lora_stride_a: int, w_ptr_b: torch.Tensor, lora_stride_b: int,
                      topk_ids: torch.Tensor, topk_weights: torch.Tensor, lora_ids: torch.Tensor,
                      rank: int, hidden_size: int, *, num_adapters: int,
                      lora_dtype: torch.dtype = torch.bfloat16, scale: float = 1.0,
                      out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None) -> torch.Tensor:
    """MoE output ``[T, H]``: the routing-weighted combine of the FC2 rows
    (``fc2_out``, permuted ``[padded_rows, H]`` in bf16, fp16 or fp32) with
    the FC2 LoRA delta added, in one pass and one rounding.  The other
    arguments are those of :func:`bgmv_moe_gemm2_lora_delta`."""
    _need(isinstance(fc2_out, torch.Tensor) and fc2_out.dim() == 2 and
          fc2_out.shape[1] == hidden_size and
          fc2_out.shape[0] == gemm1_activation_output.shape[0],
          "moe_finalize_lora: fc2_out must be [padded_rows, hidden_size]")
    _need(fc2_out.dtype in _DT, "moe_finalize_lora: fc2_out must be bf16, fp16 or fp32")
    return _delta_call(fc2_out, gemm1_activation_output, expanded_idx_to_permuted_idx, w_ptr_a,
                       lora_stride_a, w_ptr_b, lora_stride_b, topk_ids, topk_weights, lora_ids,
                       rank, hidden_size, num_adapters, lora_dtype, scale, out_dtype, out,
                       workspace)


def _delta_call(fc2, act, perm, w_ptr_a, lora_stride_a, w_ptr_b, lora_stride_b, topk_ids,
                topk_weights, lora_ids, rank, hidden_size, num_adapters, lora_dtype, scale,
                out_dtype, out, workspace):
    _need(act.dim() == 2, "bgmv_moe_gemm2_lora_delta: activation must be [padded_rows, I]")
    _need(topk_ids.dim() == 2 and topk_weights.shape == topk_ids.shape,
          "bgmv_moe_gemm2_lora_delta: topk_ids / topk_weights must be [T, top_k]")
    T, top_k = topk_ids.shape
    _need(perm.numel() == T * top_k and perm.dtype == torch.int32,
          "bgmv_moe_gemm2_lora_delta: expanded_idx_to_permuted_idx must be int32 [T*top_k]")
    _need(topk_ids.dtype == torch.int32 and lora_ids.dtype == torch.int32 and
          topk_weights.dtype == torch.float32,
          "bgmv_moe_gemm2_lora_delta: ids must be int32 and topk_weights float32")
    _need(lora_ids.numel() == T, "bgmv_moe_gemm2_lora_delta: lora_ids must be [T]")
    _need(w_ptr_a.dtype == torch.int64 and w_ptr_b.dtype == torch.int64 and
          w_ptr_a.numel() == w_ptr_b.numel(),
          "bgmv_moe_gemm2_lora_delta: w_ptr_a / w_ptr_b must be int64 [1, num_experts]")
    _need(act.dtype == lora_dtype, "bgmv_moe_gemm2_lora_delta: activation dtype must be lora_dtype")
    _need(lora_dtype in _DT and out_dtype in _DT, "bgmv_moe_gemm2_lora_delta: unsupported dtype")
    _need_cuda("bgmv_moe_gemm2_lora_delta", act, perm, w_ptr_a, w_ptr_b, topk_ids, topk_weights,
               lora_ids, out, workspace, fc2)
    E = w_ptr_a.numel()
    act = act.contiguous()
    perm, topk_ids, topk_weights, lora_ids = (x.contiguous() for x in
                                             (perm, topk_ids, topk_weights, lora_ids))
    w_ptr_a, w_ptr_b = w_ptr_a.contiguous(), w_ptr_b.contiguous()
    if out is None:
        out = torch.empty((T, hidden_size), dtype=out_dtype, device=act.device)
    _need(out.shape == (T, hidden_size) and out.dtype == out_dtype and out.is_contiguous(),
          "bgmv_moe_gemm2_lora_delta: out must be a contiguous [T, H] tensor of out_dtype")
    need = delta_workspace_bytes(T, top_k, E, num_adapters, rank) if fc2 is None else \
        finalize_workspace_bytes(T, top_k, E, num_adapters, rank, hidden_size)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=act.device)
    args = (_ptr(act), act.shape[0], act.shape[1], _ptr(perm), _ptr(w_ptr_a), int(lora_stride_a),
            _ptr(w_ptr_b), int(lora_stride_b), _ptr(topk_ids), _ptr(topk_weights), _ptr(lora_ids),
            T, top_k, E, int(num_adapters), int(rank), int(hidden_size), _DT[lora_dtype],
            float(scale), _DT[out_dtype], _ptr(out), _ptr(workspace), workspace.numel(),
            _stream(act.device))
    if fc2 is None:
        check(_lib.lib().mi_moe_fc2_lora_delta(*args))
    else:
        fc2 = fc2.contiguous()
        check(_lib.lib().mi_moe_fc2_finalize_lora(_ptr(fc2), _DT[fc2.dtype], *args))
    return out


def moe_fc1_lora_delta(act: torch.Tensor, expanded_idx_to_permuted_idx: torch.Tensor,
                       w_ptr_a: torch.Tensor, lora_stride_a: int, w_ptr_b: torch.Tensor,
                       lora_stride_b: int, topk_ids: torch.Tensor, lora_ids: torch.Tensor,
                       rank: int, out_features: int, *, num_adapters: int,
                       lora_dtype: torch.dtype = torch.bfloat16, scale: float = 1.0,
                       out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None) -> torch.Tensor:
    """FC1 (gate/up) LoRA delta ``[padded_rows, out_features]``: row
    ``perm[t*top_k+j]`` is ``scale * B[l, e] @ (A[l, e] @ act[row])`` for
    each routed slot, +0 for a slot without adapter; the ``fc1_delta`` of
    :func:`grouped_mm_swiglu`.  A fresh ``out`` is zero-filled first, so rows
    no slot points at are 0; a caller's ``out`` keeps them."""
    _need(act.dim() == 2 and act.dtype == lora_dtype,
          "moe_fc1_lora_delta: act must be [padded_rows, hidden] of lora_dtype")
    _need(topk_ids.dim() == 2 and topk_ids.dtype == torch.int32 and lora_ids.dtype == torch.int32,
          "moe_fc1_lora_delta: topk_ids must be int32 [T, top_k] and lora_ids int32 [T]")
    T, top_k = topk_ids.shape
    perm = expanded_idx_to_permuted_idx
    _need(perm.numel() == T * top_k and perm.dtype == torch.int32 and lora_ids.numel() == T,
          "moe_fc1_lora_delta: expanded_idx_to_permuted_idx must be int32 [T*top_k]")
    _need(w_ptr_a.dtype == torch.int64 and w_ptr_b.dtype == torch.int64 and
          w_ptr_a.numel() == w_ptr_b.numel(),
          "moe_fc1_lora_delta: w_ptr_a / w_ptr_b must be int64 [1, num_experts]")
    _need(lora_dtype in (torch.bfloat16, torch.float16) and out_dtype in _DT,
          "moe_fc1_lora_delta: unsupported dtype")
    _need_cuda("moe_fc1_lora_delta", act, perm, w_ptr_a, w_ptr_b, topk_ids, lora_ids, out,
               workspace)
    E = w_ptr_a.numel()
    act = act.contiguous()
    perm, topk_ids, lora_ids = perm.contiguous(), topk_ids.contiguous(), lora_ids.contiguous()
    if out is None:
        out = torch.zeros((act.shape[0], out_features), dtype=out_dtype, device=act.device)
    _need(out.shape == (act.shape[0], out_features) and out.dtype == out_dtype and
          out.is_contiguous(), "moe_fc1_lora_delta: out must be a contiguous "
          "[padded_rows, out_features] tensor of out_dtype")
    need = int(_lib.lib().mi_moe_fc1_lora_delta_workspace_size(T, top_k, E, num_adapters, rank))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=act.device)
    check(_lib.lib().mi_moe_fc1_lora_delta(
        _ptr(act), act.shape[0], act.shape[1], _ptr(perm), _ptr(w_ptr_a.contiguous()),
        int(lora_stride_a), _ptr(w_ptr_b.contiguous()), int(lora_stride_b), _ptr(topk_ids),
        _ptr(lora_ids), T, top_k, E, int(num_adapters), int(rank), int(out_features),
        _DT[lora_dtype], float(scale), _DT[out_dtype], _ptr(out), _ptr(workspace),
        workspace.numel(), _stream(act.device)))
    return out


# ---------------------------------------------------------------------------
# routing output -> permutation, permuted rows
# ---------------------------------------------------------------------------

def route_workspace_bytes(num_slots: int, num_experts: int) -> int:
    return int(_lib.lib().mi_moe_route_workspace_size(num_slots, num_experts))


def moe_route_permutation(topk_ids: torch.Tensor, num_experts: int, *,
                          with_inverse: bool = False, workspace: torch.Tensor | None = None):
    """``(m_indptr, expanded_idx_to_permuted_idx[, permuted_idx_to_expanded_idx])``
    from ``topk_ids`` int32 ``[T, top_k]``: the slots sorted stably by expert
    id, ids outside ``[0, num_experts)`` left out (entry -1).  All int32 on
    the device; ``m_indptr`` is ``[num_experts + 1]``."""
    _need(topk_ids.dim() == 2 and topk_ids.dtype == torch.int32,
          "moe_route_permutation: topk_ids must be int32 [num_tokens, top_k]")
    _need_cuda("moe_route_permutation", topk_ids, workspace)
    T, top_k = topk_ids.shape
    dev = topk_ids.device
    topk_ids = topk_ids.contiguous()
    m_indptr = torch.empty(int(num_experts) + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * top_k, dtype=torch.int32, device=dev)
    inverse = torch.empty(T * top_k, dtype=torch.int32, device=dev) if with_inverse else None
    need = route_workspace_bytes(T * top_k, num_experts)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    check(_lib.lib().mi_moe_route_permutation(
        _ptr(topk_ids), T, top_k, int(num_experts), _ptr(m_indptr), _ptr(perm), _ptr(inverse),
        _ptr(workspace), workspace.numel(), _stream(dev)))
    return (m_indptr, perm, inverse) if with_inverse else (m_indptr, perm)


def moe_permute_rows(x: torch.Tensor, expanded_idx_to_permuted_idx: torch.Tensor, top_k: int,
                     out_rows: int | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """``out[perm[t*top_k + j]] = x[t]`` for every slot whose row lies in
    ``[0, out_rows)`` (other rows of ``out`` untouched; a fresh ``out`` is
    zero-filled).  ``x`` ``[T, ...]`` of any dtype, rows of a multiple of 16 bytes."""
    _need(x.dim() >= 1, "moe_permute_rows: x must be [num_tokens, ...]")
    perm = expanded_idx_to_permuted_idx
    _need(perm.dtype == torch.int32 and perm.numel() == x.shape[0] * int(top_k),
          "moe_permute_rows: expanded_idx_to_permuted_idx must be int32 [num_tokens*top_k]")
    _need_cuda("moe_permute_rows", x, perm, out)
    x, perm = x.contiguous(), perm.contiguous()
    if out is None:
        rows = perm.numel() if out_rows is None else int(out_rows)
        out = torch.zeros((rows,) + tuple(x.shape[1:]), dtype=x.dtype, device=x.device)
    _need(out.dtype == x.dtype and out.shape[1:] == x.shape[1:] and out.is_contiguous(),
          "moe_permute_rows: out must be contiguous [out_rows, ...] of x's dtype")
    row_bytes = x[0].numel() * x.element_size() if x.shape[0] else 16
    check(_lib.lib().mi_moe_permute_rows(_ptr(x), x.shape[0], row_bytes, _ptr(perm), int(top_k),
                                         _ptr(out), out.shape[0], _stream(x.device)))
    return out


# ---------------------------------------------------------------------------
# NVFP4 + LoRA
# ---------------------------------------------------------------------------

class StaleAdapterError(ValueError):
    """A prepared adapter's alpha or source tensors changed since the fold."""


def _pin(t: torch.Tensor):
    return (t.data_ptr(), t._version, tuple(t.shape), t.device, t.dtype)


class PreparedNvFp4LoraAdapter:
    """A folded LoRA-up weight ``b_folded = bf16(lora_b * lora_scale / alpha)``
    with its device zero-adapter flag and the snapshot pins of its sources."""

    def __init__(self, lora_b, lora_scale, alpha, b_folded, fold_flags):
        self.lora_b = lora_b
        self.lora_scale = lora_scale
        self.alpha = alpha
        self.b_folded = b_folded
        self.fold_flags = fold_flags
        self.refresh_pins()

    def refresh_pins(self):
        self._pins = (_pin(self.lora_b), _pin(self.lora_scale), _pin(self.alpha))

    def check_fresh(self, alpha):
        if alpha is not self.alpha:
            raise StaleAdapterError("mm_nvfp4_lora: the prepared adapter was folded for a different "
                                    "alpha tensor; re-prepare it for this call's alpha")
        if self._pins != (_pin(self.lora_b), _pin(self.lora_scale), _pin(self.alpha)):
            raise StaleAdapterError("mm_nvfp4_lora: lora_b, lora_scale or alpha changed since the "
                                    "adapter was prepared; re-prepare it")


def _fold(lora_b, lora_scale, alpha, b_folded, fold_flags):
    check(_lib.lib().mi_prepare_lora_fold(_ptr(lora_b), lora_b.shape[0], lora_b.shape[1],
                                          _ptr(lora_scale), _ptr(alpha), _ptr(b_folded),
                                          _ptr(fold_flags), _stream(lora_b.device)))


def prepare_nvfp4_lora_adapter(lora_b: torch.Tensor, lora_scale: torch.Tensor,
                               alpha: torch.Tensor, *,
                               out: PreparedNvFp4LoraAdapter | None = None
                               ) -> PreparedNvFp4LoraAdapter:
    """Fold one adapter for the prepared path.

    ``out=None``: lora_scale and alpha are read back to the host once; a zero
    alpha or a ratio that is not finite raises ValueError, otherwise the fold
    kernel runs.  ``out=adapter``: in-place refold with no host read; the
    alpha tensor has to be the one the adapter was prepared with, and lora_b
    keeps its shape and device.
    """
    _need(lora_b.dtype == torch.bfloat16 and lora_b.dim() == 2 and lora_b.is_contiguous(),
          "prepare_nvfp4_lora_adapter: lora_b must be contiguous bf16 [N, r]")
    _need(lora_scale.dtype == torch.float32 and lora_scale.numel() == 1,
          "prepare_nvfp4_lora_adapter: lora_scale must be an fp32 tensor of shape (1,)")
    _need(alpha.dtype == torch.float32 and alpha.numel() >= 1,
          "prepare_nvfp4_lora_adapter: alpha must be an fp32 device tensor")
    _need_cuda("prepare_nvfp4_lora_adapter", lora_b, lora_scale, alpha)
    if out is None:
        host = torch.cat([lora_scale.reshape(1), alpha.reshape(-1)[:1]]).cpu().numpy()
        s, a = np.float32(host[0]), np.float32(host[1])
        _need(a != 0, "prepare_nvfp4_lora_adapter: alpha == 0 is refused (lora_scale / alpha is "
                      "undefined); use the raw path for an alpha == 0 LoRA-only call")
        with np.errstate(all="ignore"):
            _need(np.isfinite(np.float32(s / a)),
                  "prepare_nvfp4_lora_adapter: lora_scale / alpha is not finite")
        b_folded = torch.empty_like(lora_b)
        flags = torch.zeros(1, dtype=torch.int32, device=lora_b.device)
        _fold(lora_b, lora_scale, alpha, b_folded, flags)
        return PreparedNvFp4LoraAdapter(lora_b, lora_scale, alpha, b_folded, flags)
    _need(alpha is out.alpha, "prepare_nvfp4_lora_adapter: alpha must be the tensor the adapter was prepared with")
    _need(lora_b.shape == out.b_folded.shape and lora_b.device == out.b_folded.device,
          "prepare_nvfp4_lora_adapter: lora_b must keep out's [N, r] shape and device")
    _fold(lora_b, lora_scale, alpha, out.b_folded, out.fold_flags)
    out.lora_b, out.lora_scale = lora_b, lora_scale
    out.refresh_pins()
    return out


def sf_bytes_needed(rows: int, k: int) -> int:
    return (-(-rows // 128)) * (-(-(k // 16) // 4)) * 512


def mm_nvfp4_lora(a: torch.Tensor, b: torch.Tensor, a_sf: torch.Tensor, b_sf: torch.Tensor,
                  alpha: torch.Tensor, d: torch.Tensor | None = None,
                  lora_b: torch.Tensor | None = None, lora_scale: torch.Tensor | None = None, *,
                  lora_adapter: PreparedNvFp4LoraAdapter | None = None,
                  bias: torch.Tensor | None = None, out: torch.Tensor | None = None,
                  out_dtype: torch.dtype = torch.bfloat16, backend: str = "auto",
                  enable_pdl: bool | None = None) -> torch.Tensor:
    """NVFP4 base GEMM with a BF16 LoRA correction (raw or prepared path)."""
    _need(out_dtype == torch.bfloat16, "mm_nvfp4_lora: out_dtype must be torch.bfloat16")
    _need(a.dtype == torch.uint8 and b.dtype == torch.uint8 and a.dim() == 2 and b.dim() == 2,
          "mm_nvfp4_lora: a and b must be uint8 [M, K/2] and [N, K/2]")
    _need(a.shape[1] == b.shape[1], "mm_nvfp4_lora: a and b must have the same K")
    _need(a_sf.dtype == torch.uint8 and b_sf.dtype == torch.uint8,
          "mm_nvfp4_lora: a_sf / b_sf must be uint8")
    _need(alpha.dtype == torch.float32, "mm_nvfp4_lora: alpha must be an fp32 device tensor")
    raw_given = lora_b is not None or lora_scale is not None
    _need(not (lora_adapter is not None and raw_given),
          "mm_nvfp4_lora: pass either lora_b/lora_scale (raw path) or lora_adapter (prepared "
          "path), not both")
    _need_cuda("mm_nvfp4_lora", a, b, a_sf, b_sf, alpha, d, lora_b, lora_scale, bias, out)
    M, N, K = a.shape[0], b.shape[0], 2 * a.shape[1]
    a, b = a.contiguous(), b.contiguous()
    _need(a_sf.is_contiguous() and b_sf.is_contiguous(), "mm_nvfp4_lora: scale buffers must be "
          "contiguous")
    rank = 0
    d_ptr = lb_ptr = ls_ptr = bf_ptr = ff_ptr = None
    if lora_adapter is not None:
        _need(d is not None, "mm_nvfp4_lora: the prepared path requires d")
        lora_adapter.check_fresh(alpha)
        d_ptr, bf_ptr, ff_ptr = _ptr(d), _ptr(lora_adapter.b_folded), _ptr(lora_adapter.fold_flags)
        _need(lora_adapter.b_folded.shape == (N, d.shape[1]),
              "mm_nvfp4_lora: prepared adapter must be [N, r] with r = d.shape[1]")
        rank = d.shape[1]
    elif lora_scale is not None:
        _need(d is not None and lora_b is not None,
              "mm_nvfp4_lora: lora_scale needs d and lora_b (raw path)")
        _need(lora_scale.dtype == torch.float32 and lora_scale.numel() == 1,
              "mm_nvfp4_lora: lora_scale must be a one-element fp32 device tensor")
        _need(lora_b.dtype == torch.bfloat16 and lora_b.is_contiguous() and
              lora_b.shape == (N, d.shape[1]),
              "mm_nvfp4_lora: lora_b must be contiguous bf16 [N, r] (transpose a [r, N] factor)")
        d_ptr, lb_ptr, ls_ptr = _ptr(d), _ptr(lora_b), _ptr(lora_scale)
        rank = d.shape[1]
    if d_ptr is not None:
        _need(d.dtype == torch.bfloat16 and d.is_contiguous() and d.shape[0] == M,
              "mm_nvfp4_lora: d must be contiguous bf16 [M, r]")
    if bias is not None:
        _need(bias.dtype == torch.bfloat16 and bias.numel() == N and bias.is_contiguous(),
              "mm_nvfp4_lora: bias must be contiguous bf16 [N]")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _need(out.shape == (M, N) and out.dtype == torch.bfloat16 and out.is_contiguous(),
          "mm_nvfp4_lora: out must be a contiguous bf16 [M, N] tensor")
    check(_lib.lib().mi_mm_nvfp4_lora(_ptr(a), _ptr(b), _ptr(a_sf), a_sf.numel(), _ptr(b_sf),
                                      b_sf.numel(), _ptr(alpha), M, N, K, d_ptr, rank, lb_ptr,
                                      ls_ptr, bf_ptr, ff_ptr, _ptr(bias), _ptr(out),
                                      _stream(a.device)))
    return out


def grouped_mm_nvfp4(a: torch.Tensor, a_sf: torch.Tensor, b: torch.Tensor, b_sf: torch.Tensor,
                     m_indptr: torch.Tensor, alpha: torch.Tensor,
                     out: torch.Tensor | None = None,
                     out_dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """``out[m_indptr[e]:m_indptr[e+1]] = alpha[e] * dequant(a[...]) @ dequant(b[e])^T``.

    ``a`` uint8 ``(cum_m, k/2)`` with its 128x4 scales ``a_sf`` over all
    rows; ``b`` uint8 ``(batch, n, k/2)`` with ``b_sf`` holding one 128x4
    scale buffer per expert; ``alpha`` fp32 ``(batch,)``; ``m_indptr`` int32
    ``(batch+1,)`` read on the device.  Rows outside the groups of a
    caller-provided ``out`` are untouched (a fresh ``out`` is zero-filled there).
    """
    _need(a.dtype == torch.uint8 and b.dtype == torch.uint8 and a.dim() == 2 and b.dim() == 3
          and b.shape[2] == a.shape[1],
          "grouped_mm_nvfp4: a must be uint8 (cum_m, k/2) and b uint8 (batch_size, n, k/2)")
    _need(a_sf.dtype == torch.uint8 and b_sf.dtype == torch.uint8,
          "grouped_mm_nvfp4: scale buffers must be uint8")
    _need(m_indptr.dtype == torch.int32 and m_indptr.shape == (b.shape[0] + 1,),
          "grouped_mm_nvfp4: m_indptr must be int32 of shape (batch_size + 1,)")
    _need(alpha.dtype == torch.float32 and alpha.numel() == b.shape[0],
          "grouped_mm_nvfp4: alpha must be float32 with one value per expert")
    _need(out_dtype in (torch.bfloat16, torch.float32),
          "grouped_mm_nvfp4: out_dtype must be bfloat16 or float32")
    _need_cuda("grouped_mm_nvfp4", a, a_sf, b, b_sf, m_indptr, alpha, out)
    cum_m, k = a.shape[0], a.shape[1] * 2
    n = b.shape[1]
    a, b, a_sf, b_sf = a.contiguous(), b.contiguous(), a_sf.contiguous(), b_sf.contiguous()
    m_indptr, alpha = m_indptr.contiguous(), alpha.contiguous()
    if out is None:
        out = torch.zeros((cum_m, n), dtype=out_dtype, device=a.device)
    _need(out.shape == (cum_m, n) and out.dtype == out_dtype and out.is_contiguous(),
          "grouped_mm_nvfp4: out must be a contiguous (cum_m, n) tensor of out_dtype")
    check(_lib.lib().mi_grouped_mm_nvfp4(
        _ptr(a), _ptr(a_sf), a_sf.numel(), cum_m, k, _ptr(b), _ptr(b_sf), b_sf.numel(),
        b.shape[0], n, _ptr(m_indptr), _ptr(alpha), _ptr(out), _DT[out_dtype],
        _stream(a.device)))
    return out


def nvfp4_dequant(codes: torch.Tensor, sf: torch.Tensor, k: int | None = None) -> torch.Tensor:
    """bf16 ``[rows, K]`` dequantisation with the GEMM's own decoder."""
    _need(codes.dtype == torch.uint8 and codes.dim() == 2 and sf.dtype == torch.uint8,
          "nvfp4_dequant: codes [rows, K/2] and sf must be uint8")
    _need_cuda("nvfp4_dequant", codes, sf)
    k = 2 * codes.shape[1] if k is None else k
    out = torch.empty((codes.shape[0], k), dtype=torch.bfloat16, device=codes.device)
    check(_lib.lib().mi_nvfp4_dequant_bf16(_ptr(codes.contiguous()), _ptr(sf), sf.numel(),
                                           codes.shape[0], k, _ptr(out), _stream(codes.device)))
    return out


def fp4_quantize(x: torch.Tensor, global_scale: torch.Tensor, *, codes: torch.Tensor | None = None,
                 sf: torch.Tensor | None = None):
    """NVFP4 quantisation of ``x`` (bf16 / fp16 / fp32, ``[rows, K]`` or a batch
    ``[B, rows, K]`` of matrices) with fp32 global scale(s) ``global_scale``
    (one per matrix).  Returns ``(codes, sf)``: uint8 ``[..., rows, K/2]`` and
    the 128x4 scale buffer(s) (one per matrix, concatenated), the operands
    of :func:`mm_nvfp4_lora` / :func:`grouped_mm_nvfp4`."""
    _need(x.dtype in _DT and x.dim() in (2, 3), "fp4_quantize: x must be a bf16, fp16 or fp32 "
          "[rows, K] or [B, rows, K] tensor")
    _need_cuda("fp4_quantize", x, global_scale, codes, sf)
    batch = 1 if x.dim() == 2 else x.shape[0]
    rows, k = x.shape[-2], x.shape[-1]
    _need(global_scale.dtype == torch.float32 and global_scale.numel() == batch,
          "fp4_quantize: global_scale must be fp32 with one value per matrix")
    x = x.contiguous()
    per = (-(-rows // 128)) * (k // 64) * 512
    if codes is None:
        codes = torch.empty((*x.shape[:-1], k // 2), dtype=torch.uint8, device=x.device)
    if sf is None:
        sf = torch.empty(batch * per, dtype=torch.uint8, device=x.device)
    _need(codes.dtype == torch.uint8 and codes.shape == (*x.shape[:-1], k // 2) and
          codes.is_contiguous(), "fp4_quantize: codes must be contiguous uint8 [..., rows, K/2]")
    _need(sf.dtype == torch.uint8 and sf.is_contiguous(), "fp4_quantize: sf must be contiguous uint8")
    check(_lib.lib().mi_fp4_quantize(_ptr(x), batch, rows, k, _DT[x.dtype],
                                     _ptr(global_scale.contiguous()), _ptr(codes), _ptr(sf),
                                     sf.numel(), _stream(x.device)))
    return codes, sf
