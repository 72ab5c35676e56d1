"""ctypes loader for ``libmi_moe.so``; raises if the library is missing.

There is no fallback: every operation of this package runs in the HIP
library.  Build it with ``python -m moe_expert_grouped_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmi_moe.so")

MI_OK, MI_EINVAL, MI_EUNSUPPORTED, MI_EHIP = 0, 1, 2, 3
MI_BF16, MI_F16, MI_F32 = 0, 1, 2

EXPORTS = [
    "mi_last_error",
    "mi_abi_version",
    "mi_grouped_mm_bf16",
    "mi_grouped_mm_swiglu",
    "mi_moe_fc2_lora_delta_workspace_size",
    "mi_moe_fc2_lora_delta",
    "mi_moe_fc2_lora_delta_noalloc",
    "mi_moe_fc2_finalize_lora",
    "mi_moe_fc1_lora_delta_workspace_size",
    "mi_moe_fc1_lora_delta",
    "mi_moe_fc2_finalize_workspace_size",
    "mi_moe_route_workspace_size",
    "mi_moe_route_permutation",
    "mi_moe_permute_rows",
    "mi_mm_nvfp4_lora",
    "mi_grouped_mm_nvfp4",
    "mi_prepare_lora_fold",
    "mi_nvfp4_dequant_bf16",
    "mi_fp4_quantize",
]

_lib = None

P = ctypes.c_void_p
I64 = ctypes.c_int64
SZ = ctypes.c_size_t
I32 = ctypes.c_int
F32 = ctypes.c_float


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m moe_expert_grouped_amd.build); there is no CPU fallback")
        L = ctypes.CDLL(LIB_PATH)
        L.mi_last_error.restype = ctypes.c_char_p
        L.mi_last_error.argtypes = []
        L.mi_abi_version.restype = I32
        L.mi_abi_version.argtypes = []
        L.mi_grouped_mm_bf16.restype = I32
        L.mi_grouped_mm_bf16.argtypes = [P, I64, I64, I32, P, I64, I64, P, P, I32, P]
        L.mi_grouped_mm_swiglu.restype = I32
        L.mi_grouped_mm_swiglu.argtypes = [P, I64, I64, I32, P, I64, I64, P, P, P, P, P, P, I32, P]
        L.mi_moe_fc2_lora_delta_workspace_size.restype = SZ
        L.mi_moe_fc2_lora_delta_workspace_size.argtypes = [I64, I64, I64, I64, I64]
        L.mi_moe_fc2_lora_delta.restype = I32
        L.mi_moe_fc2_lora_delta.argtypes = [
            P, I64, I64,          # act, padded_rows, inter_size
            P,                    # expanded_idx_to_permuted_idx
            P, I64, P, I64,       # w_ptr_a, stride_a, w_ptr_b, stride_b
            P, P, P,              # topk_ids, topk_weights, lora_ids
            I64, I64, I64, I64, I64, I64,  # T, top_k, E, L, rank, H
            I32, F32, I32,        # lora_dtype, scale, out_dtype
            P, P, SZ, P]          # out, workspace, bytes, stream
        L.mi_moe_fc2_lora_delta_noalloc.restype = I32
        L.mi_moe_fc2_lora_delta_noalloc.argtypes = [
            P, I64, I64, P, P, I64, P, I64, P, P, P,
            I64, I64, I64, I64, I64, I64, I32, F32, I32, P, P]
        L.mi_moe_fc2_finalize_workspace_size.restype = SZ
        L.mi_moe_fc2_finalize_workspace_size.argtypes = [I64, I64, I64, I64, I64, I64]
        L.mi_moe_fc2_finalize_lora.restype = I32
        L.mi_moe_fc2_finalize_lora.argtypes = [
            P, I32,               # fc2, fc2_dtype
            *L.mi_moe_fc2_lora_delta.argtypes]
        L.mi_moe_fc1_lora_delta_workspace_size.restype = SZ
        L.mi_moe_fc1_lora_delta_workspace_size.argtypes = [I64, I64, I64, I64, I64]
        L.mi_moe_fc1_lora_delta.restype = I32
        L.mi_moe_fc1_lora_delta.argtypes = [
            P, I64, I64,          # act, padded_rows, hidden_size
            P,                    # expanded_idx_to_permuted_idx
            P, I64, P, I64,       # w_ptr_a, stride_a, w_ptr_b, stride_b
            P, P,                 # topk_ids, lora_ids
            I64, I64, I64, I64, I64, I64,  # T, top_k, E, L, rank, out_features
            I32, F32, I32,        # lora_dtype, scale, out_dtype
            P, P, SZ, P]          # out, workspace, bytes, stream
        L.mi_moe_route_workspace_size.restype = SZ
        L.mi_moe_route_workspace_size.argtypes = [I64, I64]
        L.mi_moe_route_permutation.restype = I32
        L.mi_moe_route_permutation.argtypes = [P, I64, I64, I64, P, P, P, P, SZ, P]
        L.mi_moe_permute_rows.restype = I32
        L.mi_moe_permute_rows.argtypes = [P, I64, I64, P, I64, P, I64, P]
        L.mi_mm_nvfp4_lora.restype = I32
        L.mi_mm_nvfp4_lora.argtypes = [P, P, P, SZ, P, SZ, P, I64, I64, I64, P, I64, P, P, P, P,
                                       P, P, P]
        L.mi_grouped_mm_nvfp4.restype = I32
        L.mi_grouped_mm_nvfp4.argtypes = [P, P, SZ, I64, I64, P, P, SZ, I64, I64, P, P, P, I32, P]
        L.mi_prepare_lora_fold.restype = I32
        L.mi_prepare_lora_fold.argtypes = [P, I64, I64, P, P, P, P, P]
        L.mi_nvfp4_dequant_bf16.restype = I32
        L.mi_nvfp4_dequant_bf16.argtypes = [P, P, SZ, I64, I64, P, P]
        L.mi_fp4_quantize.restype = I32
        L.mi_fp4_quantize.argtypes = [P, I64, I64, I64, I32, P, P, P, SZ, P]
        _lib = L
    return _lib


class MiError(RuntimeError):
    pass


def check(status: int) -> None:
    if status == MI_OK:
        return
    msg = lib().mi_last_error().decode()
    if status == MI_EINVAL:
        raise ValueError(msg)
    if status == MI_EUNSUPPORTED:
        raise NotImplementedError(msg)
    raise MiError(msg)
