"""Plain fp64 CPU oracle for the routed-MoE hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (``moe_expert_grouped_amd``) never imports it and
fails loudly when its HIP library is missing; there is no CPU fallback.

The oracle shares no code with the HIP path.  Every function states the
passage of the source pages it follows (cited by page title and section):

- ``flashinfer.grouped_mm.grouped_mm_bf16`` -- formula and parameters
  -> :mod:`oracle.grouped_mm`
- ``flashinfer.fused_moe.bgmv_moe_gemm2_lora_delta`` -- formula and
  parameters -> :mod:`oracle.lora_delta`
- ``flashinfer.gemm.mm_nvfp4_lora`` -- formula, raw path, prepared path,
  parameters -> :mod:`oracle.nvfp4`
- ``flashinfer.gemm.prepare_nvfp4_lora_adapter`` -- the fold recipe
  -> :mod:`oracle.fold`
- MoE finalize with the delta added (``bgmv_moe_gemm2_lora_delta``,
  description and return value) -> :mod:`oracle.finalize`
- routing output -> expert-sorted permutation and permuted rows
  (``expanded_idx_to_permuted_idx`` and ``m_indptr`` parameters) ->
  :mod:`oracle.permute`
- NVFP4 grouped GEMM (``grouped_mm_bf16`` formula with the
  ``mm_nvfp4_lora`` operand format) -> :mod:`oracle.nvfp4_grouped`
- FC1 gate/up grouped GEMM with its SwiGLU activation
  (``prims_ts_fp4_block_scale_moe`` parameters) -> :mod:`oracle.fc1`
- NVFP4 quantisation, the producer of the operands ``mm_nvfp4_lora`` takes
  (the paragraph after its formula, and its ``alpha`` parameter)
  -> :mod:`oracle.fp4_quantize`
- FC1 (gate/up) LoRA delta, the ``gemm1_lora_delta`` the delta page's
  description names -> :mod:`oracle.fc1_lora_delta`

Inputs are numpy arrays; bf16 tensors are passed as their uint16 bit patterns.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests
(brute force, closed forms, library special cases, exact probes) except two
layout conventions the pages name without defining -- the nibble order of the
packed E2M1 codes and the 128x4 scale-factor tiling.  Those two are **parity
unpinned** by the pages: they follow the public OCP / block-scaling
convention and are pinned only to that convention (two independent codings
and hand-worked offsets).
"""
from . import formats, grouped_mm, lora_delta, nvfp4, fold, finalize, permute  # noqa: F401
from . import nvfp4_grouped, fc1, fp4_quantize, fc1_lora_delta  # noqa: F401
