"""Seeded synthetic inputs for the routed-MoE grouped GEMM, the FC2 LoRA delta
and the NVFP4 + LoRA GEMM.

This module is shared by the GPU path's tests/bench and by the CPU oracle's
tests.  It draws random tensors and builds the routing bookkeeping a caller
would hand to the library (expert ids, the permutation, ``m_indptr``).  It
holds none of the operations' arithmetic: no GEMM, no dequantisation, no
scale-factor layout, no rounding recipe of the fold.
"""
from .inputs import *  # noqa: F401,F403
