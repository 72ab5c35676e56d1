"""MI355X-native routed-MoE hot path: ragged grouped GEMM, FC2 LoRA delta
(and the MoE finalize with that delta added), NVFP4 GEMM with a LoRA
epilogue and the prepared-path fold.

All work runs in ``libmi_moe.so`` (HIP, gfx950); this package only marshals
torch tensors into its C ABI.
"""
from .api import *  # noqa: F401,F403
from .api import __all__  # noqa: F401
