"""The prepared-path fold of one LoRA adapter, step by step.

Follows ``flashinfer.gemm.prepare_nvfp4_lora_adapter`` (the description of
the fold kernel and of ``out=``):

    ratio       = div.rn.f32(fp32(lora_scale), fp32(alpha[0]))
    b_folded[i] = bf16_rne(fp32(lora_b[i]) * ratio)

i.e. an IEEE fp32 division rounded to nearest even, an IEEE fp32 product
(subnormals kept, no fast-math) and one round-to-nearest-even to bf16.  The
in-place refold is bitwise the same computation.  A zero ``lora_scale``
(either sign) folds to the zero adapter, recorded in a flag.

How each step is carried out here:
- the quotient is computed in float64 and rounded once to float32; for
  division this equals the correctly rounded float32 quotient because 53 >=
  2*24 + 2 (a double rounding of this kind is innocuous);
- the product of a bf16 (8 significant bits) and a float32 (24 bits) is exact
  in float64 and is rounded once to float32;
- the float32 is rounded once to bf16 by :func:`oracle.formats.f64_to_bf16_bits`.

``prepare_host_check`` is the host-side validation of the eager prepare
(alpha == 0 or a non-finite ratio is refused).
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64, f64_to_bf16_bits


def fold_ratio(lora_scale, alpha) -> np.float32:
    s = np.float64(np.float32(lora_scale))
    a = np.float64(np.float32(alpha))
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        return np.float32(s / a)


def fold(lora_b_bits, lora_scale, alpha):
    """Return ``(b_folded_bits uint16, zero_adapter bool)``."""
    ratio = fold_ratio(lora_scale, alpha)
    with np.errstate(invalid="ignore", over="ignore"):
        prod = (bf16_to_f64(lora_b_bits) * np.float64(ratio)).astype(np.float32)
    bits = f64_to_bf16_bits(prod.astype(np.float64))
    zero = bool(np.float32(lora_scale) == 0)
    return bits, zero


def prepare_host_check(lora_scale, alpha) -> None:
    """Raise ValueError when the eager prepare must refuse (alpha == 0 or a
    non-finite ratio)."""
    if np.float32(alpha) == 0:
        raise ValueError("alpha == 0: lora_scale / alpha is undefined")
    if not np.isfinite(fold_ratio(lora_scale, alpha)):
        raise ValueError("lora_scale / alpha is not finite")
