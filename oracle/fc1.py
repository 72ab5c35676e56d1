"""FC1 of a routed MoE: the gate/up grouped GEMM and its SwiGLU activation.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows the FP4 fused-MoE page (``flashinfer.fused_moe.prims_ts_fp4_block_scale_moe``,
parameters ``gemm1_weights``, ``gemm1_alpha``, ``gemm1_beta``,
``gemm1_clamp_limit``, ``activation_type`` = SwiGLU by default) and the delta
page (``bgmv_moe_gemm2_lora_delta``: FC1 is run with ``gemm1_lora_delta`` set and
returns the permuted post-SwiGLU activation that FC2 consumes), with the
ragged grouped product of ``flashinfer.grouped_mm.grouped_mm_bf16`` (formula).

Readings (each listed with its reason in the design notes):
- ``b[e]`` is ``[2I, K]``: rows ``0..I-1`` are the gate projection, rows
  ``I..2I-1`` the up projection; ``h = a @ b[e]^T`` for the expert's rows;
- ``gemm1_lora_delta``, when given, is an additive ``[rows, 2I]`` term added
  to ``h`` before the activation;
- the activation, with per-expert ``alpha`` (default 1), ``beta`` (default 0)
  and clamp ``limit`` (default none):
      g = min(h_gate, limit),  u = clip(h_up, -limit, limit)
      out = g * sigmoid(alpha * g) * (u + beta)
  which is the plain SwiGLU ``silu(h_gate) * h_up`` at the defaults.  The
  page names the three parameters but not the formula; this one is read
  as the identity-preserving extension of SwiGLU;
- exact products in float64; the GPU forms ``h`` in fp32, applies the
  activation in fp32 and rounds once.  Rows outside the groups are not written.
"""
from __future__ import annotations

import numpy as np

from .formats import to_f64


def _sigmoid(z):
    # evaluated without overflow for either sign of z
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def swiglu(h_gate, h_up, alpha=1.0, beta=0.0, limit=None):
    """float64 activation of one expert's rows (scalars of that expert)."""
    g = np.asarray(h_gate, dtype=np.float64)
    u = np.asarray(h_up, dtype=np.float64)
    if limit is not None:
        g = np.minimum(g, limit)
        u = np.clip(u, -limit, limit)
    return g * _sigmoid(alpha * g) * (u + beta)


def grouped_mm_swiglu(a_bits, b_bits, m_indptr, dtype="bf16", delta_bits=None, alpha=None,
                      beta=None, limit=None):
    """Return ``(out, written)``: float64 ``[cum_m, I]`` and a bool row mask.

    ``a_bits`` ``[cum_m, K]``, ``b_bits`` ``[E, 2I, K]`` (uint16 patterns of
    ``dtype``), ``delta_bits`` bf16 patterns ``[cum_m, 2I]`` or None;
    ``alpha``/``beta``/``limit`` float32 ``[E]`` or None (defaults).
    """
    A = to_f64(a_bits, dtype)
    B = to_f64(b_bits, dtype)
    m_indptr = np.asarray(m_indptr, dtype=np.int64)
    E, two_i, _ = B.shape
    inter = two_i // 2
    D = None if delta_bits is None else to_f64(delta_bits, "bf16")
    f32 = lambda v: None if v is None else np.asarray(v, dtype=np.float32).astype(np.float64)
    alpha, beta, limit = f32(alpha), f32(beta), f32(limit)
    out = np.zeros((A.shape[0], inter), dtype=np.float64)
    written = np.zeros(A.shape[0], dtype=bool)
    for e in range(E):
        s, t = int(m_indptr[e]), int(m_indptr[e + 1])
        if t <= s:
            continue
        h = A[s:t] @ B[e].T
        if D is not None:
            h = h + D[s:t]
        out[s:t] = swiglu(h[:, :inter], h[:, inter:],
                          1.0 if alpha is None else alpha[e],
                          0.0 if beta is None else beta[e],
                          None if limit is None else limit[e])
        written[s:t] = True
    return out, written
