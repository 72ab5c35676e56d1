"""Acceptance rule for floating-point outputs and helpers shared by tests.

A GPU element passes iff

    |gpu - oracle| <= 2 * ulp_bf16(|oracle|) + 1e-3 * rms(oracle)

where ``rms`` is taken over every compared element of that call and
``ulp_bf16(x) = 2**(floor(log2 x) - 7)`` for normal x, ``2**-133`` below the
smallest normal and 0 at x == 0.  Any NaN/Inf in the GPU output fails.
"""
from __future__ import annotations

import numpy as np
import torch


def ulp_bf16(x) -> np.ndarray:
    ax = np.abs(np.asarray(x, dtype=np.float64))
    out = np.zeros_like(ax)
    nz = ax > 0
    e = np.floor(np.log2(np.where(nz, ax, 1.0)))
    out = np.where(ax >= 2.0 ** -126, np.ldexp(1.0, (e - 7).astype(np.int64)), 2.0 ** -133)
    return np.where(nz, out, 0.0)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def bits16(t: torch.Tensor) -> np.ndarray:
    """Raw uint16 patterns of a bf16/fp16 tensor."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def check_close(gpu, ref, what: str = "", rms_over=None):
    """Assert the tolerance rule element by element; return the max ratio
    |err| / tol (useful for reporting)."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    rms_src = r if rms_over is None else np.asarray(rms_over, dtype=np.float64)
    rms = float(np.sqrt(np.mean(rms_src ** 2))) if rms_src.size else 0.0
    tol = 2.0 * ulp_bf16(r) + 1e-3 * rms
    err = np.abs(g - r)
    bad = err > tol
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = [(tuple(i), float(g[tuple(i)]), float(r[tuple(i)]), float(tol[tuple(i)]))
                  for i in idx]
        raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} elements out of tolerance; "
                             f"first (index, gpu, oracle, tol): {detail}")
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(tol > 0, err / tol, np.where(err > 0, np.inf, 0.0))
    return float(ratio.max()) if ratio.size else 0.0


def sqnr_db(gpu, ref) -> float:
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    return float(10 * np.log10(np.sum(r ** 2) / max(np.sum((g - r) ** 2), 1e-300)))


def bank_view(bank: torch.Tensor):
    """uint16 numpy view of a bank tensor plus its base byte address."""
    return bits16(bank.reshape(-1)), bank.data_ptr()
