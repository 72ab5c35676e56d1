"""Seeded input recipes.

Every tensor is drawn from ``torch.Generator`` seeded per workload, so the
same seed gives the same bytes on the same device type.  Small workloads are
drawn on the CPU (and copied to the GPU by the caller) so that the oracle and
the GPU see identical values; the large ones are drawn directly on the GPU
and the oracle reads back the slices it needs.

bf16 tensors are produced by drawing float32 and converting with torch's own
cast.  Block scales of the NVFP4 operands are drawn as raw bytes over the
whole (padded) scale buffer, so nothing here knows the scale-factor layout.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = [
    "gen",
    "bf16_normal",
    "bf16_ints",
    "route",
    "routing_ids",
    "softmax_weights",
    "distinct_topk",
    "zipf_counts",
    "sf_buffer_bytes",
    "GroupedCase",
    "DeltaCase",
    "Nvfp4Case",
    "grouped_tiny",
    "grouped_uniform",
    "grouped_zipf",
    "grouped_int_probe",
    "delta_tiny",
    "delta_at_scale",
    "delta_int_probe",
    "nvfp4_lora_case",
    "nvfp4_probe",
    "nvfp4_scale_probe",
    "Nvfp4GroupedCase",
    "nvfp4_grouped_case",
    "nvfp4_grouped_scale_probe",
    "Fc1Case",
    "fc1_case",
]


def gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def bf16_normal(shape, std: float, g: torch.Generator, device="cpu") -> torch.Tensor:
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def bf16_ints(shape, lo: int, hi: int, g: torch.Generator, device="cpu") -> torch.Tensor:
    """Uniform integers in [lo, hi] stored as bf16 (exact for |v| <= 256)."""
    return torch.randint(lo, hi + 1, shape, generator=g, device=device).to(torch.bfloat16)


def sf_buffer_bytes(rows: int, k: int) -> int:
    """Bytes of a 128x4-tiled UE4M3 scale buffer: rows padded to 128, scale
    columns (k/16) padded to 4; 512 bytes per 128x4 tile."""
    cols = -(-k // 16)
    return (-(-rows // 128)) * (-(-cols // 4)) * 512


# ----------------------------------------------------------------------------
# routing bookkeeping
# ----------------------------------------------------------------------------

def route(topk_ids: torch.Tensor, num_experts: int, g: torch.Generator,
          inactive_frac: float = 0.1, padded_rows: int | None = None):
    """Expert-sorted permutation of the T*top_k routed rows.

    Row ``x = t*top_k + j`` goes to position ``perm[x]`` of a stable sort of
    the flattened ids; ``m_indptr`` holds the per-expert cumulative counts.
    Afterwards ``round(inactive_frac * T*top_k)`` random entries of ``perm``
    are set to -1 (the row stays in the GEMM, the slot drops out of the delta).
    """
    flat = topk_ids.reshape(-1).to(torch.int64).cpu()
    order = torch.argsort(flat, stable=True)
    perm = torch.empty_like(order)
    perm[order] = torch.arange(flat.numel())
    counts = torch.bincount(flat, minlength=num_experts)
    m_indptr = torch.zeros(num_experts + 1, dtype=torch.int64)
    m_indptr[1:] = torch.cumsum(counts, 0)
    n_off = int(round(inactive_frac * flat.numel()))
    if n_off:
        off = torch.randperm(flat.numel(), generator=g)[:n_off]
        perm[off] = -1
    return perm.to(torch.int32), m_indptr.to(torch.int32)


def distinct_topk(T: int, E: int, k: int, g: torch.Generator) -> torch.Tensor:
    return torch.rand(T, E, generator=g).argsort(dim=1)[:, :k].to(torch.int32)


def routing_ids(seed: int, T: int, top_k: int, E: int, invalid_frac: float = 0.0,
                zipf_s: float = 0.0) -> torch.Tensor:
    """Router output ``topk_ids`` int32 ``[T, top_k]`` (CPU).

    ``zipf_s == 0``: each token's ``top_k`` experts are distinct and uniform.
    ``zipf_s > 0``: every slot draws an expert independently with probability
    ``~ rank**-zipf_s`` over a seeded rank order (hot experts; repeats allowed).
    Then ``round(invalid_frac * T*top_k)`` random slots get an id outside
    ``[0, E)`` (-1, E, or a large value), i.e. an expert not held here.
    """
    g = gen(seed)
    if zipf_s == 0.0:
        ids = distinct_topk(T, E, top_k, g) if top_k <= E else \
            torch.randint(0, E, (T, top_k), generator=g, dtype=torch.int32)
    else:
        order = torch.randperm(E, generator=g)
        p = torch.arange(1, E + 1, dtype=torch.float64) ** (-zipf_s)
        draw = torch.multinomial(p, T * top_k, replacement=True, generator=g)
        ids = order[draw].reshape(T, top_k).to(torch.int32)
    n_bad = int(round(invalid_frac * T * top_k))
    if n_bad:
        flat = ids.reshape(-1)
        where = torch.randperm(flat.numel(), generator=g)[:n_bad]
        bad = torch.tensor([-1, E, E + 4096, -(1 << 30)], dtype=torch.int32)
        flat[where] = bad[torch.randint(0, 4, (n_bad,), generator=g)]
    return ids


def softmax_weights(T: int, k: int, g: torch.Generator) -> torch.Tensor:
    return torch.softmax(torch.randn(T, k, generator=g, dtype=torch.float32), dim=1)


def zipf_counts(total: int, num_experts: int, num_zero: int, s: float, cap: int,
                seed: int) -> np.ndarray:
    """Per-expert row counts: ``num_zero`` seeded empty experts, the rest get
    proportions ``p_i ~ rank_i**-s`` over a seeded rank order, capped at
    ``cap`` with the excess spread over the uncapped experts in proportion to
    p, and rounded to integers by largest remainder so they sum to ``total``."""
    rng = np.random.default_rng(seed)
    zero = rng.choice(num_experts, num_zero, replace=False)
    live = np.setdiff1d(np.arange(num_experts), zero)
    order = rng.permutation(live)
    p = np.arange(1, live.size + 1, dtype=np.float64) ** (-s)
    counts = np.zeros(num_experts, dtype=np.int64)
    capped = np.zeros(live.size, dtype=bool)
    remaining = total
    while True:
        free = ~capped
        ideal = np.zeros(live.size)
        ideal[free] = remaining * p[free] / p[free].sum()
        over = free & (ideal > cap)
        if not over.any():
            break
        capped |= over
        remaining = total - cap * int(capped.sum())
    base = np.floor(ideal).astype(np.int64)
    base[capped] = cap
    short = total - int(base.sum())
    frac = ideal - np.floor(ideal)
    frac[capped] = -1.0
    for i in np.argsort(-frac, kind="stable")[:short]:
        base[i] += 1
    counts[order] = base
    assert counts.sum() == total and counts.max() <= cap
    return counts


# ----------------------------------------------------------------------------
# grouped GEMM workloads
# ----------------------------------------------------------------------------

@dataclass
class GroupedCase:
    name: str
    a: torch.Tensor          # [cum_m, k] bf16
    b: torch.Tensor          # [E, n, k] bf16
    m_indptr: torch.Tensor   # [E+1] int32
    extra: dict = field(default_factory=dict)


def grouped_tiny(seed: int = 1) -> GroupedCase:
    """Tiny MoE FC2: E=4, T=16, top_k=2 (32 routed rows), I=128, H=256."""
    d = delta_tiny(seed)
    return GroupedCase("tiny-moe-fc2 E=4 cum_m=32 k=128 n=256", d.extra["gemm_a"],
                       d.extra["gemm_b"], d.extra["m_indptr"])


def grouped_uniform(seed: int = 2, device="cpu", E=8, tpe=128, k=4096, n=2048) -> GroupedCase:
    """Uniform grouped GEMM: E experts x tpe rows, a ~ N(0,1), b ~ N(0, 1/k)."""
    g = gen(seed, device)
    a = bf16_normal((E * tpe, k), 1.0, g, device)
    b = bf16_normal((E, n, k), 1.0 / math.sqrt(k), g, device)
    m_indptr = (torch.arange(E + 1, dtype=torch.int32) * tpe).to(device)
    return GroupedCase(f"uniform E={E} tpe={tpe} k={k} n={n}", a, b, m_indptr)


def grouped_zipf(seed: int = 3, device="cpu", E=128, T=4096, top_k=8, k=2048, n=7168,
                 num_zero=8, s=1.1) -> GroupedCase:
    """Skewed ragged MoE FC2: cum_m = T*top_k rows over E experts with Zipf(s)
    counts and ``num_zero`` empty experts; a ~ N(0,1), b ~ N(0, 1/k)."""
    counts = zipf_counts(T * top_k, E, num_zero, s, T, seed)
    m_indptr = torch.zeros(E + 1, dtype=torch.int32)
    m_indptr[1:] = torch.from_numpy(np.cumsum(counts)).to(torch.int32)
    g = gen(seed, device)
    a = bf16_normal((T * top_k, k), 1.0, g, device)
    b = torch.empty((E, n, k), dtype=torch.bfloat16, device=device)
    for e in range(E):  # per expert to bound the float32 staging buffer
        b[e] = bf16_normal((n, k), 1.0 / math.sqrt(k), g, device)
    return GroupedCase(f"zipf E={E} cum_m={T*top_k} k={k} n={n}", a, b, m_indptr.to(device),
                       {"counts": counts})


def grouped_int_probe(seed: int = 101, counts=(0, 1, 17, 128, 0, 255), n=256, k=128,
                      lo=-3, hi=3) -> GroupedCase:
    """Small-integer operands: every fp32 partial sum is exact, so the rounded
    result is unique.  Covers empty groups and ragged tails."""
    g = gen(seed)
    E = len(counts)
    m_indptr = torch.zeros(E + 1, dtype=torch.int32)
    m_indptr[1:] = torch.cumsum(torch.tensor(counts, dtype=torch.int32), 0)
    cum = int(m_indptr[-1])
    a = bf16_ints((cum, k), lo, hi, g)
    b = bf16_ints((E, n, k), lo, hi, g)
    return GroupedCase(f"int-probe counts={list(counts)} n={n} k={k}", a, b, m_indptr)


# ----------------------------------------------------------------------------
# FC2 LoRA delta workloads
# ----------------------------------------------------------------------------

@dataclass
class DeltaCase:
    name: str
    act: torch.Tensor          # [padded_rows, I] bf16 (permuted activation)
    perm: torch.Tensor         # [T*top_k] int32, <0 inactive
    A: torch.Tensor            # [L, E, r, I] bf16 (A_down bank)
    B: torch.Tensor            # [L, E, H, r] bf16 (B_down bank)
    topk_ids: torch.Tensor     # [T, top_k] int32
    topk_weights: torch.Tensor # [T, top_k] fp32
    lora_ids: torch.Tensor     # [T] int32, -1 none
    scale: float
    extra: dict = field(default_factory=dict)

    @property
    def T(self):
        return self.topk_ids.shape[0]

    @property
    def top_k(self):
        return self.topk_ids.shape[1]

    @property
    def L(self):
        return self.A.shape[0]

    @property
    def E(self):
        return self.A.shape[1]

    @property
    def rank(self):
        return self.A.shape[2]

    @property
    def I(self):
        return self.A.shape[3]

    @property
    def H(self):
        return self.B.shape[2]

    def cast(self, dtype: torch.dtype) -> "DeltaCase":
        """The same case with the activation and both banks stored as
        ``dtype`` (torch's conversion; exact for the small-integer probes)."""
        return DeltaCase(f"{self.name} {str(dtype).replace('torch.', '')}", self.act.to(dtype),
                         self.perm, self.A.to(dtype), self.B.to(dtype), self.topk_ids,
                         self.topk_weights, self.lora_ids, self.scale, dict(self.extra))


def delta_tiny(seed: int = 1) -> DeltaCase:
    """Tiny MoE FC2 with LoRA delta: E=4, T=16, top_k=2, I=128, H=256,
    2 adapters of rank 8, lora_ids in {-1,0,1}, scale 2."""
    T, k, E, I, H, L, r = 16, 2, 4, 128, 256, 2, 8
    g = gen(seed)
    topk_ids = distinct_topk(T, E, k, g)
    topk_weights = softmax_weights(T, k, g)
    perm, m_indptr = route(topk_ids, E, g, 0.1)
    act = bf16_normal((T * k, I), 1.0, g)
    gemm_b = bf16_normal((E, H, I), 1.0 / math.sqrt(I), g)
    A = bf16_normal((L, E, r, I), 0.02, g)
    B = bf16_normal((L, E, H, r), 0.02, g)
    lora_ids = torch.randint(-1, L, (T,), generator=g).to(torch.int32)
    return DeltaCase("tiny T=16 top_k=2 E=4 I=128 H=256 L=2 r=8", act, perm, A, B, topk_ids,
                     topk_weights, lora_ids, 2.0,
                     {"gemm_a": act, "gemm_b": gemm_b, "m_indptr": m_indptr})


def delta_at_scale(seed: int = 4, device="cpu", T=8192, top_k=8, E=64, I=2048, H=4096, L=8,
                   r=16, inactive_frac=0.1) -> DeltaCase:
    """MoE FC2 LoRA delta at scale: a random permutation of T*top_k rows with
    10% of the slots inactive, 8 adapters of rank 16, lora_ids in {-1..L-1}."""
    g = gen(seed)  # routing on the CPU, large tensors on `device`
    topk_ids = distinct_topk(T, E, top_k, g)
    topk_weights = softmax_weights(T, top_k, g)
    n = T * top_k
    perm = torch.randperm(n, generator=g)
    off = torch.randperm(n, generator=g)[: int(round(inactive_frac * n))]
    perm[off] = -1
    lora_ids = torch.randint(-1, L, (T,), generator=g).to(torch.int32)
    gd = gen(seed + 1000, device)
    act = bf16_normal((n, I), 1.0, gd, device)
    A = bf16_normal((L, E, r, I), 0.02, gd, device)
    B = bf16_normal((L, E, H, r), 0.02, gd, device)
    return DeltaCase(f"at-scale T={T} top_k={top_k} E={E} I={I} H={H} L={L} r={r}",
                     act, perm.to(torch.int32).to(device), A, B, topk_ids.to(device),
                     topk_weights.to(device), lora_ids.to(device), 2.0)


def delta_int_probe(seed: int = 102, T=24, top_k=3, E=5, I=64, H=256, L=3, r=16,
                    pad_rows=7) -> DeltaCase:
    """Small-integer delta probe: act in {-2..2}, A,B in {-1,0,1}, weights in
    {1/4,1/2,3/4,1}, scale 2 -- every intermediate is exact in fp32.  The
    permutation has inactive slots and unused padded rows; lora_ids include
    -1; the bank is later addressed through a shuffled pointer table."""
    g = gen(seed)
    topk_ids = distinct_topk(T, E, top_k, g)
    topk_weights = (torch.randint(1, 5, (T, top_k), generator=g).to(torch.float32) / 4.0)
    n = T * top_k
    perm = torch.randperm(n + pad_rows, generator=g)[:n]
    off = torch.randperm(n, generator=g)[: n // 6]
    perm[off] = -1
    lora_ids = torch.randint(-1, L, (T,), generator=g).to(torch.int32)
    act = bf16_ints((n + pad_rows, I), -2, 2, g)
    A = bf16_ints((L, E, r, I), -1, 1, g)
    B = bf16_ints((L, E, H, r), -1, 1, g)
    return DeltaCase(f"int-probe T={T} top_k={top_k} E={E} I={I} H={H} L={L} r={r}", act,
                     perm.to(torch.int32), A, B, topk_ids, topk_weights, lora_ids, 2.0)


# ----------------------------------------------------------------------------
# NVFP4 + LoRA workloads
# ----------------------------------------------------------------------------

@dataclass
class Nvfp4Case:
    name: str
    a: torch.Tensor        # [M, K/2] uint8
    b: torch.Tensor        # [N, K/2] uint8
    a_sf: torch.Tensor     # flat uint8, 128x4-tiled UE4M3
    b_sf: torch.Tensor
    alpha: torch.Tensor    # fp32 [1]
    d: torch.Tensor        # [M, r] bf16
    lora_b: torch.Tensor   # [N, r] bf16
    lora_scale: torch.Tensor  # fp32 [1]
    bias: torch.Tensor | None  # [N] bf16
    K: int

    @property
    def M(self):
        return self.a.shape[0]

    @property
    def N(self):
        return self.b.shape[0]

    @property
    def rank(self):
        return self.d.shape[1]


def _scale_codes(nbytes: int, lo: int, hi: int, g, device):
    return torch.randint(lo, hi + 1, (nbytes,), generator=g, device=device).to(torch.uint8)


def nvfp4_lora_case(seed: int = 5, device="cpu", M=4096, N=8192, K=8192, r=16,
                    alpha=0.01, lora_scale=0.5, with_bias=True) -> Nvfp4Case:
    """NVFP4 base GEMM with LoRA: code bytes uniform over 0..255 (both nibbles
    uniform over the 16 E2M1 codes), UE4M3 scale bytes uniform over
    0x28..0x48 (values 0.25..4) across the whole padded buffer,
    d ~ N(0,1), lora_b ~ N(0, 0.02), bias ~ N(0, 0.1)."""
    g = gen(seed, device)
    a = torch.randint(0, 256, (M, K // 2), generator=g, device=device).to(torch.uint8)
    b = torch.randint(0, 256, (N, K // 2), generator=g, device=device).to(torch.uint8)
    a_sf = _scale_codes(sf_buffer_bytes(M, K), 0x28, 0x48, g, device)
    b_sf = _scale_codes(sf_buffer_bytes(N, K), 0x28, 0x48, g, device)
    d = bf16_normal((M, r), 1.0, g, device)
    lora_b = bf16_normal((N, r), 0.02, g, device)
    bias = bf16_normal((N,), 0.1, g, device) if with_bias else None
    return Nvfp4Case(f"nvfp4 M={M} N={N} K={K} r={r}", a, b, a_sf, b_sf,
                     torch.tensor([alpha], dtype=torch.float32, device=device), d, lora_b,
                     torch.tensor([lora_scale], dtype=torch.float32, device=device), bias, K)


def nvfp4_probe(kind: str, seed: int = 103, M=128, N=256, K=256, r=16) -> Nvfp4Case:
    """Structured NVFP4 probes (all scales = 0x38 i.e. 1.0 unless noted):

    - ``exact``: random codes, alpha 1, no LoRA/bias; all sums are exact.
    - ``identity``: b selects column n of a for n < K (code 0x2 = 1.0 on the
      diagonal), so the output equals the dequantised a.
    - ``lora_only``: all codes zero, random LoRA and bias; the output is the
      LoRA term plus bias alone.
    - ``zero_codes_scaled``: random scales over the full finite UE4M3 range
      but zero codes -- base must vanish exactly.
    """
    g = gen(seed)
    one = 0x38
    a_sf = torch.full((sf_buffer_bytes(M, K),), one, dtype=torch.uint8)
    b_sf = torch.full((sf_buffer_bytes(N, K),), one, dtype=torch.uint8)
    d = bf16_normal((M, r), 1.0, g)
    lora_b = bf16_normal((N, r), 0.02, g)
    bias = None
    alpha = torch.tensor([1.0], dtype=torch.float32)
    lora_scale = torch.tensor([0.0], dtype=torch.float32)
    if kind == "exact":
        a = torch.randint(0, 256, (M, K // 2), generator=g).to(torch.uint8)
        b = torch.randint(0, 256, (N, K // 2), generator=g).to(torch.uint8)
    elif kind == "identity":
        a = torch.randint(0, 256, (M, K // 2), generator=g).to(torch.uint8)
        b = torch.zeros((N, K // 2), dtype=torch.uint8)
        for nn in range(min(N, K)):
            b[nn, nn // 2] = 0x02 if nn % 2 == 0 else 0x20
    elif kind == "lora_only":
        a = torch.zeros((M, K // 2), dtype=torch.uint8)
        b = torch.zeros((N, K // 2), dtype=torch.uint8)
        a_sf = _scale_codes(a_sf.numel(), 0x01, 0x7E, g, "cpu")
        b_sf = _scale_codes(b_sf.numel(), 0x01, 0x7E, g, "cpu")
        bias = bf16_normal((N,), 0.1, g)
        lora_scale = torch.tensor([0.5], dtype=torch.float32)
        alpha = torch.tensor([0.01], dtype=torch.float32)
    elif kind == "zero_codes_scaled":
        a = torch.zeros((M, K // 2), dtype=torch.uint8)
        b = torch.zeros((N, K // 2), dtype=torch.uint8)
        a_sf = _scale_codes(a_sf.numel(), 0x00, 0x7E, g, "cpu")
        b_sf = _scale_codes(b_sf.numel(), 0x00, 0x7E, g, "cpu")
    else:
        raise ValueError(kind)
    return Nvfp4Case(f"nvfp4-probe-{kind} M={M} N={N} K={K}", a, b, a_sf, b_sf, alpha, d,
                     lora_b, lora_scale, bias, K)


def _selector(rows: int, K: int) -> torch.Tensor:
    """uint8 ``[rows, K/2]`` codes with E2M1 1.0 (code 0x2) at element
    ``(i, i % K)`` of row i and zeros elsewhere."""
    codes = torch.zeros((rows, K // 2), dtype=torch.uint8)
    i = torch.arange(rows)
    col = i % K
    codes[i, col // 2] = torch.where(col % 2 == 0, torch.tensor(0x02, dtype=torch.uint8),
                                     torch.tensor(0x20, dtype=torch.uint8))
    return codes


def nvfp4_scale_probe(side: str, seed: int = 104, M=300, N=512, K=512) -> Nvfp4Case:
    """Probes of the GEMM's own scale decode.  One operand has random codes
    and scale bytes uniform over every finite UE4M3 code 0x00..0x7E; the
    other selects one element per output (E2M1 1.0 at scale 1.0), so every
    output is a single exact product, alpha 1, no LoRA and no bias:

    - ``a``: ``b`` row n selects element n, so ``out[m, n] = dequant(a)[m, n]``
      for ``n < K``;
    - ``b``: ``a`` row m selects element m, so ``out[m, n] = dequant(b)[n, m]``
      for ``m < K``.
    """
    g = gen(seed)
    one = 0x38
    if side == "a":
        a = torch.randint(0, 256, (M, K // 2), generator=g).to(torch.uint8)
        a_sf = _scale_codes(sf_buffer_bytes(M, K), 0x00, 0x7E, g, "cpu")
        b = _selector(N, K)
        b_sf = torch.full((sf_buffer_bytes(N, K),), one, dtype=torch.uint8)
    elif side == "b":
        a = _selector(M, K)
        a_sf = torch.full((sf_buffer_bytes(M, K),), one, dtype=torch.uint8)
        b = torch.randint(0, 256, (N, K // 2), generator=g).to(torch.uint8)
        b_sf = _scale_codes(sf_buffer_bytes(N, K), 0x00, 0x7E, g, "cpu")
    else:
        raise ValueError(side)
    return Nvfp4Case(f"nvfp4-scale-probe-{side} M={M} N={N} K={K}", a, b, a_sf, b_sf,
                     torch.tensor([1.0], dtype=torch.float32), bf16_normal((M, 16), 1.0, g),
                     bf16_normal((N, 16), 0.02, g), torch.tensor([0.0], dtype=torch.float32),
                     None, K)


@dataclass
class Nvfp4GroupedCase:
    name: str
    a: torch.Tensor          # uint8 [cum_m, K/2]
    a_sf: torch.Tensor       # uint8, 128x4 layout over cum_m rows
    b: torch.Tensor          # uint8 [E, N, K/2]
    b_sf: torch.Tensor       # uint8, E consecutive 128x4 buffers of [N, K/16]
    alpha: torch.Tensor      # fp32 [E]
    m_indptr: torch.Tensor   # int32 [E+1]
    k: int


def nvfp4_grouped_case(seed: int = 6, device="cpu", counts=None, E=128, T=4096, top_k=8,
                       n=7168, k=2048, exact=False) -> Nvfp4GroupedCase:
    """NVFP4 grouped GEMM operands.  Default: the skewed MoE FC2 routing of
    ``grouped_zipf`` (E=128, cum_m=32768, Zipf 1.1 counts with 8 empty
    experts) with FP4 weights of n=7168, k=2048.  Code bytes uniform over
    0..255; scale bytes uniform over 0x28..0x48 (0.25..4); alpha per expert
    uniform over 0.005..0.02.  ``exact``: all scales 1.0 and alpha a power of
    two per expert, so every fp32 sum is exact."""
    if counts is None:
        counts = zipf_counts(T * top_k, E, 8, 1.1, T, 3)
    counts = np.asarray(counts, dtype=np.int64)
    E = len(counts)
    m_indptr = torch.zeros(E + 1, dtype=torch.int32)
    m_indptr[1:] = torch.from_numpy(np.cumsum(counts)).to(torch.int32)
    cum = int(m_indptr[-1])
    g = gen(seed, device)
    a = torch.randint(0, 256, (cum, k // 2), generator=g, device=device).to(torch.uint8)
    b = torch.randint(0, 256, (E, n, k // 2), generator=g, device=device).to(torch.uint8)
    a_bytes, b_bytes = sf_buffer_bytes(cum, k), E * sf_buffer_bytes(n, k)
    if exact:
        a_sf = torch.full((a_bytes,), 0x38, dtype=torch.uint8, device=device)
        b_sf = torch.full((b_bytes,), 0x38, dtype=torch.uint8, device=device)
        ex = torch.randint(-3, 2, (E,), generator=g, device=device)
        alpha = torch.pow(2.0, ex.to(torch.float32))
    else:
        a_sf = _scale_codes(a_bytes, 0x28, 0x48, g, device)
        b_sf = _scale_codes(b_bytes, 0x28, 0x48, g, device)
        alpha = 0.005 + 0.015 * torch.rand(E, generator=g, device=device, dtype=torch.float32)
    return Nvfp4GroupedCase(f"nvfp4-grouped E={E} cum_m={cum} n={n} k={k}", a, a_sf, b, b_sf,
                            alpha.to(torch.float32), m_indptr.to(device), k)


def nvfp4_grouped_scale_probe(side: str, counts, n=512, k=512, seed=105) -> Nvfp4GroupedCase:
    """The scale-decode probes of :func:`nvfp4_scale_probe` through the
    grouped walk: ``a`` side -- a random codes with scales over every finite
    UE4M3 code, each expert's b selects element n for output column n;
    ``b`` side -- a's row i selects element ``i % k``, the experts' b have
    random codes and scales over every finite code.  alpha 1 for every
    expert, so each output is one exact product."""
    counts = np.asarray(counts, dtype=np.int64)
    E = len(counts)
    m_indptr = torch.zeros(E + 1, dtype=torch.int32)
    m_indptr[1:] = torch.from_numpy(np.cumsum(counts)).to(torch.int32)
    cum = int(m_indptr[-1])
    g = gen(seed)
    a_bytes, per = sf_buffer_bytes(cum, k), sf_buffer_bytes(n, k)
    if side == "a":
        a = torch.randint(0, 256, (cum, k // 2), generator=g).to(torch.uint8)
        a_sf = _scale_codes(a_bytes, 0x00, 0x7E, g, "cpu")
        b = _selector(n, k).unsqueeze(0).repeat(E, 1, 1)
        b_sf = torch.full((E * per,), 0x38, dtype=torch.uint8)
    elif side == "b":
        a = _selector(cum, k)
        a_sf = torch.full((a_bytes,), 0x38, dtype=torch.uint8)
        b = torch.randint(0, 256, (E, n, k // 2), generator=g).to(torch.uint8)
        b_sf = _scale_codes(E * per, 0x00, 0x7E, g, "cpu")
    else:
        raise ValueError(side)
    return Nvfp4GroupedCase(f"nvfp4-grouped-scale-probe-{side} E={E} cum_m={cum} n={n} k={k}",
                            a, a_sf, b, b_sf, torch.ones(E, dtype=torch.float32), m_indptr, k)


@dataclass
class Fc1Case:
    name: str
    a: torch.Tensor          # [cum_m, hidden] bf16 (permuted FC1 input)
    b: torch.Tensor          # [E, 2*inter, hidden] bf16 (gate rows, then up rows)
    m_indptr: torch.Tensor   # [E+1] int32
    delta: torch.Tensor | None   # [cum_m, 2*inter] bf16
    alpha: torch.Tensor | None   # [E] fp32
    beta: torch.Tensor | None
    limit: torch.Tensor | None


def fc1_case(seed: int = 7, device="cpu", counts=None, E=128, T=4096, top_k=8, hidden=7168,
             inter=2048, with_delta=False, act_params=False, ints=False) -> Fc1Case:
    """FC1 operands.  Default: the skewed routing of ``grouped_zipf`` (E=128,
    cum_m=32768) with hidden=7168 and inter=2048; a ~ N(0,1), b ~ N(0, 1/hidden)
    (so h ~ N(0,1)).  ``with_delta``: an additive FC1 delta ~ N(0, 0.1);
    ``act_params``: per-expert alpha uniform 1..2, beta uniform -1..1, clamp
    limit uniform 0.5..4 (so the clamp acts on part of h).  ``ints``: small
    integers (h exact in fp32)."""
    if counts is None:
        counts = zipf_counts(T * top_k, E, 8, 1.1, T, 3)
    counts = np.asarray(counts, dtype=np.int64)
    E = len(counts)
    m_indptr = torch.zeros(E + 1, dtype=torch.int32)
    m_indptr[1:] = torch.from_numpy(np.cumsum(counts)).to(torch.int32)
    cum = int(m_indptr[-1])
    g = gen(seed, device)
    if ints:
        a = bf16_ints((cum, hidden), -2, 2, g, device)
        b = bf16_ints((E, 2 * inter, hidden), -1, 1, g, device)
    else:
        a = bf16_normal((cum, hidden), 1.0, g, device)
        b = torch.empty((E, 2 * inter, hidden), dtype=torch.bfloat16, device=device)
        for e in range(E):  # per expert to bound the float32 staging buffer
            b[e] = bf16_normal((2 * inter, hidden), hidden ** -0.5, g, device)
    delta = bf16_normal((cum, 2 * inter), 0.1, g, device) if with_delta else None
    alpha = beta = limit = None
    if act_params:
        alpha = 1.0 + torch.rand(E, generator=g, device=device, dtype=torch.float32)
        beta = 2.0 * torch.rand(E, generator=g, device=device, dtype=torch.float32) - 1.0
        limit = 0.5 + 3.5 * torch.rand(E, generator=g, device=device, dtype=torch.float32)
    return Fc1Case(f"fc1 E={E} cum_m={cum} hidden={hidden} inter={inter}", a, b,
                   m_indptr.to(device), delta, alpha, beta, limit)
