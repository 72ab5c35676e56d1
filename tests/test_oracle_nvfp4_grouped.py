"""Pins of the NVFP4 grouped GEMM oracle (no GPU): a literal exact loop over
bit fields, the one-expert case against the dense NVFP4 oracle, per-expert
alpha, unwritten rows and the sampled-rows helper."""
from fractions import Fraction

import numpy as np

from oracle.nvfp4 import base_product, mm_nvfp4_off
from oracle.nvfp4_grouped import expert_sf_bytes, grouped_mm_nvfp4, grouped_mm_nvfp4_rows

E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]  # magnitudes of codes 0..7 (OCP E2M1); bit 3 is the sign


def e2m1(c):
    return -E2M1[c & 7] if c & 8 else E2M1[c & 7]


def ue4m3(u):
    e, m = u >> 3, u & 7
    return Fraction(m, 512) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def tiled(row, col, k):
    """128x4 tiled scale offset, written out: 512-byte tiles of 128 rows x 4
    scale columns, row-block major."""
    col_tiles = (k // 16 + 3) // 4
    return ((row // 128) * col_tiles + col // 4) * 512 + (row % 32) * 16 + (row % 128) // 32 * 4 \
        + col % 4


def make(rng, counts, n, k):
    E, cum = len(counts), int(sum(counts))
    m_indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    a = rng.integers(0, 256, (cum, k // 2), dtype=np.uint8)
    b = rng.integers(0, 256, (E, n, k // 2), dtype=np.uint8)
    a_sf = rng.integers(0x20, 0x50, ((cum + 127) // 128) * ((k // 16 + 3) // 4) * 512,
                        dtype=np.uint8)
    b_sf = rng.integers(0x20, 0x50, E * expert_sf_bytes(n, k), dtype=np.uint8)
    alpha = rng.uniform(0.01, 2.0, E).astype(np.float32)
    return a, a_sf, b, b_sf, alpha, m_indptr


def test_literal_exact_loop():
    rng = np.random.default_rng(0)
    counts, n, k = (2, 0, 3, 1), 5, 48
    a, a_sf, b, b_sf, alpha, mi = make(rng, counts, n, k)
    out, written = grouped_mm_nvfp4(a, a_sf, b, b_sf, alpha, mi, k)
    per = expert_sf_bytes(n, k)
    for e in range(len(counts)):
        for r in range(mi[e], mi[e + 1]):
            for c in range(n):
                acc = Fraction(0)
                for kk in range(k):
                    ca = (int(a[r, kk // 2]) >> (4 * (kk % 2))) & 0xF
                    cb = (int(b[e, c, kk // 2]) >> (4 * (kk % 2))) & 0xF
                    sa = ue4m3(int(a_sf[tiled(r, kk // 16, k)]))
                    sb = ue4m3(int(b_sf[e * per + tiled(c, kk // 16, k)]))
                    acc += e2m1(ca) * sa * e2m1(cb) * sb
                assert out[r, c] == float(Fraction(float(alpha[e])) * acc), (e, r, c)
    assert written.all()


def test_one_expert_is_the_dense_nvfp4_product():
    rng = np.random.default_rng(1)
    a, a_sf, b, b_sf, alpha, mi = make(rng, (200,), 256, 256)
    out, written = grouped_mm_nvfp4(a, a_sf, b, b_sf, alpha, mi, 256)
    dense = mm_nvfp4_off(base_product(a, b[0], a_sf, b_sf, 256), float(alpha[0]))
    assert written.all() and np.array_equal(out, dense)


def test_per_expert_alpha_unwritten_rows_and_sampled_rows():
    rng = np.random.default_rng(2)
    counts, n, k = (5, 0, 7, 3), 8, 64
    a, a_sf, b, b_sf, alpha, mi = make(rng, counts, n, k)
    mi_off = mi + 2  # two leading rows outside every group
    a2 = np.concatenate([rng.integers(0, 256, (2, k // 2), dtype=np.uint8), a,
                         rng.integers(0, 256, (3, k // 2), dtype=np.uint8)])
    a2_sf = rng.integers(0x20, 0x50, ((a2.shape[0] + 127) // 128) * 512, dtype=np.uint8)
    out, written = grouped_mm_nvfp4(a2, a2_sf, b, b_sf, alpha, mi_off, k)
    assert not written[:2].any() and not written[-3:].any() and written[2:-3].all()
    assert (out[~written] == 0).all()
    alpha2 = alpha.copy()
    alpha2[2] *= 2
    out2, _ = grouped_mm_nvfp4(a2, a2_sf, b, b_sf, alpha2, mi_off, k)
    g2 = slice(mi_off[2], mi_off[3])
    assert np.array_equal(out2[g2], 2 * out[g2])
    keep = np.ones(out.shape[0], dtype=bool)
    keep[g2] = False
    assert np.array_equal(out2[keep], out[keep])
    rows, cols = [2, 6, 7, 13, 14, 16], [0, 3, 7]
    samp = grouped_mm_nvfp4_rows(a2[rows], a2_sf, lambda e: b[e][cols], b_sf, alpha, mi_off, k,
                                 8, rows, cols)
    assert np.array_equal(samp, out[np.ix_(rows, cols)])
