"""The pages' one printed example (grouped_mm_bf16, Examples section) against
the uniform grouped-GEMM workload and the oracle's output shape."""
import os

import numpy as np

import synth
from oracle.grouped_mm import grouped_mm

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden(name):
    kv = {}
    for line in open(os.path.join(HERE, "golden", name)):
        line = line.split("#", 1)[0].strip()
        if "=" in line:
            k, v = line.split("=", 1)
            kv[k.strip()] = [int(x) for x in v.split()]
    return kv


def test_uniform_workload_is_the_pages_example():
    g = _golden("grouped_mm_example.txt")
    case = synth.grouped_uniform()
    assert list(case.a.shape) == g["a_shape"]
    assert list(case.b.shape) == g["b_shape"]
    assert case.m_indptr.tolist() == g["m_indptr"]
    E, tpe = g["E"][0], g["tpe"][0]
    assert g["m_indptr"] == [e * tpe for e in range(E + 1)]


def test_oracle_output_shape_on_a_reduced_example():
    # same boundaries rule (arange(E+1) * tpe), reduced k and n so it runs fast
    g = _golden("grouped_mm_example.txt")
    E, tpe = g["E"][0], 4
    k, n = 16, 8
    rng = np.random.default_rng(0)
    a = rng.integers(-2, 3, (E * tpe, k)).astype(np.float64)
    b = rng.integers(-2, 3, (E, n, k)).astype(np.float64)
    from oracle.formats import f64_to_bf16_bits
    out, written = grouped_mm(f64_to_bf16_bits(a), f64_to_bf16_bits(b),
                              np.arange(E + 1, dtype=np.int32) * tpe)
    assert out.shape == (E * tpe, n)
    assert written.all()
