"""A whole LoRA MoE layer through the library, checked stage by stage against
the oracle: routing -> permuted rows -> FC1 with SwiGLU -> FC2 grouped GEMM
-> finalize with the FC2 LoRA delta.  Each stage's oracle takes the previous
stage's GPU output as its input, so the check isolates each stage while the
chaining (layouts, m_indptr, the permutation) is what the layer uses."""
import numpy as np
import pytest
import torch

import synth
from moe_expert_grouped_amd import (fill_w_ptr, grouped_mm_bf16, grouped_mm_swiglu,
                                    moe_finalize_lora, moe_permute_rows, moe_route_permutation)
from oracle.fc1 import grouped_mm_swiglu as fc1_ref
from oracle.finalize import moe_finalize
from oracle.grouped_mm import grouped_mm
from oracle.lora_delta import Bank, moe_fc2_lora_delta
from oracle.permute import permute_rows, route_permutation
from tests.parity import bits16, check_close, to_f64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,top_k,E,hidden,inter,L,r,zipf", [
    (200, 4, 8, 256, 128, 3, 16, 0.0),
    (333, 8, 16, 512, 256, 2, 8, 1.1),   # skewed routing, some experts empty
])
def test_moe_layer_stage_by_stage(gpu, T, top_k, E, hidden, inter, L, r, zipf):
    print(f"moe layer: T={T} top_k={top_k} E={E} hidden={hidden} inter={inter}", flush=True)
    g = synth.gen(T + E)
    ids = synth.routing_ids(seed=T, T=T, top_k=top_k, E=E, zipf_s=zipf)
    w = synth.softmax_weights(T, top_k, g)
    lora_ids = torch.randint(-1, L, (T,), generator=g).to(torch.int32)
    x = synth.bf16_normal((T, hidden), 1.0, g)
    w1 = synth.bf16_normal((E, 2 * inter, hidden), hidden ** -0.5, g)
    w2 = synth.bf16_normal((E, hidden, inter), inter ** -0.5, g)
    A = synth.bf16_normal((L, E, r, inter), 0.02, g)
    B = synth.bf16_normal((L, E, hidden, r), 0.02, g)

    dev = lambda t: t.to(gpu)
    m_indptr, perm = moe_route_permutation(dev(ids), E)
    a1 = moe_permute_rows(dev(x), perm, top_k)
    act = grouped_mm_swiglu(a1, dev(w1), m_indptr)
    fc2 = grouped_mm_bf16(act, dev(w2), m_indptr)
    Ad, Bd = dev(A), dev(B)
    wa, wb = fill_w_ptr(Ad), fill_w_ptr(Bd)
    sa, sb = E * r * inter, E * hidden * r
    out = moe_finalize_lora(fc2, act, perm, wa, sa, wb, sb, dev(ids), dev(w), dev(lora_ids), r,
                            hidden, num_adapters=L, scale=2.0, out_dtype=torch.float32)
    torch.cuda.synchronize()

    # routing and permuted rows: bitwise
    m_r, perm_r, _ = route_permutation(ids.numpy(), E)
    assert np.array_equal(m_indptr.cpu().numpy(), m_r)
    assert np.array_equal(perm.cpu().numpy(), perm_r)
    rows = T * top_k
    a1_r = permute_rows(bits16(x), perm_r, top_k, np.zeros((rows, hidden), np.uint16))
    assert np.array_equal(bits16(a1), a1_r)
    # FC1 + SwiGLU on the permuted rows
    h_ref, written = fc1_ref(a1_r, bits16(w1), m_r)
    assert written.all()
    check_close(to_f64(act), h_ref, "layer FC1 + SwiGLU")
    # FC2 on the GPU's FC1 output
    y_ref, _ = grouped_mm(bits16(act), bits16(w2), m_r)
    check_close(to_f64(fc2), y_ref, "layer FC2")
    # finalize: the combine of the GPU's FC2 rows plus the delta on the GPU's FC1 output
    delta = moe_fc2_lora_delta(bits16(act), perm_r, Bank(bits16(A.reshape(-1)), Ad.data_ptr()),
                               wa.cpu().numpy(), sa, Bank(bits16(B.reshape(-1)), Bd.data_ptr()),
                               wb.cpu().numpy(), sb, ids.numpy(), w.numpy(), lora_ids.numpy(),
                               r, hidden, 2.0)
    ref = moe_finalize(bits16(fc2), "bf16", perm_r, w.numpy(), delta)
    check_close(to_f64(out), ref, "layer finalize + delta")
