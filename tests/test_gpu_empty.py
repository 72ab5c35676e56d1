"""Empty inputs through every entry point: zero tokens, zero rows, no rows
inside any group.  Each call must succeed, write nothing outside its output
and leave a caller-provided output's untouched rows as they were."""
import pytest
import torch

import synth
from moe_expert_grouped_amd import (bgmv_moe_gemm2_lora_delta, fill_w_ptr, grouped_mm_bf16,
                                    grouped_mm_nvfp4, grouped_mm_swiglu, mm_nvfp4_lora,
                                    moe_finalize_lora, moe_permute_rows, moe_route_permutation)

pytestmark = pytest.mark.gpu


def test_grouped_gemms_with_no_rows(gpu):
    print("empty: grouped GEMMs with cum_m = 0", flush=True)
    E, n, k = 4, 256, 128
    m0 = torch.zeros(E + 1, dtype=torch.int32, device=gpu)
    a = torch.empty((0, k), dtype=torch.bfloat16, device=gpu)
    b = synth.bf16_normal((E, n, k), 1.0, synth.gen(1, gpu), gpu)
    assert grouped_mm_bf16(a, b, m0).shape == (0, n)
    assert grouped_mm_swiglu(a, b, m0).shape == (0, n // 2)
    k4 = 256  # NVFP4 K: a multiple of 256
    a4 = torch.empty((0, k4 // 2), dtype=torch.uint8, device=gpu)
    b4 = torch.zeros((E, n, k4 // 2), dtype=torch.uint8, device=gpu)
    sf = torch.zeros(E * synth.sf_buffer_bytes(n, k4), dtype=torch.uint8, device=gpu)
    alpha = torch.ones(E, dtype=torch.float32, device=gpu)
    out = grouped_mm_nvfp4(a4, torch.empty(0, dtype=torch.uint8, device=gpu), b4, sf, m0, alpha)
    torch.cuda.synchronize()
    assert out.shape == (0, n)


def test_grouped_gemms_with_rows_but_no_groups(gpu):
    """cum_m > 0 but every group empty: a caller's output keeps all its rows."""
    print("empty: grouped GEMMs whose groups hold no rows", flush=True)
    E, n, k, m = 4, 256, 128, 40
    g = synth.gen(2, gpu)
    m0 = torch.full((E + 1,), 17, dtype=torch.int32, device=gpu)  # every group [17, 17)
    a = synth.bf16_normal((m, k), 1.0, g, gpu)
    b = synth.bf16_normal((E, n, k), 1.0, g, gpu)
    fill = synth.bf16_normal((m, n), 1.0, g, gpu)
    out = fill.clone()
    grouped_mm_bf16(a, b, m0, out=out)
    fill_h = synth.bf16_normal((m, n // 2), 1.0, g, gpu)
    out_h = fill_h.clone()
    grouped_mm_swiglu(a, b, m0, out=out_h)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), fill.view(torch.int16))
    assert torch.equal(out_h.view(torch.int16), fill_h.view(torch.int16))


def _delta_args(T, top_k, E, I, H, L, r, padded_rows, gpu):
    g = synth.gen(3, gpu)
    A = synth.bf16_normal((L, E, r, I), 0.02, g, gpu)
    B = synth.bf16_normal((L, E, H, r), 0.02, g, gpu)
    act = synth.bf16_normal((padded_rows, I), 1.0, g, gpu)
    ids = torch.randint(0, E, (T, top_k), generator=g, device=gpu, dtype=torch.int32)
    w = torch.rand((T, top_k), generator=g, device=gpu, dtype=torch.float32)
    lora = torch.randint(0, L, (T,), generator=g, device=gpu, dtype=torch.int32)
    perm = torch.randint(0, max(padded_rows, 1), (T * top_k,), generator=g, device=gpu,
                         dtype=torch.int32)
    return act, perm, fill_w_ptr(A), E * r * I, fill_w_ptr(B), E * H * r, ids, w, lora


def test_delta_and_finalize_with_no_tokens(gpu):
    print("empty: delta and finalize with T = 0", flush=True)
    E, I, H, L, r = 8, 128, 256, 2, 16
    act, perm, wa, sa, wb, sb, ids, w, lora = _delta_args(0, 4, E, I, H, L, r, 0, gpu)
    out = bgmv_moe_gemm2_lora_delta(act, perm, wa, sa, wb, sb, ids, w, lora, r, H, num_adapters=L)
    fin = moe_finalize_lora(torch.empty((0, H), dtype=torch.bfloat16, device=gpu), act, perm,
                            wa, sa, wb, sb, ids, w, lora, r, H, num_adapters=L)
    torch.cuda.synchronize()
    assert out.shape == (0, H) and fin.shape == (0, H)


def test_delta_and_finalize_with_no_activation_rows(gpu):
    """padded_rows = 0: every slot's row lies outside [0, padded_rows), so
    every slot is inactive -- the delta is +0 everywhere and the finalize,
    with no FC2 row to combine, is +0 too (bitwise)."""
    print("empty: delta and finalize with padded_rows = 0", flush=True)
    T, top_k, E, I, H, L, r = 37, 4, 8, 128, 256, 2, 16
    act, perm, wa, sa, wb, sb, ids, w, lora = _delta_args(T, top_k, E, I, H, L, r, 0, gpu)
    out = bgmv_moe_gemm2_lora_delta(act, perm, wa, sa, wb, sb, ids, w, lora, r, H,
                                    num_adapters=L, out=torch.full((T, H), 7.0,
                                                                   dtype=torch.bfloat16,
                                                                   device=gpu))
    fin = moe_finalize_lora(torch.empty((0, H), dtype=torch.bfloat16, device=gpu), act, perm,
                            wa, sa, wb, sb, ids, w, lora, r, H, num_adapters=L)
    torch.cuda.synchronize()
    assert not out.view(torch.int16).any(), "delta must be +0 rows"
    assert not fin.view(torch.int16).any(), "finalize must be +0 rows"


def test_routing_and_permuted_rows_with_no_tokens(gpu):
    print("empty: routing and permuted rows with T = 0", flush=True)
    ids = torch.empty((0, 8), dtype=torch.int32, device=gpu)
    m, perm = moe_route_permutation(ids, 16)
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=gpu)
    out = moe_permute_rows(x, perm, 8)
    # rows to write into but no token: the caller's rows stay as they were
    fill = synth.bf16_normal((5, 64), 1.0, synth.gen(4, gpu), gpu)
    kept = moe_permute_rows(x, perm, 8, out=fill.clone())
    torch.cuda.synchronize()
    assert m.tolist() == [0] * 17 and perm.numel() == 0 and out.shape == (0, 64)
    assert torch.equal(kept.view(torch.int16), fill.view(torch.int16))


def test_nvfp4_rejects_empty_shapes(gpu):
    """M = 0 has no output to write; the call refuses it with ValueError
    (M >= 1 is required) instead of launching anything."""
    print("empty: NVFP4 GEMM with M = 0 is refused", flush=True)
    k, n = 256, 256
    a = torch.empty((0, k // 2), dtype=torch.uint8, device=gpu)
    b = torch.zeros((n, k // 2), dtype=torch.uint8, device=gpu)
    sf_b = torch.zeros(synth.sf_buffer_bytes(n, k), dtype=torch.uint8, device=gpu)
    alpha = torch.ones(1, dtype=torch.float32, device=gpu)
    with pytest.raises(ValueError):
        mm_nvfp4_lora(a, b, torch.empty(0, dtype=torch.uint8, device=gpu), sf_b, alpha)
    torch.cuda.synchronize()
