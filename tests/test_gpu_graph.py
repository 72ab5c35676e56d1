"""The calls inside a captured HIP graph: no host read, no allocation and no
memset in the library, so a captured sequence replays the same kernels on
the same buffers.  Each test replays a graph several times, changing the
inputs in place between replays (eager work and synchronisations in between),
and checks every replay bitwise against the same calls made eagerly.

The NVFP4 prepared path pins the adapter-switch protocol the prepared-path
bullet of mm_nvfp4_lora describes: the in-place refold (no host read) and the
call, captured together, follow new lora_b / lora_scale values on replay."""
import pytest
import torch

import synth
from moe_expert_grouped_amd import (bgmv_moe_gemm2_lora_delta, delta_workspace_bytes,
                                    fill_w_ptr, finalize_workspace_bytes, grouped_mm_bf16,
                                    mm_nvfp4_lora, moe_finalize_lora, moe_permute_rows,
                                    moe_route_permutation, prepare_nvfp4_lora_adapter,
                                    route_workspace_bytes)

pytestmark = pytest.mark.gpu


def _same(x, y):
    return torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_prepared_adapter_switch_in_a_graph(gpu):
    print("graph: refold in place + NVFP4 prepared call, 4 replays", flush=True)
    c = synth.nvfp4_lora_case(seed=11, device=gpu, M=300, N=512, K=512, r=16)
    adapter = prepare_nvfp4_lora_adapter(c.lora_b, c.lora_scale, c.alpha)
    out = torch.empty((c.M, c.N), dtype=torch.bfloat16, device=gpu)

    def step():
        prepare_nvfp4_lora_adapter(c.lora_b, c.lora_scale, c.alpha, out=adapter)
        mm_nvfp4_lora(c.a, c.b, c.a_sf, c.b_sf, c.alpha, c.d, lora_adapter=adapter, bias=c.bias,
                      out=out)

    step()  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    g = synth.gen(12, gpu)
    for rnd, s in enumerate((0.5, 0.25, 0.0, 3.0)):
        c.lora_b.copy_(synth.bf16_normal(tuple(c.lora_b.shape), 0.02, g, gpu))
        c.lora_scale.fill_(s)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        # eager reference: a fresh adapter folded from the same values
        ref_ad = prepare_nvfp4_lora_adapter(c.lora_b, c.lora_scale, c.alpha)
        ref = mm_nvfp4_lora(c.a, c.b, c.a_sf, c.b_sf, c.alpha, c.d, lora_adapter=ref_ad,
                            bias=c.bias)
        torch.cuda.synchronize()
        assert _same(out, ref), f"replay {rnd} (lora_scale {s}) differs from the eager call"


def test_moe_fc2_sequence_in_a_graph(gpu):
    """Routing -> permuted rows -> FC2 grouped GEMM -> finalize with the delta,
    and the delta on its own, captured once and replayed with new activations,
    routing weights and routing."""
    print("graph: routing, permuted rows, grouped GEMM, finalize, delta; 3 replays", flush=True)
    T, k, E, I, H, L, r = 257, 4, 8, 256, 512, 3, 16
    g = synth.gen(21, gpu)
    ids = synth.routing_ids(seed=21, T=T, top_k=k, E=E, zipf_s=1.0).to(gpu)
    w = synth.softmax_weights(T, k, synth.gen(22)).to(gpu)
    lora_ids = torch.randint(-1, L, (T,), generator=synth.gen(23)).to(torch.int32).to(gpu)
    x = synth.bf16_normal((T, I), 1.0, g, gpu)
    w2 = synth.bf16_normal((E, H, I), I ** -0.5, g, gpu)
    A = synth.bf16_normal((L, E, r, I), 0.02, g, gpu)
    B = synth.bf16_normal((L, E, H, r), 0.02, g, gpu)
    wa, wb, sa, sb = fill_w_ptr(A), fill_w_ptr(B), E * r * I, E * H * r
    act = torch.empty((T * k, I), dtype=torch.bfloat16, device=gpu)
    fc2 = torch.empty((T * k, H), dtype=torch.bfloat16, device=gpu)
    fin = torch.empty((T, H), dtype=torch.bfloat16, device=gpu)
    dlt = torch.empty((T, H), dtype=torch.float32, device=gpu)
    rws = torch.empty(route_workspace_bytes(T * k, E), dtype=torch.uint8, device=gpu)
    fws = torch.empty(finalize_workspace_bytes(T, k, E, L, r, H), dtype=torch.uint8, device=gpu)
    dws = torch.empty(delta_workspace_bytes(T, k, E, L, r), dtype=torch.uint8, device=gpu)

    def step(into):
        m, perm = moe_route_permutation(ids, E, workspace=rws)
        moe_permute_rows(x, perm, k, out=into["act"])
        grouped_mm_bf16(into["act"], w2, m, out=into["fc2"])
        moe_finalize_lora(into["fc2"], into["act"], perm, wa, sa, wb, sb, ids, w, lora_ids, r, H,
                          num_adapters=L, scale=2.0, out=into["fin"], workspace=fws)
        bgmv_moe_gemm2_lora_delta(into["act"], perm, wa, sa, wb, sb, ids, w, lora_ids, r, H,
                                  num_adapters=L, scale=2.0, out_dtype=torch.float32,
                                  out=into["dlt"], workspace=dws)

    bufs = dict(act=act, fc2=fc2, fin=fin, dlt=dlt)
    step(bufs)  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(bufs)
    for rnd in range(3):
        x.copy_(synth.bf16_normal((T, I), 1.0, g, gpu))
        w.copy_(torch.rand((T, k), generator=g, device=gpu, dtype=torch.float32))
        ids.copy_(synth.routing_ids(seed=30 + rnd, T=T, top_k=k, E=E, zipf_s=0.5 * rnd).to(gpu))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = dict(act=torch.zeros_like(act), fc2=torch.zeros_like(fc2),
                   fin=torch.empty_like(fin), dlt=torch.empty_like(dlt))
        step(ref)
        torch.cuda.synchronize()
        for name in ("act", "fc2", "fin"):
            assert _same(bufs[name], ref[name]), f"replay {rnd}: {name} differs from eager"
        assert torch.equal(bufs["dlt"], ref["dlt"]), f"replay {rnd}: delta differs from eager"
