"""GPU parity of the routing permutation and the permuted rows against the
oracle: index work, so every comparison is bit-exact."""
import numpy as np
import pytest
import torch

import synth
from moe_expert_grouped_amd import (grouped_mm_bf16, moe_permute_rows, moe_route_permutation,
                                    route_workspace_bytes)
from oracle.permute import permute_rows, route_permutation

pytestmark = pytest.mark.gpu


def check_route(ids, E, gpu, with_inverse=True):
    print(f"route: T={ids.shape[0]} top_k={ids.shape[1]} E={E}", flush=True)
    got = moe_route_permutation(ids.to(gpu), E, with_inverse=with_inverse)
    torch.cuda.synchronize()
    ref = route_permutation(ids.numpy(), E)
    names = ("m_indptr", "expanded_idx_to_permuted_idx", "permuted_idx_to_expanded_idx")
    for name, g, r in zip(names, got, ref):
        g = g.cpu().numpy().astype(np.int64)
        assert g.shape == r.shape, name
        bad = np.nonzero(g != r)[0]
        assert bad.size == 0, f"{name}: {bad.size} mismatches, first at {bad[:5]}"
    return got


@pytest.mark.parametrize("T,k,E,invalid,zipf", [
    (1, 1, 1, 0.0, 0.0),          # one slot
    (37, 3, 5, 0.0, 0.0),         # one chunk, ragged
    (41, 4, 7, 0.2, 0.0),         # ids outside [0, E) left out
    (3000, 8, 64, 0.0, 0.0),      # 24 chunks with a ragged tail
    (3001, 7, 64, 0.05, 1.2),     # hot experts, empty experts, invalid ids
    (1500, 8, 1024, 0.01, 0.0),   # the largest expert count
    (2048, 4, 1, 0.3, 0.0),       # one expert
    (256, 16, 300, 0.0, 0.8),     # E not a power of two, repeats inside a token
])
def test_route_matches_oracle(gpu, T, k, E, invalid, zipf):
    ids = synth.routing_ids(seed=T + 7 * E, T=T, top_k=k, E=E, invalid_frac=invalid, zipf_s=zipf)
    check_route(ids, E, gpu)


def test_route_all_invalid_and_empty(gpu):
    ids = torch.full((100, 8), -1, dtype=torch.int32)
    m, perm, inv = check_route(ids, 16, gpu)
    assert int(m[-1]) == 0
    m, perm = moe_route_permutation(torch.empty((0, 8), dtype=torch.int32, device=gpu), 16)
    torch.cuda.synchronize()
    assert m.tolist() == [0] * 17 and perm.numel() == 0


def test_route_at_scale_and_without_inverse(gpu):
    """T=8192 tokens, top_k=8, E=64 (65536 slots), and 2^21 slots over 256 experts."""
    ids = synth.routing_ids(seed=21, T=8192, top_k=8, E=64)
    check_route(ids, 64, gpu)
    check_route(ids, 64, gpu, with_inverse=False)
    big = synth.routing_ids(seed=22, T=262144, top_k=8, E=256, invalid_frac=0.01, zipf_s=1.0)
    check_route(big, 256, gpu)


def test_route_workspace_is_reused_without_clearing(gpu):
    ids = synth.routing_ids(seed=23, T=4000, top_k=8, E=128, zipf_s=1.1)
    ws = torch.full((route_workspace_bytes(32000, 128),), 0x5A, dtype=torch.uint8, device=gpu)
    a = moe_route_permutation(ids.to(gpu), 128, with_inverse=True, workspace=ws)
    b = moe_route_permutation(ids.to(gpu), 128, with_inverse=True, workspace=ws)
    torch.cuda.synchronize()
    ref = route_permutation(ids.numpy(), 128)
    for g1, g2, r in zip(a, b, ref):
        assert np.array_equal(g1.cpu().numpy(), r) and np.array_equal(g2.cpu().numpy(), r)


@pytest.mark.parametrize("T,k,row_bytes,out_rows", [
    (13, 3, 16, None),       # the smallest row
    (29, 4, 48, 100),        # out_rows past the routed rows
    (64, 8, 8192, 300),      # bf16 rows of 4096, some slots past out_rows
    (33, 2, 8192 + 4112, None),  # a row that is not a multiple of the wave's piece
])
def test_permute_rows_bitwise(gpu, T, k, row_bytes, out_rows):
    print(f"permute_rows: T={T} top_k={k} row_bytes={row_bytes} out_rows={out_rows}", flush=True)
    E = 6
    ids = synth.routing_ids(seed=T * k, T=T, top_k=k, E=E, invalid_frac=0.1)
    _, perm, _ = route_permutation(ids.numpy(), E)
    rows = T * k if out_rows is None else out_rows
    g = synth.gen(T)
    x = torch.randint(0, 256, (T, row_bytes), generator=g, dtype=torch.uint8)
    fill = torch.randint(0, 256, (rows, row_bytes), generator=g, dtype=torch.uint8)
    out = fill.clone().to(gpu)
    moe_permute_rows(x.to(gpu), torch.from_numpy(perm).to(torch.int32).to(gpu), k, out=out)
    torch.cuda.synchronize()
    ref = permute_rows(x.numpy(), perm, k, fill.numpy().copy())
    assert np.array_equal(out.cpu().numpy(), ref)


def test_permute_rows_tokens_past_the_grid(gpu):
    """More tokens than the launch has wavefronts (they stride), bf16 rows."""
    T, k, H = 40000, 2, 64
    ids = synth.routing_ids(seed=31, T=T, top_k=k, E=8)
    m, perm = moe_route_permutation(ids.to(gpu), 8)
    x = synth.bf16_normal((T, H), 1.0, synth.gen(32, gpu), gpu)
    out = moe_permute_rows(x, perm, k)
    torch.cuda.synchronize()
    p = perm.cpu().numpy()
    ref = permute_rows(x.view(torch.int16).cpu().numpy(), p, k,
                       np.zeros((T * k, H), dtype=np.int16))
    assert np.array_equal(out.view(torch.int16).cpu().numpy(), ref)


def test_route_then_grouped_gemm(gpu):
    """Routing output -> permuted rows -> grouped GEMM: each permuted row is
    its token's row times its expert's weight (a property at any size)."""
    T, k, E, K, N = 300, 4, 8, 128, 256
    ids = synth.routing_ids(seed=41, T=T, top_k=k, E=E, zipf_s=1.0)
    m, perm = moe_route_permutation(ids.to(gpu), E)
    g = synth.gen(42, gpu)
    x = synth.bf16_ints((T, K), -2, 2, g, gpu)
    w = synth.bf16_ints((E, N, K), -2, 2, g, gpu)
    a = moe_permute_rows(x, perm, k)
    y = grouped_mm_bf16(a, w, m, out_dtype=torch.float32)
    torch.cuda.synchronize()
    p = perm.cpu().long().view(T, k)
    xs, ws = x.float().cpu(), w.float().cpu()
    for t in range(0, T, 7):
        for j in range(k):
            e = int(ids[t, j])
            assert torch.equal(y[p[t, j]].cpu(), ws[e] @ xs[t]), (t, j)


def test_route_top1_many_experts_and_long_lists(gpu):
    """top_k = 1 over the largest expert count, and one hot expert taking
    most of 2^20 slots (long runs inside every chunk)."""
    ids = synth.routing_ids(seed=51, T=20000, top_k=1, E=1024, invalid_frac=0.02)
    check_route(ids, 1024, gpu)
    hot = synth.routing_ids(seed=52, T=131072, top_k=8, E=16, zipf_s=3.0)
    check_route(hot, 16, gpu)
