"""Pins of the FC1 LoRA-delta oracle (no GPU): literal loops, an exact
integer probe, the FC2 delta oracle at top_k 1 with unit weights, the
two-GEMM chain, zero and not-written rows, and the pointer semantics.

The cases reuse the FC2 delta's case type: ``act`` is the permuted FC1 input
``[padded_rows, hidden]`` (the case's ``I``), ``B`` is ``[L, E, 2I, r]`` (the
case's ``H`` = out_features); the routing weights are not used."""
from fractions import Fraction

import numpy as np
import torch

import synth
from oracle import formats as F
from oracle.fc1_lora_delta import moe_fc1_lora_delta
from oracle.lora_delta import moe_fc2_lora_delta
from tests.delta_helpers import ORACLE_DTYPE, contiguous_tables, oracle_bank, scattered_bank
from tests.parity import bits16


def run(case, tables=None, rows=None, **over):
    if tables is None:
        wa, sa = contiguous_tables(case.A)
        wb, sb = contiguous_tables(case.B)
        tables = ((oracle_bank(case.A), wa, sa), (oracle_bank(case.B), wb, sb))
    (ba, wa, sa), (bb, wb, sb) = tables
    kw = dict(perm=case.perm.numpy(), topk_ids=case.topk_ids.numpy(),
              lora_ids=case.lora_ids.numpy(), scale=case.scale)
    kw.update(over)
    return moe_fc1_lora_delta(bits16(case.act), kw["perm"], ba, wa.numpy(), sa, bb, wb.numpy(), sb,
                              kw["topk_ids"], kw["lora_ids"], case.rank, case.H, kw["scale"],
                              case.E, rows=rows, lora_dtype=ORACLE_DTYPE[case.act.dtype])


def small_case(seed=7, T=6, k=2, E=3, hidden=8, out=12, L=2, r=4, pad=3):
    g = synth.gen(seed)
    topk = synth.inputs.distinct_topk(T, E, k, g)
    n = T * k
    perm = torch.randperm(n + pad, generator=g)[:n].to(torch.int32)
    perm[[1, 6]] = -1
    return synth.DeltaCase("fc1-small", synth.bf16_normal((n + pad, hidden), 1.0, g), perm,
                           synth.bf16_normal((L, E, r, hidden), 0.3, g),
                           synth.bf16_normal((L, E, out, r), 0.3, g), topk,
                           torch.ones(T, k), torch.tensor([0, -1, 1, 1, 0, 1], dtype=torch.int32),
                           1.5)


def literal(case):
    act = F.bf16_to_f64(bits16(case.act))
    A = F.bf16_to_f64(bits16(case.A))
    B = F.bf16_to_f64(bits16(case.B))
    rows = act.shape[0]
    out = [[0.0] * case.H for _ in range(rows)]
    wr = [False] * rows
    T, k = case.topk_ids.shape
    for t in range(T):
        l = int(case.lora_ids[t])
        for j in range(k):
            p = int(case.perm[t * k + j])
            if p < 0:
                continue
            wr[p] = True
            if l < 0:
                continue
            e = int(case.topk_ids[t, j])
            u = [sum(A[l, e, q, i] * act[p, i] for i in range(case.I)) for q in range(case.rank)]
            for h in range(case.H):
                out[p][h] = case.scale * sum(B[l, e, h, q] * u[q] for q in range(case.rank))
    return np.array(out), np.array(wr)


def test_literal_loops_and_rows_written():
    case = small_case()
    ours, wr = run(case)
    ref, wr_ref = literal(case)
    assert np.array_equal(wr, wr_ref)
    assert wr.sum() == 10 and not wr[[i for i in range(15) if i not in case.perm.tolist()]].any()
    assert np.allclose(ours, ref, rtol=1e-12, atol=1e-14)
    p_none = case.perm[2:4]  # token 1 has no adapter: its rows are written as +0
    assert not ours[p_none[p_none >= 0].long().numpy()].any()


def test_integer_probe_exact_with_fractions():
    case = synth.delta_int_probe(T=8, top_k=3, E=4, I=16, H=8, L=3, r=4, pad_rows=5)
    ours, wr = run(case)
    act = case.act.to(torch.int64).numpy()
    A = case.A.to(torch.int64).numpy()
    B = case.B.to(torch.int64).numpy()
    for t in range(case.T):
        l = int(case.lora_ids[t])
        for j in range(case.top_k):
            p = int(case.perm[t * case.top_k + j])
            if p < 0:
                continue
            assert wr[p]
            e = int(case.topk_ids[t, j])
            for h in range(case.H):
                want = Fraction(0)
                if l >= 0:
                    u = [int(np.dot(A[l, e, q], act[p])) for q in range(case.rank)]
                    want = Fraction(case.scale) * sum(int(B[l, e, h, q]) * u[q]
                                                      for q in range(case.rank))
                assert ours[p, h] == float(want)


def test_top1_unit_weights_equals_the_fc2_delta():
    """With top_k 1 and unit weights the FC2 formula has one slot per token,
    so its delta row t is the FC1 delta row perm[t] (the FC2 oracle is pinned
    on its own)."""
    g = synth.gen(12)
    T, E, hidden, out, L, r = 9, 3, 16, 8, 2, 4
    topk = torch.randint(0, E, (T, 1), generator=g).to(torch.int32)
    perm = torch.randperm(T + 2, generator=g)[:T].to(torch.int32)
    perm[4] = -1
    case = synth.DeltaCase("top1", synth.bf16_normal((T + 2, hidden), 1.0, g), perm,
                           synth.bf16_normal((L, E, r, hidden), 0.3, g),
                           synth.bf16_normal((L, E, out, r), 0.3, g), topk, torch.ones(T, 1),
                           torch.randint(-1, L, (T,), generator=g).to(torch.int32), 0.75)
    fc1, wr = run(case)
    (wa, sa), (wb, sb) = contiguous_tables(case.A), contiguous_tables(case.B)
    fc2 = moe_fc2_lora_delta(bits16(case.act), perm.numpy(), oracle_bank(case.A), wa.numpy(), sa,
                             oracle_bank(case.B), wb.numpy(), sb, topk.numpy(),
                             np.ones((T, 1), np.float32), case.lora_ids.numpy(), r, out, 0.75)
    for t in range(T):
        p = int(perm[t])
        if p >= 0:
            assert wr[p] and np.array_equal(fc1[p], fc2[t])
        else:
            assert not fc2[t].any()


def test_single_expert_is_the_two_gemm_chain():
    g = synth.gen(10)
    n, hidden, out, r = 7, 16, 10, 4
    case = synth.DeltaCase("chain", synth.bf16_normal((n, hidden), 1.0, g),
                           torch.arange(n).int(), synth.bf16_normal((1, 1, r, hidden), 0.5, g),
                           synth.bf16_normal((1, 1, out, r), 0.5, g),
                           torch.zeros(n, 1, dtype=torch.int32), torch.ones(n, 1),
                           torch.zeros(n, dtype=torch.int32), 0.75)
    x = F.bf16_to_f64(bits16(case.act))
    A = F.bf16_to_f64(bits16(case.A))[0, 0]
    B = F.bf16_to_f64(bits16(case.B))[0, 0]
    ours, wr = run(case)
    assert wr.all()
    assert np.allclose(ours, 0.75 * np.matmul(np.matmul(x, A.T), B.T), rtol=1e-12, atol=1e-14)


def test_zero_cases_and_out_of_range_experts():
    case = small_case(8)
    z, wr = run(case, lora_ids=np.full(case.T, -1))
    assert not z.any() and wr.sum() == 10
    z, wr = run(case, perm=np.full(case.T * case.top_k, -1))
    assert not z.any() and not wr.any()
    ids = case.topk_ids.numpy().copy()
    ids[2, 0] = case.E  # token 2 (adapter 1), slot 0: expert outside [0, E)
    out, wr = run(case, topk_ids=ids)
    p = int(case.perm[2 * case.top_k])
    full, _ = run(case)
    assert wr[p] and not out[p].any() and full[p].any()
    others = [i for i in range(out.shape[0]) if i != p]
    assert np.array_equal(out[others], full[others])


def test_row_subset_and_pointer_semantics():
    case = small_case(11)
    full, wr = run(case)
    rows = [5, 0, 14, 3]
    sub, swr = run(case, rows=rows)
    assert np.array_equal(sub, full[rows]) and np.array_equal(swr, wr[rows])
    flat_a, wa, sa = scattered_bank(case.A, seed=1)
    flat_b, wb, sb = scattered_bank(case.B, seed=2)
    tables = ((oracle_bank(flat_a), wa, sa), (oracle_bank(flat_b), wb, sb))
    scat, _ = run(case, tables=tables)
    assert np.array_equal(scat, full)
