"""Pins of the LoRA-delta oracle (no GPU): literal loops, an exact integer
probe, invariants, a two-GEMM special case and the pointer semantics."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle.lora_delta import moe_fc2_lora_delta
from tests.delta_helpers import ORACLE_DTYPE, contiguous_tables, oracle_bank, scattered_bank
from tests.parity import bits16


def run_oracle(case, A=None, B=None, tables=None, **over):
    A = case.A if A is None else A
    B = case.B if B is None else B
    if tables is None:
        wa, sa = contiguous_tables(A)
        wb, sb = contiguous_tables(B)
        ba, bb = oracle_bank(A), oracle_bank(B)
    else:
        (ba, wa, sa), (bb, wb, sb) = tables
    kw = dict(perm=case.perm.numpy(), topk_ids=case.topk_ids.numpy(),
              topk_weights=case.topk_weights.numpy(), lora_ids=case.lora_ids.numpy(),
              scale=case.scale)
    kw.update(over)
    return moe_fc2_lora_delta(bits16(case.act), kw["perm"], ba, wa.numpy(), sa, bb, wb.numpy(),
                              sb, kw["topk_ids"], kw["topk_weights"], kw["lora_ids"],
                              case.rank, case.H, kw["scale"],
                              lora_dtype=ORACLE_DTYPE[case.act.dtype])


def decode(t: torch.Tensor) -> np.ndarray:
    """float64 values of a bf16 tensor (oracle decoder) or an fp16 tensor
    (numpy's own IEEE half decoder, independent of the oracle's)."""
    if t.dtype == torch.float16:
        return bits16(t).view(np.float16).astype(np.float64)
    return F.bf16_to_f64(bits16(t))


def literal_loops(case):
    """The formula with plain Python floats and explicit index loops."""
    act = decode(case.act)
    A = decode(case.A)
    B = decode(case.B)
    T, k = case.topk_ids.shape
    out = [[0.0] * case.H for _ in range(T)]
    for t in range(T):
        l = int(case.lora_ids[t])
        if l < 0:
            continue
        for j in range(k):
            p = int(case.perm[t * k + j])
            if p < 0:
                continue
            e = int(case.topk_ids[t, j])
            w = float(case.topk_weights[t, j])
            u = [sum(A[l, e, r, i] * act[p, i] for i in range(case.I)) for r in range(case.rank)]
            for h in range(case.H):
                out[t][h] += case.scale * w * sum(B[l, e, h, r] * u[r] for r in range(case.rank))
    return np.array(out)


def small_case(seed=7):
    g = synth.gen(seed)
    T, k, E, I, H, L, r = 6, 2, 3, 8, 12, 2, 4
    topk = synth.inputs.distinct_topk(T, E, k, g)
    w = synth.inputs.softmax_weights(T, k, g)
    perm, _ = synth.route(topk, E, g, 0.25)
    return synth.DeltaCase("small", synth.bf16_normal((T * k, I), 1.0, g), perm,
                           synth.bf16_normal((L, E, r, I), 0.3, g),
                           synth.bf16_normal((L, E, H, r), 0.3, g), topk, w,
                           torch.tensor([0, -1, 1, 1, 0, 1], dtype=torch.int32), 1.5)


def test_literal_loops():
    case = small_case()
    ours = run_oracle(case)
    ref = literal_loops(case)
    assert np.allclose(ours, ref, rtol=1e-12, atol=1e-14)
    assert not ours[1].any()          # token 1 has no adapter


def test_fp16_lora_dtype_literal_loops():
    """lora_dtype fp16: activation and banks decode as IEEE half.  The case's
    values are not all representable in bf16, so decoding them as bf16 fails."""
    case = small_case(12).cast(torch.float16)
    g = torch.Generator().manual_seed(3)
    case.act += torch.randn(case.act.shape, generator=g).half() * 1e-3
    assert not torch.equal(case.act.bfloat16().half(), case.act)
    ours = run_oracle(case)
    assert np.allclose(ours, literal_loops(case), rtol=1e-12, atol=1e-14)
    # the same bits read as bf16 give other numbers (the pin can fail)
    ba, bb = oracle_bank(case.A), oracle_bank(case.B)
    ba.dtype = bb.dtype = "bf16"
    (wa, sa), (wb, sb) = contiguous_tables(case.A), contiguous_tables(case.B)
    wrong = moe_fc2_lora_delta(bits16(case.act), case.perm.numpy(), ba, wa.numpy(), sa, bb,
                               wb.numpy(), sb, case.topk_ids.numpy(), case.topk_weights.numpy(),
                               case.lora_ids.numpy(), case.rank, case.H, case.scale)
    assert not np.allclose(wrong, ours)
    with pytest.raises(AssertionError):  # banks and activation must agree on the dtype
        run_oracle(case, tables=((ba, wa, sa), (oracle_bank(case.B), wb, sb)))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_integer_probe_exact_with_fractions(dtype):
    case = synth.delta_int_probe(T=8, top_k=3, E=4, I=16, H=8, L=3, r=4, pad_rows=5).cast(dtype)
    ours = run_oracle(case)
    act = case.act.to(torch.int64).numpy()
    A = case.A.to(torch.int64).numpy()
    B = case.B.to(torch.int64).numpy()
    for t in range(case.T):
        l = int(case.lora_ids[t])
        for h in range(case.H):
            s = Fraction(0)
            if l >= 0:
                for j in range(case.top_k):
                    p = int(case.perm[t * case.top_k + j])
                    if p < 0:
                        continue
                    e = int(case.topk_ids[t, j])
                    w = Fraction(float(case.topk_weights[t, j]))
                    u = [int(np.dot(A[l, e, r], act[p])) for r in range(case.rank)]
                    s += w * sum(int(B[l, e, h, r]) * u[r] for r in range(case.rank))
            assert ours[t, h] == float(Fraction(case.scale) * s)


def test_no_adapter_and_no_active_slot_give_zero():
    case = small_case(8)
    z = run_oracle(case, lora_ids=np.full(case.T, -1))
    assert not z.any()
    z = run_oracle(case, perm=np.full(case.T * case.top_k, -1))
    assert not z.any()


def test_scale_is_linear():
    case = small_case(9)
    one = run_oracle(case, scale=1.25)
    two = run_oracle(case, scale=2.5)
    assert np.array_equal(2 * one, two)


def test_single_expert_single_slot_is_two_gemm_chain():
    g = synth.gen(10)
    T, I, H, r = 7, 16, 10, 4
    case = synth.DeltaCase("chain", synth.bf16_normal((T, I), 1.0, g), torch.arange(T).int(),
                           synth.bf16_normal((1, 1, r, I), 0.5, g),
                           synth.bf16_normal((1, 1, H, r), 0.5, g),
                           torch.zeros(T, 1, dtype=torch.int32),
                           torch.rand(T, 1, generator=g), torch.zeros(T, dtype=torch.int32), 0.75)
    act = F.bf16_to_f64(bits16(case.act))
    A = F.bf16_to_f64(bits16(case.A))[0, 0]
    B = F.bf16_to_f64(bits16(case.B))[0, 0]
    w = case.topk_weights.numpy().astype(np.float64)
    ref = 0.75 * w * np.matmul(np.matmul(act, A.T), B.T)
    assert np.allclose(run_oracle(case), ref, rtol=1e-12, atol=1e-14)


def test_pointer_table_and_stride_semantics():
    case = small_case(11)
    flat_a, wa, sa = scattered_bank(case.A, seed=1)
    flat_b, wb, sb = scattered_bank(case.B, seed=2)
    tables = ((oracle_bank(flat_a), wa, sa), (oracle_bank(flat_b), wb, sb))
    assert np.array_equal(run_oracle(case, tables=tables), run_oracle(case))


def test_token_subset_equals_rows_of_the_whole():
    """The ``tokens=`` path (what the at-scale GPU tests sample through) gives
    the rows of the all-token result and of the literal loops, in the order
    asked, repeats and tokens without adapter included."""
    case = small_case(13)
    full = run_oracle(case)
    lit = literal_loops(case)
    S = [5, 0, 3, 3, 1]
    (wa, sa), (wb, sb) = contiguous_tables(case.A), contiguous_tables(case.B)
    sub = moe_fc2_lora_delta(bits16(case.act), case.perm.numpy(), oracle_bank(case.A), wa.numpy(),
                             sa, oracle_bank(case.B), wb.numpy(), sb, case.topk_ids.numpy(),
                             case.topk_weights.numpy(), case.lora_ids.numpy(), case.rank, case.H,
                             case.scale, tokens=S)
    assert sub.shape == (len(S), case.H)
    assert np.array_equal(sub, full[S])
    assert np.allclose(sub, lit[S], rtol=1e-12, atol=1e-14)
    assert not sub[4].any()  # token 1 has no adapter
