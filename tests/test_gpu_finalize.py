"""GPU parity of the MoE finalize with the FC2 LoRA delta added, against the
fp64 oracle (combine of the FC2 rows + the exact delta)."""
import numpy as np
import pytest
import torch

import synth
from moe_expert_grouped_amd import (bgmv_moe_gemm2_lora_delta, delta_workspace_bytes,
                                    moe_finalize_lora)
from oracle.finalize import moe_finalize
from oracle.formats import f64_to_bf16_bits, f64_to_f16_bits
from tests.parity import bits16, check_close, to_f64
from tests.test_gpu_delta import run_oracle, tables, to_dev

pytestmark = pytest.mark.gpu

ORACLE_ROWS = {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}


def fc2_host(fc2):
    """The oracle's view of the FC2 rows: 16-bit patterns or float32 values."""
    if fc2.dtype == torch.float32:
        return fc2.cpu().numpy()
    return bits16(fc2)


def run_fin(case, tb, fc2, out_dtype=torch.bfloat16, fused=False, **over):
    """The finalize; ``fused`` gives it only the delta's workspace, which
    selects the single-pass path (the default workspace selects two passes)."""
    fa, wa, sa, fb, wb, sb = tb
    kw = dict(perm=case.perm, lora_ids=case.lora_ids, scale=case.scale, num_adapters=case.L)
    kw.update(over)
    dev = case.act.device
    ws = None
    if fused:
        ws = torch.empty(delta_workspace_bytes(case.T, case.top_k, case.E, kw["num_adapters"],
                                               case.rank), dtype=torch.uint8, device=dev)
    out = moe_finalize_lora(fc2, case.act, kw["perm"], wa.to(dev), sa, wb.to(dev), sb,
                            case.topk_ids, case.topk_weights, kw["lora_ids"], case.rank, case.H,
                            num_adapters=kw["num_adapters"], lora_dtype=case.act.dtype,
                            scale=kw["scale"], out_dtype=out_dtype, workspace=ws)
    torch.cuda.synchronize()
    return out


def oracle_fin(case, tb, fc2, tokens=None, **over):
    kw = dict(perm=case.perm, lora_ids=case.lora_ids)
    kw.update(over)
    # rows past padded_rows are not routed here: the delta oracle knows such
    # slots by a negative row (the finalize oracle checks both bounds itself)
    rows = case.act.shape[0]
    delta = run_oracle(case, tb, tokens=tokens, lora_ids=kw["lora_ids"],
                       perm=torch.where(kw["perm"] >= rows, -1, kw["perm"]))
    return moe_finalize(fc2_host(fc2), ORACLE_ROWS[fc2.dtype], kw["perm"].cpu().numpy(),
                        case.topk_weights.cpu().numpy(), delta, tokens=tokens)


def int_case(seed, fc2_dtype, r=16, I=128, H=256):
    case = to_dev(synth.delta_int_probe(seed=seed, r=r, I=I, H=H), "cuda")
    g = synth.gen(seed + 1)
    fc2 = synth.bf16_ints((case.act.shape[0], H), -3, 3, g).to(fc2_dtype).cuda()
    return case, fc2


@pytest.mark.parametrize("fc2_dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("r,I", [(16, 128), (24, 64)])
def test_integer_probe_bitwise(gpu, fc2_dtype, r, I):
    """Small integers, weights in quarters: every partial sum is exact, so
    each output type is the exact value rounded once (both shrink paths)."""
    case, fc2 = int_case(201, fc2_dtype, r=r, I=I)
    tb = tables(case, scattered=True)
    ref = oracle_fin(case, tb, fc2)
    for fused in (False, True):  # two passes, and the single-pass write-out
        assert np.array_equal(bits16(run_fin(case, tb, fc2, fused=fused)), f64_to_bf16_bits(ref))
        assert np.array_equal(bits16(run_fin(case, tb, fc2, torch.float16, fused=fused)),
                              f64_to_f16_bits(ref))
        assert np.array_equal(to_f64(run_fin(case, tb, fc2, torch.float32, fused=fused)), ref)


def test_no_adapters_is_the_plain_combine(gpu):
    case, fc2 = int_case(203, torch.bfloat16)
    tb = tables(case)
    none = torch.full_like(case.lora_ids, -1)
    ref = oracle_fin(case, tb, fc2, lora_ids=none)
    assert np.array_equal(bits16(run_fin(case, tb, fc2, lora_ids=none)), f64_to_bf16_bits(ref))
    # num_adapters == 0: every token is a token without adapter
    out = run_fin(case, tb, fc2, num_adapters=0)
    assert np.array_equal(bits16(out), f64_to_bf16_bits(ref))


def test_slots_past_padded_rows_are_skipped(gpu):
    case, fc2 = int_case(205, torch.float32)
    tb = tables(case)
    perm = case.perm.clone()
    perm[2::7] = case.act.shape[0] + 3
    ref = oracle_fin(case, tb, fc2, perm=perm)
    assert np.array_equal(to_f64(run_fin(case, tb, fc2, torch.float32, perm=perm)), ref)


def test_random_and_equal_to_delta_plus_combine(gpu):
    case = to_dev(synth.delta_at_scale(seed=11, T=512, top_k=4, E=12, I=256, H=512, L=3), gpu)
    g = synth.gen(12, gpu)
    fc2 = synth.bf16_normal((case.act.shape[0], case.H), 1.0, g, gpu)
    tb = tables(case)
    out = run_fin(case, tb, fc2)
    ref = oracle_fin(case, tb, fc2)
    check_close(to_f64(out), ref, "finalize medium")
    # the two paths do the same arithmetic in the same order: bitwise equal
    for dt, it in ((torch.bfloat16, torch.int16), (torch.float32, torch.int32)):
        two = run_fin(case, tb, fc2, dt).view(it)
        one = run_fin(case, tb, fc2, dt, fused=True).view(it)
        assert torch.equal(two, one), f"two-pass and single-pass finalize differ ({dt})"
    # the unfused composition: delta (fp32) + the combine in torch (fp32)
    fa, wa, sa, fb, wb, sb = tb
    delta = bgmv_moe_gemm2_lora_delta(case.act, case.perm, wa.to(gpu), sa, wb.to(gpu), sb,
                                      case.topk_ids, case.topk_weights, case.lora_ids, case.rank,
                                      case.H, num_adapters=case.L, scale=case.scale,
                                      out_dtype=torch.float32)
    p = case.perm.view(case.T, case.top_k).long()
    ok = (p >= 0) & (p < case.act.shape[0])
    rows = fc2.float()[p.clamp(min=0)] * (case.topk_weights * ok)[..., None]
    check_close(to_f64(out), (delta + rows.sum(1)).double().cpu().numpy(), "fused vs unfused")


@pytest.mark.slow
def test_at_scale_sampled(gpu):
    """T=8192, top_k=8, E=64, I=2048, H=4096, 8 adapters of rank 16, FC2 rows
    bf16 [65536, 4096]; sampled tokens, all columns."""
    case = synth.delta_at_scale(device=gpu)
    g = synth.gen(13, gpu)
    fc2 = synth.bf16_normal((case.act.shape[0], case.H), 1.0, g, gpu)
    tb = tables(case)
    out = run_fin(case, tb, fc2)
    toks = np.sort(np.random.default_rng(3).choice(case.T, 32, replace=False)).tolist()
    ref = oracle_fin(case, tb, fc2, tokens=toks)
    idx = torch.tensor(toks, device=gpu)
    check_close(to_f64(out.index_select(0, idx)), ref, "finalize at scale (sampled tokens)")
