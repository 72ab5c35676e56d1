"""GPU parity of the FC2 MoE LoRA delta against the fp64 oracle."""
import numpy as np
import pytest
import torch

import synth
from moe_expert_grouped_amd import bgmv_moe_gemm2_lora_delta
from oracle.formats import f64_to_bf16_bits
from oracle.lora_delta import moe_fc2_lora_delta
from tests.delta_helpers import ORACLE_DTYPE, contiguous_tables, oracle_bank, scattered_bank
from tests.parity import bits16, check_close, to_f64

pytestmark = pytest.mark.gpu


def to_dev(case, dev):
    return synth.DeltaCase(case.name, case.act.to(dev), case.perm.to(dev), case.A.to(dev),
                           case.B.to(dev), case.topk_ids.to(dev), case.topk_weights.to(dev),
                           case.lora_ids.to(dev), case.scale, case.extra)


def tables(case, scattered=False):
    """(flatA, w_ptr_a, stride_a, flatB, w_ptr_b, stride_b); banks on the case's device."""
    if scattered:
        fa, wa, sa = scattered_bank(case.A, seed=3)
        fb, wb, sb = scattered_bank(case.B, seed=4)
        return fa, wa, sa, fb, wb, sb
    wa, sa = contiguous_tables(case.A)
    wb, sb = contiguous_tables(case.B)
    return case.A, wa, sa, case.B, wb, sb


def run_gpu(case, tb, out_dtype=torch.bfloat16, **over):
    fa, wa, sa, fb, wb, sb = tb
    kw = dict(perm=case.perm, topk_ids=case.topk_ids, topk_weights=case.topk_weights,
              lora_ids=case.lora_ids, scale=case.scale)
    kw.update(over)
    dev = case.act.device
    out = bgmv_moe_gemm2_lora_delta(case.act, kw["perm"], wa.to(dev), sa, wb.to(dev), sb,
                                    kw["topk_ids"], kw["topk_weights"], kw["lora_ids"], case.rank,
                                    case.H, num_adapters=case.L, lora_dtype=case.act.dtype,
                                    scale=kw["scale"], out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out


def run_oracle(case, tb, tokens=None, **over):
    fa, wa, sa, fb, wb, sb = tb
    kw = dict(perm=case.perm, topk_ids=case.topk_ids, topk_weights=case.topk_weights,
              lora_ids=case.lora_ids, scale=case.scale)
    kw.update(over)
    c = lambda t: t.detach().cpu().numpy()
    return moe_fc2_lora_delta(bits16(case.act), c(kw["perm"]), oracle_bank(fa), c(wa), sa,
                              oracle_bank(fb), c(wb), sb, c(kw["topk_ids"]), c(kw["topk_weights"]),
                              c(kw["lora_ids"]), case.rank, case.H, kw["scale"], tokens=tokens,
                              lora_dtype=ORACLE_DTYPE[case.act.dtype])


def test_tiny(gpu):
    case = to_dev(synth.delta_tiny(), gpu)
    tb = tables(case)
    out = run_gpu(case, tb)
    check_close(to_f64(out), run_oracle(case, tb), "tiny delta")
    no = (case.lora_ids < 0).cpu().numpy()
    assert not bits16(out)[no].any(), "tokens without adapter must be +0"


@pytest.mark.parametrize("r,I,H", [(16, 64, 256), (8, 200, 128), (32, 96, 384), (24, 128, 256),
                                   (40, 64, 256), (48, 72, 128),
                                   # A_le held in LDS (rank <= 32, I % 128 == 0): the
                                   # shrink by (adapter, expert), up to its largest A_le
                                   (16, 256, 256), (8, 384, 128), (32, 1024, 128),
                                   # 64 to 128 KB of A_le: one workgroup per CU
                                   (16, 4096, 128), (32, 2048, 256), (8, 3968, 128)])
def test_integer_probe_bitwise_scattered_bank(gpu, r, I, H):
    case = to_dev(synth.delta_int_probe(r=r, I=I, H=H), gpu)
    tb = tables(case, scattered=True)
    out = run_gpu(case, tb)
    ref = run_oracle(case, tb)
    assert np.array_equal(bits16(out), f64_to_bf16_bits(ref))
    out32 = run_gpu(case, tb, torch.float32)
    assert np.array_equal(to_f64(out32), ref)


def test_all_inactive_and_no_adapter_give_plus_zero(gpu):
    case = to_dev(synth.delta_tiny(seed=3), gpu)
    tb = tables(case)
    z = run_gpu(case, tb, lora_ids=torch.full_like(case.lora_ids, -1))
    assert not bits16(z).any()
    z = run_gpu(case, tb, perm=torch.full_like(case.perm, -1))
    assert not bits16(z).any()


def test_out_of_range_ids_are_inactive(gpu):
    case = to_dev(synth.delta_int_probe(seed=105), gpu)
    tb = tables(case)
    lids = case.lora_ids.clone()
    lids[::3] = case.L + 2                      # adapter id past the bank
    perm = case.perm.clone()
    perm[1::5] = case.act.shape[0] + 10         # row past padded_rows
    out = run_gpu(case, tb, lora_ids=lids, perm=perm)
    ref = run_oracle(case, tb, lora_ids=torch.where(lids >= case.L, -1, lids),
                     perm=torch.where(perm >= case.act.shape[0], -1, perm))
    assert np.array_equal(bits16(out), f64_to_bf16_bits(ref))


def test_scale_doubling_is_exact(gpu):
    case = to_dev(synth.delta_tiny(seed=5), gpu)
    tb = tables(case)
    o1 = run_gpu(case, tb, torch.float32, scale=1.5)
    o2 = run_gpu(case, tb, torch.float32, scale=3.0)
    assert torch.equal(o1 * 2, o2)


def test_deterministic(gpu):
    case = to_dev(synth.delta_at_scale(T=1024, E=16, I=512, H=1024, L=4), gpu)
    tb = tables(case)
    o1 = run_gpu(case, tb)
    o2 = run_gpu(case, tb)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_medium_random(gpu):
    case = to_dev(synth.delta_at_scale(seed=9, T=512, top_k=4, E=12, I=256, H=512, L=3), gpu)
    tb = tables(case)
    out = run_gpu(case, tb)
    check_close(to_f64(out), run_oracle(case, tb), "medium delta")


@pytest.mark.slow
@pytest.mark.parametrize("lora_dtype", [torch.bfloat16, torch.float16])
def test_at_scale_sampled(gpu, lora_dtype):
    """T=8192, top_k=8, E=64, I=2048, H=4096, 8 adapters of rank 16 (the
    bench's launch), checked on sampled tokens (all columns)."""
    case = synth.delta_at_scale(device=gpu).cast(lora_dtype)
    tb = tables(case)
    out = run_gpu(case, tb)
    rng = np.random.default_rng(2)
    toks = np.sort(rng.choice(case.T, 48, replace=False)).tolist()
    ref = run_oracle(case, tb, tokens=toks)
    idx = torch.tensor(toks, device=gpu)
    check_close(to_f64(out.index_select(0, idx)), ref, "delta at scale (sampled tokens)")
    out2 = run_gpu(case, tb)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("lora_dtype", [torch.bfloat16, torch.float16])
def test_workspace_contents_do_not_matter(gpu, lora_dtype):
    """Every workspace byte the kernels read is written earlier in the same
    call: a workspace full of garbage gives the same bits as a zeroed one."""
    from moe_expert_grouped_amd import delta_workspace_bytes
    case = to_dev(synth.delta_int_probe(seed=107, r=24, I=128, H=256).cast(lora_dtype), gpu)
    tb = tables(case, scattered=True)
    fa, wa, sa, fb, wb, sb = tb
    nbytes = delta_workspace_bytes(case.T, case.topk_ids.shape[1], case.A.shape[1], case.L,
                                   case.rank)
    outs = []
    for fill in (0, 0xFF, 0x5A):
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device=gpu)
        outs.append(bgmv_moe_gemm2_lora_delta(case.act, case.perm, wa.to(gpu), sa, wb.to(gpu), sb,
                                              case.topk_ids, case.topk_weights, case.lora_ids,
                                              case.rank, case.H, num_adapters=case.L,
                                              lora_dtype=lora_dtype, scale=case.scale,
                                              workspace=ws))
    torch.cuda.synchronize()
    ref = run_oracle(case, tb)
    for o in outs:
        assert np.array_equal(bits16(o), f64_to_bf16_bits(ref))


@pytest.mark.parametrize("lora_dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("I", [64, 128])
def test_token_routed_twice_to_one_expert(gpu, lora_dtype, I):
    """Routing that repeats an expert for a token: both slots count (the
    formula sums over j); such tiles accumulate with LDS atomics."""
    case = synth.delta_int_probe(seed=109, T=40, top_k=4, E=6, I=I, H=256, L=2, r=16)
    ids = case.topk_ids.clone()
    ids[::3, 1] = ids[::3, 0]      # every third token: slot 1 repeats slot 0's expert
    ids[5, 2] = ids[5, 3] = ids[5, 0]
    case = to_dev(synth.DeltaCase(case.name, case.act, case.perm, case.A, case.B, ids,
                                  case.topk_weights, case.lora_ids, case.scale,
                                  case.extra).cast(lora_dtype), gpu)
    tb = tables(case, scattered=True)
    out = run_gpu(case, tb)
    ref = run_oracle(case, tb)
    assert np.array_equal(bits16(out), f64_to_bf16_bits(ref))
    out2 = run_gpu(case, tb)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


def test_fp16_output_integer_probe_bitwise(gpu):
    """out_dtype fp16 (the delta is added to an fp16 MoE output): the exact
    value rounded once to fp16."""
    from oracle.formats import f64_to_f16_bits
    case = to_dev(synth.delta_int_probe(seed=113, r=16, I=64, H=256), gpu)
    tb = tables(case, scattered=True)
    out = run_gpu(case, tb, torch.float16)
    assert np.array_equal(bits16(out), f64_to_f16_bits(run_oracle(case, tb)))


# ---------------------------------------------------------------------------
# lora_dtype fp16
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("r,I,H", [(16, 64, 256), (8, 200, 128), (40, 64, 256), (48, 72, 128),
                                   (64, 128, 256), (128, 64, 128), (16, 4096, 128)])
def test_fp16_lora_integer_probe_bitwise(gpu, r, I, H):
    """Activation and banks in fp16: every intermediate of the integer probe
    is exact, so each output type is the exact value rounded once."""
    from oracle.formats import f64_to_f16_bits
    case = to_dev(synth.delta_int_probe(seed=115, r=r, I=I, H=H).cast(torch.float16), gpu)
    tb = tables(case, scattered=True)
    ref = run_oracle(case, tb)
    assert np.array_equal(bits16(run_gpu(case, tb)), f64_to_bf16_bits(ref))
    assert np.array_equal(bits16(run_gpu(case, tb, torch.float16)), f64_to_f16_bits(ref))
    assert np.array_equal(to_f64(run_gpu(case, tb, torch.float32)), ref)


def test_fp16_lora_medium_random(gpu):
    case = to_dev(synth.delta_at_scale(seed=9, T=512, top_k=4, E=12, I=256, H=512,
                                       L=3).cast(torch.float16), gpu)
    tb = tables(case)
    check_close(to_f64(run_gpu(case, tb)), run_oracle(case, tb), "medium delta fp16")


@pytest.mark.parametrize("act_mul,a_mul", [(2.0 ** 10, 2.0 ** 7), (2.0 ** -7, 2.0 ** -8)])
def test_fp16_lora_far_from_one(gpu, act_mul, a_mul):
    """A @ act far from fp16's range: up to ~1.8e5 (past its largest finite
    value, 65504) or with a median of ~6.5e-6 (below its smallest normal,
    6.1e-5).  The per-slot power-of-two scaling keeps ~22 significant bits,
    so the fp32 output is within 1e-5 of the largest |delta|; fp16 hi + lo
    without it would overflow or lose the low part."""
    base = synth.delta_at_scale(seed=21, T=256, top_k=4, E=8, I=256, H=256, L=2)
    case = synth.DeltaCase(base.name, (base.act.float() * act_mul).half(), base.perm,
                           (base.A.float() * a_mul).half(), base.B.half(), base.topk_ids,
                           base.topk_weights, base.lora_ids, base.scale)
    case = to_dev(case, gpu)
    tb = tables(case)
    ref = run_oracle(case, tb)
    out = to_f64(run_gpu(case, tb, torch.float32))
    assert np.all(np.isfinite(out))
    err = np.abs(out - ref).max()
    assert err <= 1e-5 * np.abs(ref).max(), (err, np.abs(ref).max())
    check_close(to_f64(run_gpu(case, tb)), ref, "fp16 delta far from one")


@pytest.mark.parametrize("T,top_k,E,L,r,I,H", [
    (40, 32, 40, 3, 16, 64, 128),     # the largest top_k (tiles of 32 tokens)
    (64, 4, 512, 2, 8, 64, 128),      # the largest expert count
    (24, 3, 5, 2, 128, 64, 256),      # the largest rank (8 rank chunks of 16)
    (96, 2, 3, 40, 8, 128, 128),      # many adapters, few tokens each
    (16500, 2, 4, 2, 8, 64, 128),     # many tokens: 258 tiles over two adapters
])
def test_integer_probe_at_the_limits(gpu, T, top_k, E, L, r, I, H):
    """Every fp32 intermediate is exact, so the output is the exact delta
    rounded once, at the largest top_k, expert count and rank the entry
    point takes, and with many adapters."""
    case = to_dev(synth.delta_int_probe(seed=T + E + r, T=T, top_k=top_k, E=E, I=I, H=H, L=L,
                                        r=r), gpu)
    tb = tables(case, scattered=True)
    ref = run_oracle(case, tb)
    assert np.array_equal(bits16(run_gpu(case, tb)), f64_to_bf16_bits(ref))
    assert np.array_equal(to_f64(run_gpu(case, tb, torch.float32)), ref)
