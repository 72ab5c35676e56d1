"""GPU parity of the FC1 (gate/up) LoRA delta against the fp64 oracle: the
exact integer probe bitwise (every output type, both lora dtypes, a
scattered pointer table), random operands within the tolerance over the
rank variants and both shrink paths, the rows that must be +0 or untouched,
and the full-size routing on sampled rows.

Cases reuse the FC2 delta's case type: ``act`` is the permuted FC1 input
``[padded_rows, hidden]`` (the case's ``I``) and ``B`` is ``[L, E, out, r]``
(the case's ``H`` is the output width)."""
import numpy as np
import pytest
import torch

import synth
from moe_expert_grouped_amd import fill_w_ptr, moe_fc1_lora_delta
from oracle.fc1_lora_delta import moe_fc1_lora_delta as oracle_fc1
from oracle.formats import f64_to_bf16_bits, f64_to_f16_bits
from tests.delta_helpers import ORACLE_DTYPE, contiguous_tables, oracle_bank, scattered_bank
from tests.parity import bits16, check_close, to_f64

pytestmark = pytest.mark.gpu

SENTINEL = -7.0


def to_dev(case, dev):
    return synth.DeltaCase(case.name, case.act.to(dev), case.perm.to(dev), case.A.to(dev),
                           case.B.to(dev), case.topk_ids.to(dev), case.topk_weights.to(dev),
                           case.lora_ids.to(dev), case.scale, case.extra)


def tables(case, scattered=False):
    if scattered:
        fa, wa, sa = scattered_bank(case.A, seed=5)
        fb, wb, sb = scattered_bank(case.B, seed=6)
        return fa, wa, sa, fb, wb, sb
    wa, sa = contiguous_tables(case.A)
    wb, sb = contiguous_tables(case.B)
    return case.A, wa, sa, case.B, wb, sb


def run_gpu(case, tb, out_dtype=torch.bfloat16, **over):
    fa, wa, sa, fb, wb, sb = tb
    kw = dict(perm=case.perm, topk_ids=case.topk_ids, lora_ids=case.lora_ids, scale=case.scale,
              L=case.L)
    kw.update(over)
    dev = case.act.device
    out = torch.full((case.act.shape[0], case.H), SENTINEL, dtype=out_dtype, device=dev)
    print(f"moe_fc1_lora_delta: {case.name} out={out_dtype}", flush=True)
    moe_fc1_lora_delta(case.act, kw["perm"], wa.to(dev), sa, wb.to(dev), sb, kw["topk_ids"],
                       kw["lora_ids"], case.rank, case.H, num_adapters=kw["L"],
                       lora_dtype=case.act.dtype, scale=kw["scale"], out_dtype=out_dtype, out=out)
    torch.cuda.synchronize()
    return out


def run_oracle(case, tb, rows=None, **over):
    fa, wa, sa, fb, wb, sb = tb
    kw = dict(perm=case.perm, topk_ids=case.topk_ids, lora_ids=case.lora_ids, scale=case.scale)
    kw.update(over)
    c = lambda t: t.detach().cpu().numpy() if isinstance(t, torch.Tensor) else np.asarray(t)
    return oracle_fc1(bits16(case.act), c(kw["perm"]), oracle_bank(fa), c(wa), sa,
                      oracle_bank(fb), c(wb), sb, c(kw["topk_ids"]), c(kw["lora_ids"]), case.rank,
                      case.H, kw["scale"], case.E, rows=rows,
                      lora_dtype=ORACLE_DTYPE[case.act.dtype])


def check_untouched(out, written):
    assert np.all(to_f64(out)[~written] == SENTINEL)


@pytest.mark.parametrize("lora_dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("scattered", [False, True])
def test_integer_probe_bitwise(gpu, lora_dtype, scattered):
    """Small integers: every product and sum is exact, so each output type is
    the exact value rounded once."""
    case = to_dev(synth.delta_int_probe(T=40, top_k=3, E=5, I=64, H=256, L=3, r=16,
                                        pad_rows=9).cast(lora_dtype), gpu)
    tb = tables(case, scattered)
    ref, wr = run_oracle(case, tb)
    assert wr.sum() > 0 and (~wr).sum() > 0
    for odt, enc in [(torch.bfloat16, f64_to_bf16_bits), (torch.float16, f64_to_f16_bits)]:
        out = run_gpu(case, tb, odt)
        assert np.array_equal(bits16(out)[wr], enc(ref[wr])), odt
        check_untouched(out, wr)
    out = run_gpu(case, tb, torch.float32)
    assert np.array_equal(to_f64(out)[wr], ref[wr])
    check_untouched(out, wr)


@pytest.mark.parametrize("hidden,out_w,rank", [(256, 384, 16), (256, 256, 24), (192, 128, 64),
                                               (2048, 256, 8), (320, 256, 128), (4096, 640, 16),
                                               (4096, 256, 32), (128, 1024, 16)])
def test_random_within_tolerance(gpu, hidden, out_w, rank):
    """Rank 8..128 (one to eight 16-rank chunks, partial chunks masked) and
    both shrink paths (A_le in LDS when it fits, per tile otherwise)."""
    g = synth.gen(hidden + rank)
    T, k, E, L = 50, 4, 6, 3
    topk = synth.inputs.distinct_topk(T, E, k, g)
    n = T * k
    perm = torch.randperm(n + 11, generator=g)[:n].to(torch.int32)
    perm[torch.randperm(n, generator=g)[:n // 8]] = -1
    case = to_dev(synth.DeltaCase(
        f"fc1 random hidden={hidden} out={out_w} r={rank}",
        synth.bf16_normal((n + 11, hidden), 1.0, g), perm,
        synth.bf16_normal((L, E, rank, hidden), 0.05, g),
        synth.bf16_normal((L, E, out_w, rank), 0.05, g), topk, torch.ones(T, k),
        torch.randint(-1, L, (T,), generator=g).to(torch.int32), 1.75), gpu)
    tb = tables(case)
    ref, wr = run_oracle(case, tb)
    out = run_gpu(case, tb)
    check_close(to_f64(out)[wr], ref[wr], f"fc1 delta {hidden}/{out_w}/{rank}")
    check_untouched(out, wr)
    out2 = run_gpu(case, tb)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), "not deterministic"


def test_invalid_ids_give_zero_rows(gpu):
    """Adapter ids at or past num_adapters and out-of-range experts: the row is
    written as +0; a slot whose row is past padded_rows writes nothing; no
    adapter at all (num_adapters 0) zeroes every routed row."""
    case = to_dev(synth.delta_int_probe(T=24, top_k=3, E=5, I=64, H=128, L=3, r=8,
                                        pad_rows=4), gpu)
    tb = tables(case)
    lids = case.lora_ids.clone()
    lids[0], lids[1] = 3, 1000              # >= num_adapters: no adapter
    ids = case.topk_ids.clone()
    ids[2, 1], ids[3, 0] = 5, -3            # experts outside [0, E)
    perm = case.perm.clone()
    perm[4 * 3 + 2] = case.act.shape[0] + 2  # past padded_rows: not routed here
    ref, wr = run_oracle(case, tb, lora_ids=np.where(lids.cpu().numpy() >= 3, -1,
                                                     lids.cpu().numpy()),
                         topk_ids=ids, perm=np.where(perm.cpu().numpy() >= case.act.shape[0],
                                                     -1, perm.cpu().numpy()))
    out = run_gpu(case, tb, torch.float32, lora_ids=lids, topk_ids=ids, perm=perm)
    assert np.array_equal(to_f64(out)[wr], ref[wr])
    check_untouched(out, wr)
    for t in (0, 1):
        rows = [int(p) for p in perm[t * 3:(t + 1) * 3].tolist() if 0 <= p < case.act.shape[0]]
        assert not to_f64(out)[rows].any()
    out0 = run_gpu(case, tb, torch.float32, L=0, perm=perm)
    p_ok = perm.cpu().numpy()
    p_ok = p_ok[(p_ok >= 0) & (p_ok < case.act.shape[0])]
    assert not to_f64(out0)[p_ok].any()
    assert np.sum(to_f64(out0) == SENTINEL) == (case.act.shape[0] - len(p_ok)) * case.H


@pytest.mark.slow
def test_full_size_sampled(gpu):
    """The FC1 side of the delta workload's routing (T=8192, top_k=8, E=64,
    8 adapters of rank 16, 10% inactive slots) with hidden 4096 and 4096
    output columns (gate and up of I=2048), in the launch the bench times:
    40 sampled rows against the oracle, all columns; determinism."""
    case = synth.delta_at_scale(device=gpu, I=4096, H=4096)
    wa, wb = fill_w_ptr(case.A), fill_w_ptr(case.B)
    sa, sb = case.E * case.rank * case.I, case.E * case.H * case.rank
    out = moe_fc1_lora_delta(case.act, case.perm, wa, sa, wb, sb, case.topk_ids, case.lora_ids,
                             case.rank, case.H, num_adapters=case.L, scale=case.scale)
    out2 = moe_fc1_lora_delta(case.act, case.perm, wa, sa, wb, sb, case.topk_ids, case.lora_ids,
                              case.rank, case.H, num_adapters=case.L, scale=case.scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), "not deterministic"
    perm = case.perm.cpu().numpy()
    rng = np.random.default_rng(2)
    rows = sorted(rng.choice(perm[perm >= 0], 40, replace=False).tolist())
    tb = (case.A, wa.cpu(), sa, case.B, wb.cpu(), sb)
    ref, wr = run_oracle(case, tb, rows=rows)
    assert wr.all()
    rt = torch.tensor(rows, device=gpu)
    check_close(to_f64(out.index_select(0, rt)), ref, "fc1 delta full size (sampled)")
    unrouted = np.setdiff1d(np.arange(case.act.shape[0]), perm)
    assert len(unrouted) > 0 and not to_f64(out[torch.from_numpy(unrouted[:64]).to(gpu)]).any()
