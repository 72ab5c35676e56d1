"""GPU parity of the FC1 gate/up grouped GEMM with its SwiGLU epilogue
against the fp64 oracle (the activation is not exact, so every comparison
uses the tolerance)."""
import numpy as np
import pytest
import torch

import synth
from moe_expert_grouped_amd import grouped_mm_bf16, grouped_mm_swiglu
from oracle.fc1 import grouped_mm_swiglu as oracle_fc1
from tests.parity import bits16, check_close, to_f64

pytestmark = pytest.mark.gpu


def host(t):
    return None if t is None else t.cpu()


def run(c, gpu, out_dtype=torch.bfloat16, out=None):
    print(f"grouped_mm_swiglu: {c.name} delta={c.delta is not None} "
          f"params={c.alpha is not None} out={out_dtype}", flush=True)
    d = lambda t: None if t is None else t.to(gpu)
    o = grouped_mm_swiglu(c.a.to(gpu), c.b.to(gpu), c.m_indptr.to(gpu), fc1_delta=d(c.delta),
                          gemm1_alpha=d(c.alpha), gemm1_beta=d(c.beta),
                          gemm1_clamp_limit=d(c.limit), out=out, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o


def oracle(c):
    np_ = lambda t: None if t is None else t.cpu().numpy()
    return oracle_fc1(bits16(c.a.cpu()), bits16(c.b.cpu()), c.m_indptr.cpu().numpy(),
                      delta_bits=None if c.delta is None else bits16(c.delta.cpu()),
                      alpha=np_(c.alpha), beta=np_(c.beta), limit=np_(c.limit))


@pytest.mark.parametrize("counts,inter,k,kw", [
    # 256-row tiles, 128-row tails (1, 40, 128 rows), a 129-row tail, empty experts; odd K steps
    ((0, 1, 128, 129, 255, 300, 0, 40), 256, 192, dict(ints=True)),
    ((300, 0, 513, 1), 128, 256, dict(with_delta=True, act_params=True)),
    ((200, 260), 384, 320, dict(act_params=True)),
    # average >= 192 rows and I % 256 == 0: the direct-to-LDS tiles -- 384-row
    # tiles, 256-row tails (129 rows), 128-row tails on 512-wide panels (1, 40 rows)
    ((0, 385, 1, 700, 129, 0, 300, 40), 256, 192, dict(with_delta=True, act_params=True)),
    ((769, 0, 200), 512, 256, dict(ints=True)),
])
def test_small_cases(gpu, counts, inter, k, kw):
    c = synth.fc1_case(seed=len(counts), counts=counts, hidden=k, inter=inter, **kw)
    ref, written = oracle(c)
    for dt in (torch.bfloat16, torch.float32, torch.float16):
        out = run(c, gpu, dt)
        check_close(to_f64(out)[written], ref[written], f"swiglu {c.name} {dt}")


@pytest.mark.parametrize("counts,inter", [((5, 0, 40), 128),      # register-staged tiles
                                          ((5, 0, 600), 256)])    # direct-to-LDS tiles
def test_rows_outside_groups_untouched(gpu, counts, inter):
    base = synth.fc1_case(seed=5, counts=counts, hidden=128, inter=inter, ints=True)
    g = synth.gen(6)
    a = torch.cat([synth.bf16_ints((3, 128), -2, 2, g), base.a, synth.bf16_ints((7, 128), -2, 2, g)])
    c = synth.Fc1Case("offset rows", a, base.b, base.m_indptr + 3, None, None, None, None)
    sentinel = torch.full((a.shape[0], inter), -7.0, dtype=torch.bfloat16, device=gpu)
    out = run(c, gpu, out=sentinel)
    ref, written = oracle(c)
    assert not written[:3].any() and not written[-7:].any() and written.sum() == sum(counts)
    assert (to_f64(out)[~written] == -7.0).all()
    check_close(to_f64(out)[written], ref[written], "swiglu offset rows")


def test_matches_unfused_gemm_then_activation(gpu):
    """The fused epilogue against the plain grouped GEMM (fp32 h) followed by
    the activation in torch fp32."""
    c = synth.fc1_case(seed=8, counts=(400, 50, 0, 333), hidden=256, inter=256,
                       with_delta=True, act_params=True)
    out = run(c, gpu, torch.float32)
    h = grouped_mm_bf16(c.a.to(gpu), c.b.to(gpu), c.m_indptr.to(gpu), out_dtype=torch.float32)
    h = h + c.delta.to(gpu).float()
    e_of = torch.repeat_interleave(torch.arange(4, device=gpu),
                                   torch.diff(c.m_indptr.to(gpu)).long())
    al, be, li = (t.to(gpu)[e_of][:, None] for t in (c.alpha, c.beta, c.limit))
    gte = torch.minimum(h[:, :256], li)
    up = torch.maximum(torch.minimum(h[:, 256:], li), -li)
    want = gte * torch.sigmoid(al * gte) * (up + be)
    check_close(to_f64(out), want.double().cpu().numpy(), "fused vs unfused")


@pytest.mark.slow
def test_full_size_sampled(gpu):
    """E=128 experts with the Zipf(1.1) routing of 4096 tokens x top-8
    (cum_m=32768), hidden=7168, inter=2048, bf16 out, in the launch
    configuration the bench times: first/last row of every non-empty expert
    plus random rows, 96 random output columns, via the oracle on the
    sampled sub-problem."""
    c = synth.fc1_case(device=gpu)
    out = run(c, gpu)
    mi = c.m_indptr.cpu().numpy()
    rng = np.random.default_rng(0)
    rows = set()
    for e in range(len(mi) - 1):
        if mi[e + 1] > mi[e]:
            rows.update({int(mi[e]), int(mi[e + 1]) - 1})
    rows.update(rng.integers(0, int(mi[-1]), 32).tolist())
    rows = np.array(sorted(rows))
    inter = c.b.shape[1] // 2
    cols = np.sort(rng.choice(inter, 96, replace=False))
    pick = torch.from_numpy(np.concatenate([cols, inter + cols])).to(gpu)
    experts = np.searchsorted(mi, rows, side="right") - 1
    sub_indptr = np.searchsorted(experts, np.arange(len(mi)), side="left")
    sub = synth.Fc1Case("sampled", c.a[torch.from_numpy(rows).to(gpu)].cpu(),
                        c.b.index_select(1, pick).cpu(), torch.from_numpy(sub_indptr).int(),
                        None, None, None, None)
    ref, written = oracle(sub)
    assert written.all()
    got = to_f64(out[torch.from_numpy(rows).to(gpu)][:, torch.from_numpy(cols).to(gpu)])
    check_close(got, ref, "swiglu full size (sampled)")


@pytest.mark.parametrize("counts,inter", [((150, 0, 300, 7), 128),          # register-staged
                                          ((300, 0, 513, 1, 200), 256)])   # direct-to-LDS
def test_fp16_operands(gpu, counts, inter):
    """fp16 a and b (the GEMM's other input type), every output type."""
    c = synth.fc1_case(seed=13, counts=counts, hidden=192, inter=inter, act_params=True)
    c16 = synth.Fc1Case("fp16 operands", c.a.to(torch.float16), c.b.to(torch.float16),
                        c.m_indptr, None, c.alpha, c.beta, c.limit)
    np_ = lambda t: t.cpu().numpy()
    ref, written = oracle_fc1(bits16(c16.a), bits16(c16.b), c16.m_indptr.numpy(), dtype="f16",
                              alpha=np_(c.alpha), beta=np_(c.beta), limit=np_(c.limit))
    for dt in (torch.bfloat16, torch.float16, torch.float32):
        out = run(c16, gpu, dt)
        check_close(to_f64(out)[written], ref[written], f"swiglu fp16 operands {dt}")
