"""GPU parity of the NVFP4 + LoRA GEMM, the fold and the dequantiser."""
import numpy as np
import pytest
import torch

import synth
from moe_expert_grouped_amd import (StaleAdapterError, mm_nvfp4_lora, nvfp4_dequant,
                                    prepare_nvfp4_lora_adapter)
from oracle import nvfp4 as NV
from oracle.fold import fold
from oracle.formats import f64_to_bf16_bits
from tests.parity import bits16, check_close, sqnr_db, to_f64

pytestmark = pytest.mark.gpu


def _dev(case, dev):
    c = synth.Nvfp4Case(case.name, *(None if x is None else x.to(dev) for x in
                                     (case.a, case.b, case.a_sf, case.b_sf, case.alpha, case.d,
                                      case.lora_b, case.lora_scale, case.bias)), case.K)
    return c


def _np(t):
    return t.detach().cpu().numpy()


def _base(case, a_rows=None, b_rows=None):
    a = _np(case.a) if a_rows is None else _np(case.a[a_rows])
    b = _np(case.b) if b_rows is None else _np(case.b[b_rows])
    ar = None if a_rows is None else np.asarray(a_rows)
    br = None if b_rows is None else np.asarray(b_rows)
    return NV.base_product(a, b, _np(case.a_sf), _np(case.b_sf), case.K, ar, br)


def _bits(t):
    return None if t is None else bits16(t)


def test_dequant_bitwise(gpu):
    g = synth.gen(21)
    rows, k = 300, 512
    codes = torch.randint(0, 256, (rows, k // 2), generator=g).to(torch.uint8)
    sf = torch.randint(0, 0x7F, (synth.sf_buffer_bytes(rows, k),), generator=g).to(torch.uint8)
    got = nvfp4_dequant(codes.to(gpu), sf.to(gpu))
    torch.cuda.synchronize()
    want = f64_to_bf16_bits(NV.dequant(codes.numpy(), sf.numpy(), k))
    assert np.array_equal(bits16(got), want)


def test_identity_probe_bitwise(gpu):
    case = _dev(synth.nvfp4_probe("identity", M=128, N=256, K=256), gpu)
    out = mm_nvfp4_lora(case.a, case.b, case.a_sf, case.b_sf, case.alpha)
    torch.cuda.synchronize()
    want = f64_to_bf16_bits(NV.dequant(_np(case.a), _np(case.a_sf), 256))
    got = bits16(out)
    # the GEMM sums exact zeros onto each value: -0 may come back as +0
    assert np.array_equal(got & 0x7FFF, want & 0x7FFF)
    assert np.array_equal(got[want != 0x8000], want[want != 0x8000])


def _same_up_to_zero_sign(got, want):
    """Bitwise equality, except that the GEMM may return +0 where the exact
    value is -0 (it sums exact zeros onto each product)."""
    nz = (want & 0x7FFF) != 0
    assert np.array_equal(got[nz], want[nz])
    assert np.all((got[~nz] & 0x7FFF) == 0)


@pytest.mark.parametrize("side", ["a", "b"])
def test_gemm_scale_decode_all_codes_bitwise(gpu, side):
    """The K loop's own UE4M3 decode over every finite scale code 0x00..0x7E,
    on either operand: each output is one exact product (the other operand
    selects one element at scale 1.0), so it must equal the exact dequantised
    value bitwise."""
    case = synth.nvfp4_scale_probe(side)
    sf = case.a_sf if side == "a" else case.b_sf
    assert set(sf.unique().tolist()) == set(range(0x7F))  # every finite code drawn
    c = _dev(case, gpu)
    out = mm_nvfp4_lora(c.a, c.b, c.a_sf, c.b_sf, c.alpha)
    torch.cuda.synchronize()
    want = f64_to_bf16_bits(_base(case))
    M, N, K = case.M, case.N, case.K
    if side == "a":
        deq = NV.dequant(_np(case.a), _np(case.a_sf), K)[:, :N]
    else:
        deq = NV.dequant(_np(case.b), _np(case.b_sf), K)[:, :M].T
    _same_up_to_zero_sign(want, f64_to_bf16_bits(deq))  # the probe is the identity it claims
    _same_up_to_zero_sign(bits16(out), want)


def test_zero_codes_scaled_probe(gpu):
    """All codes zero with scales over every finite code: the product is +0
    everywhere (no scale decodes to NaN or Inf)."""
    c = _dev(synth.nvfp4_probe("zero_codes_scaled", M=200, N=512, K=512), gpu)
    out = mm_nvfp4_lora(c.a, c.b, c.a_sf, c.b_sf, c.alpha)
    torch.cuda.synchronize()
    assert np.all(bits16(out) == 0)


@pytest.mark.parametrize("M,N,K", [(128, 256, 256), (300, 520, 512), (1, 1, 256), (33, 258, 256),
                                   (70, 301, 256)])
def test_exact_probe_bitwise(gpu, M, N, K):
    case = _dev(synth.nvfp4_probe("exact", M=M, N=N, K=K), gpu)
    out = mm_nvfp4_lora(case.a, case.b, case.a_sf, case.b_sf, case.alpha)
    torch.cuda.synchronize()
    ref = _base(case)
    assert np.array_equal(bits16(out), f64_to_bf16_bits(ref))


def test_lora_only_probe(gpu):
    """Base is exactly zero; the output is the raw LoRA term plus bias alone,
    which C5-sized data could not resolve against its base."""
    case = _dev(synth.nvfp4_probe("lora_only", M=256, N=512, K=256), gpu)
    out = mm_nvfp4_lora(case.a, case.b, case.a_sf, case.b_sf, case.alpha, case.d, case.lora_b,
                        case.lora_scale, bias=case.bias)
    torch.cuda.synchronize()
    ref = NV.mm_nvfp4_raw(np.zeros((256, 512)), 0.01, _bits(case.d), _bits(case.lora_b), 0.5,
                         _bits(case.bias))
    check_close(to_f64(out), ref, "lora-only")
    # and without bias: pure LoRA term
    out = mm_nvfp4_lora(case.a, case.b, case.a_sf, case.b_sf, case.alpha, case.d, case.lora_b,
                        case.lora_scale)
    ref = NV.mm_nvfp4_raw(np.zeros((256, 512)), 0.01, _bits(case.d), _bits(case.lora_b), 0.5)
    check_close(to_f64(out), ref, "lora-only no bias")


def _all_paths(case):
    """(off, raw, prepared) GPU outputs and the prepared adapter."""
    off = mm_nvfp4_lora(case.a, case.b, case.a_sf, case.b_sf, case.alpha, bias=case.bias)
    raw = mm_nvfp4_lora(case.a, case.b, case.a_sf, case.b_sf, case.alpha, case.d, case.lora_b,
                        case.lora_scale, bias=case.bias)
    ad = prepare_nvfp4_lora_adapter(case.lora_b, case.lora_scale, case.alpha)
    prep = mm_nvfp4_lora(case.a, case.b, case.a_sf, case.b_sf, case.alpha, case.d,
                         lora_adapter=ad, bias=case.bias)
    torch.cuda.synchronize()
    return off, raw, prep, ad


@pytest.mark.parametrize("M,N,K,r", [(300, 520, 512, 16), (256, 256, 256, 8), (129, 384, 768, 32),
                                     (64, 256, 256, 24), (70, 301, 256, 16)])
def test_small_all_paths(gpu, M, N, K, r):
    case = _dev(synth.nvfp4_lora_case(seed=M + N, M=M, N=N, K=K, r=r), gpu)
    off, raw, prep, ad = _all_paths(case)
    base = _base(case)
    alpha, s = float(case.alpha[0]), float(case.lora_scale[0])
    bias = _bits(case.bias)
    check_close(to_f64(off), NV.mm_nvfp4_off(base, alpha, bias), "off")
    check_close(to_f64(raw), NV.mm_nvfp4_raw(base, alpha, _bits(case.d), _bits(case.lora_b), s,
                                            bias), "raw")
    fb, zero = fold(_bits(case.lora_b), s, alpha)
    assert np.array_equal(bits16(ad.b_folded), fb)
    check_close(to_f64(prep), NV.mm_nvfp4_prepared(base, alpha, _bits(case.d), fb, zero, bias),
                "prepared")


def test_misaligned_out_matches_aligned_bitwise(gpu):
    """An output that is not 8-byte aligned (a contiguous view one element
    into its buffer) takes per-element stores; it must hold the same bits as
    the aligned output, on every path (off, raw with bias, prepared)."""
    case = _dev(synth.nvfp4_lora_case(seed=37, M=130, N=520, K=256), gpu)
    off, raw, prep, ad = _all_paths(case)
    for ref, kw in ((off, {}), (raw, dict(d=case.d, lora_b=case.lora_b, lora_scale=case.lora_scale)),
                    (prep, dict(d=case.d, lora_adapter=ad))):
        buf = torch.full((130 * 520 + 8,), float("nan"), dtype=torch.bfloat16, device=gpu)
        out = buf[1:1 + 130 * 520].view(130, 520)
        assert out.data_ptr() % 8 != 0
        mm_nvfp4_lora(case.a, case.b, case.a_sf, case.b_sf, case.alpha, bias=case.bias, out=out, **kw)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        assert torch.isnan(buf[0]) and torch.isnan(buf[1 + 130 * 520:]).all()


def test_zero_adapter_outputs_are_bitwise_adapter_off(gpu):
    case = _dev(synth.nvfp4_lora_case(seed=31, M=200, N=300, K=512), gpu)
    off = mm_nvfp4_lora(case.a, case.b, case.a_sf, case.b_sf, case.alpha, bias=case.bias)
    zero = torch.zeros(1, dtype=torch.float32, device=gpu)
    raw0 = mm_nvfp4_lora(case.a, case.b, case.a_sf, case.b_sf, case.alpha, case.d, case.lora_b,
                         zero, bias=case.bias)
    none = mm_nvfp4_lora(case.a, case.b, case.a_sf, case.b_sf, case.alpha, case.d, case.lora_b,
                         None, bias=case.bias)
    ad0 = prepare_nvfp4_lora_adapter(case.lora_b, zero, case.alpha)
    prep0 = mm_nvfp4_lora(case.a, case.b, case.a_sf, case.b_sf, case.alpha, case.d,
                          lora_adapter=ad0, bias=case.bias)
    negz = torch.tensor([-0.0], dtype=torch.float32, device=gpu)
    raw_neg0 = mm_nvfp4_lora(case.a, case.b, case.a_sf, case.b_sf, case.alpha, case.d,
                             case.lora_b, negz, bias=case.bias)
    torch.cuda.synchronize()
    for name, t in [("raw s=0", raw0), ("s=None", none), ("prepared s=0", prep0),
                    ("raw s=-0", raw_neg0)]:
        assert torch.equal(t.view(torch.int16), off.view(torch.int16)), name
    assert int(ad0.fold_flags[0]) == 1


def test_fold_bitwise_and_refold_in_place(gpu):
    g = synth.gen(41)
    lb = synth.bf16_normal((8192, 16), 0.02, g).to(gpu)
    for s, a in [(0.5, 0.01), (1e-38, 1.0), (3.0e38, 0.5), (1.0, 3.0), (-0.75, 0.3)]:
        st = torch.tensor([s], dtype=torch.float32, device=gpu)
        at = torch.tensor([a], dtype=torch.float32, device=gpu)
        if not np.isfinite(np.float32(s) / np.float32(a)):
            with pytest.raises(ValueError):
                prepare_nvfp4_lora_adapter(lb, st, at)
            continue
        ad = prepare_nvfp4_lora_adapter(lb, st, at)
        torch.cuda.synchronize()
        want, zero = fold(bits16(lb), s, a)
        assert np.array_equal(bits16(ad.b_folded), want), (s, a)
        assert int(ad.fold_flags[0]) == int(zero)
    # every finite bf16 pattern through one inexact ratio and a subnormal one
    pats = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    pats = pats[torch.isfinite(pats.float())].contiguous()
    lb2 = pats[: (pats.numel() // 8) * 8].reshape(-1, 8).to(gpu)
    for s, a in [(1.0, 3.0), (1e-30, 7.0), (2.0 ** 100, 1.5)]:
        st = torch.tensor([s], dtype=torch.float32, device=gpu)
        at = torch.tensor([a], dtype=torch.float32, device=gpu)
        ad = prepare_nvfp4_lora_adapter(lb2, st, at)
        torch.cuda.synchronize()
        want, _ = fold(bits16(lb2), s, a)
        got = bits16(ad.b_folded)
        assert np.array_equal(got, want), (s, a)
    # in-place refold equals the eager fold, with a new lora_scale tensor
    st1 = torch.tensor([0.5], dtype=torch.float32, device=gpu)
    at1 = torch.tensor([0.01], dtype=torch.float32, device=gpu)
    ad = prepare_nvfp4_lora_adapter(lb, st1, at1)
    lb_new = synth.bf16_normal((8192, 16), 0.05, g).to(gpu)
    st2 = torch.tensor([0.125], dtype=torch.float32, device=gpu)
    prepare_nvfp4_lora_adapter(lb_new, st2, at1, out=ad)
    eager = prepare_nvfp4_lora_adapter(lb_new, st2, at1)
    torch.cuda.synchronize()
    assert torch.equal(ad.b_folded.view(torch.int16), eager.b_folded.view(torch.int16))
    assert ad.lora_scale is st2


def test_stale_adapter_and_argument_errors(gpu):
    case = _dev(synth.nvfp4_lora_case(seed=51, M=64, N=256, K=256), gpu)
    ad = prepare_nvfp4_lora_adapter(case.lora_b, case.lora_scale, case.alpha)
    mm_nvfp4_lora(case.a, case.b, case.a_sf, case.b_sf, case.alpha, case.d, lora_adapter=ad)
    case.lora_b.mul_(2)  # a copy_/in-place write into a source makes the adapter stale
    with pytest.raises(StaleAdapterError):
        mm_nvfp4_lora(case.a, case.b, case.a_sf, case.b_sf, case.alpha, case.d, lora_adapter=ad)
    ad = prepare_nvfp4_lora_adapter(case.lora_b, case.lora_scale, case.alpha)
    other_alpha = case.alpha.clone()
    with pytest.raises(StaleAdapterError):
        mm_nvfp4_lora(case.a, case.b, case.a_sf, case.b_sf, other_alpha, case.d, lora_adapter=ad)
    with pytest.raises(ValueError, match="not both"):
        mm_nvfp4_lora(case.a, case.b, case.a_sf, case.b_sf, case.alpha, case.d, case.lora_b,
                      case.lora_scale, lora_adapter=ad)
    with pytest.raises(ValueError, match="alpha == 0"):
        prepare_nvfp4_lora_adapter(case.lora_b, case.lora_scale,
                                   torch.zeros(1, dtype=torch.float32, device=gpu))
    with pytest.raises(ValueError, match="multiple of 256"):
        mm_nvfp4_lora(case.a[:, :64], case.b[:, :64], case.a_sf, case.b_sf, case.alpha)
    with pytest.raises(ValueError, match="requires d"):
        mm_nvfp4_lora(case.a, case.b, case.a_sf, case.b_sf, case.alpha, lora_adapter=ad)


@pytest.mark.slow
def test_full_size_sampled(gpu):
    """M=4096, N=8192, K=8192, r=16 (the bench's launch): raw, prepared and
    off on sampled rows x columns, plus SQNR against fp64 for context."""
    case = synth.nvfp4_lora_case(device=gpu)
    off, raw, prep, ad = _all_paths(case)
    rng = np.random.default_rng(1)
    rows = np.sort(np.concatenate([[0, 4095], rng.choice(4096, 30, replace=False)]))
    cols = np.sort(np.concatenate([[0, 8191], rng.choice(8192, 126, replace=False)]))
    base = _base(case, rows.tolist(), cols.tolist())
    alpha, s = float(case.alpha[0]), float(case.lora_scale[0])
    rt, ct = torch.from_numpy(rows).to(gpu), torch.from_numpy(cols).to(gpu)
    d = _bits(case.d[rt])
    lb = _bits(case.lora_b[ct])
    bias = _bits(case.bias[ct])
    sel = lambda t: to_f64(t.index_select(0, rt).index_select(1, ct))
    check_close(sel(off), NV.mm_nvfp4_off(base, alpha, bias), "off full")
    ref_raw = NV.mm_nvfp4_raw(base, alpha, d, lb, s, bias)
    check_close(sel(raw), ref_raw, "raw full")
    fb, zero = fold(_bits(case.lora_b), s, alpha)
    assert np.array_equal(bits16(ad.b_folded), fb)
    ref_prep = NV.mm_nvfp4_prepared(base, alpha, d, fb[cols], zero, bias)
    check_close(sel(prep), ref_prep, "prepared full")
    print(f"\nSQNR raw {sqnr_db(sel(raw), ref_raw):.1f} dB, prepared vs raw-formula "
          f"{sqnr_db(sel(prep), ref_raw):.1f} dB")
    # the zero-adapter forms at this shape: bitwise the adapter-off output over
    # the whole [4096, 8192] result
    zero = torch.zeros(1, dtype=torch.float32, device=gpu)
    negz = torch.tensor([-0.0], dtype=torch.float32, device=gpu)
    ad0 = prepare_nvfp4_lora_adapter(case.lora_b, zero, case.alpha)
    forms = {
        "raw s=0": lambda o: mm_nvfp4_lora(case.a, case.b, case.a_sf, case.b_sf, case.alpha,
                                           case.d, case.lora_b, zero, bias=case.bias, out=o),
        "raw s=-0": lambda o: mm_nvfp4_lora(case.a, case.b, case.a_sf, case.b_sf, case.alpha,
                                            case.d, case.lora_b, negz, bias=case.bias, out=o),
        "s=None": lambda o: mm_nvfp4_lora(case.a, case.b, case.a_sf, case.b_sf, case.alpha,
                                          case.d, case.lora_b, None, bias=case.bias, out=o),
        "prepared s=0": lambda o: mm_nvfp4_lora(case.a, case.b, case.a_sf, case.b_sf,
                                                case.alpha, case.d, lora_adapter=ad0,
                                                bias=case.bias, out=o),
    }
    offv = off.view(torch.int16)
    buf = torch.empty_like(off)
    for name, fn in forms.items():
        buf.fill_(7.0)
        fn(buf)
        torch.cuda.synchronize()
        assert torch.equal(buf.view(torch.int16), offv), name
