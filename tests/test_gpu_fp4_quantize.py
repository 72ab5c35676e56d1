"""GPU parity of the NVFP4 quantiser against the oracle: codes and every
scale byte (padding included) bitwise, for each input type, batched
matrices with their own global scales, the special blocks, the full-size
skewed MoE FC2 activations on sampled rows, and the quantised operands fed
to the NVFP4 GEMMs."""
import numpy as np
import pytest
import torch

import synth
from moe_expert_grouped_amd import fp4_quantize, grouped_mm_nvfp4, mm_nvfp4_lora
from oracle import fp4_quantize as Q
from oracle import nvfp4 as NV
from oracle.formats import f64_to_bf16_bits
from oracle.nvfp4_grouped import grouped_mm_nvfp4 as oracle_grouped
from tests.parity import bits16, check_close, to_f64

pytestmark = pytest.mark.gpu


def _gpu(x, g, gpu, garbage=True):
    """Quantise on the GPU into buffers pre-filled with garbage, so that a
    byte the kernel fails to write shows up."""
    batch = 1 if x.dim() == 2 else x.shape[0]
    rows, k = x.shape[-2], x.shape[-1]
    per = (-(-rows // 128)) * (k // 64) * 512
    codes = torch.full((*x.shape[:-1], k // 2), 0xA5 if garbage else 0, dtype=torch.uint8,
                       device=gpu)
    sf = torch.full((batch * per,), 0x5A if garbage else 0, dtype=torch.uint8, device=gpu)
    print(f"fp4_quantize: {tuple(x.shape)} {x.dtype}", flush=True)
    c, s = fp4_quantize(x.to(gpu), g.to(gpu), codes=codes, sf=sf)
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy()


def _x32(x):
    return x.float().numpy()


def _gscale(x):
    return torch.tensor([448.0 * 6.0 / float(x.float().abs().max())], dtype=torch.float32)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("rows,k", [(300, 512), (1, 64), (128, 192), (129, 1024)])
def test_bitwise_against_oracle(gpu, dtype, rows, k):
    g = synth.gen(rows + k)
    x = (torch.randn((rows, k), generator=g) * torch.exp(torch.randn((rows, 1), generator=g))
         ).to(dtype)
    gs = _gscale(x)
    codes, sf = _gpu(x, gs, gpu)
    rc, rsf = Q.fp4_quantize(_x32(x), np.float32(gs[0]))
    assert np.array_equal(codes, rc)
    assert np.array_equal(sf, rsf)


def test_batched_matrices_with_own_scales(gpu):
    g = synth.gen(8)
    x = synth.bf16_normal((3, 130, 128), 1.0, g)
    x[1] *= 40
    gs = torch.tensor([0.5, 3.0, 1e-3], dtype=torch.float32)
    codes, sf = _gpu(x, gs, gpu)
    per = 2 * 2 * 512
    for b in range(3):
        rc, rsf = Q.fp4_quantize(_x32(x[b]), np.float32(gs[b]))
        assert np.array_equal(codes[b], rc), b
        assert np.array_equal(sf[b * per:(b + 1) * per], rsf), b


def test_special_blocks(gpu):
    """Zero and -0 blocks, blocks that underflow the scale, a global scale that
    saturates it, exact E2M1 midpoints (ties) and values past 6."""
    x = torch.zeros((4, 128), dtype=torch.float32)
    x[0, 16:32] = -0.0
    x[1, :16] = 1e-30 * torch.tensor([1.0, -1.0] * 8)
    x[2, :16] = torch.tensor([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25,
                              -1.75, -2.5, -3.5, -5.0, 4.0])
    x[2, 16:32] = torch.linspace(-9, 9, 16)
    x[3, :] = torch.randn(128, generator=synth.gen(3))
    for gval in (1.0, 1e6, 1e-6):
        gs = torch.tensor([gval], dtype=torch.float32)
        codes, sf = _gpu(x, gs, gpu)
        rc, rsf = Q.fp4_quantize(x.numpy(), np.float32(gval))
        assert np.array_equal(codes, rc), gval
        assert np.array_equal(sf, rsf), gval


def test_element_rounding_sweep(gpu):
    """Every block holds +-6 and g = 1, so its scale is 1.0 (code 0x38) and each
    other element is rounded as it is: values within 8 ulps of every E2M1
    midpoint and grid value (ties to the even code), both signs, and random
    values up to 6 -- bitwise against the oracle."""
    grid = [0.0, 0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0]
    vals = []
    for v in grid:
        b = np.float32(v).view(np.int32)
        for d in range(-8, 9):
            x = np.int32(b + d).view(np.float32) if v > 0 else np.float32(d * 1e-39)
            if 0 <= x <= 6:
                vals += [x, -x]
    rng = np.random.default_rng(7)
    vals += list(rng.uniform(-6, 6, 20000).astype(np.float32))
    vals = np.asarray(vals, dtype=np.float32)
    nblk = -(-len(vals) // 15)
    pad = np.resize(vals, nblk * 15).reshape(nblk, 15)
    blocks = np.concatenate([np.where(np.arange(nblk) % 2 == 0, 6.0, -6.0)[:, None], pad],
                            axis=1).astype(np.float32)
    rows = -(-nblk // 4)
    x = np.resize(blocks, (rows * 4, 16)).reshape(rows, 64)
    xt = torch.from_numpy(x)
    codes, sf = _gpu(xt, torch.tensor([1.0]), gpu)
    rc, rsf = Q.fp4_quantize(x, np.float32(1.0))
    assert np.all(rsf[NV.sf_offset(np.arange(rows)[:, None], np.arange(4)[None, :], 64)] == 0x38)
    assert np.array_equal(codes, rc)
    assert np.array_equal(sf, rsf)


@pytest.mark.slow
def test_full_size_skewed_activations_sampled(gpu):
    """The skewed MoE FC2 activations [32768, 2048] bf16 quantised in the
    launch the bench times: 24 sampled rows (first, last and both sides of a
    128-row tile edge among them) bitwise against the oracle, codes and their
    scale bytes; two launches agree on every byte of both outputs."""
    x = synth.bf16_normal((32768, 2048), 1.0, synth.gen(3, gpu), gpu)
    gs = torch.tensor([448.0 * 6.0 / float(x.float().abs().max())], dtype=torch.float32,
                      device=gpu)
    codes, sf = fp4_quantize(x, gs)
    codes2, sf2 = fp4_quantize(x, gs)
    torch.cuda.synchronize()
    assert torch.equal(codes, codes2) and torch.equal(sf, sf2)
    rng = np.random.default_rng(0)
    rows = np.sort(np.concatenate([[0, 127, 128, 32767], rng.choice(32768, 20, replace=False)]))
    rt = torch.from_numpy(rows).to(gpu)
    xr = x.index_select(0, rt).float().cpu().numpy()
    rc, rs = Q.quantize_rows(xr, np.float32(gs.cpu()[0]))
    assert np.array_equal(codes.index_select(0, rt).cpu().numpy(), rc)
    sfh = sf.cpu().numpy()
    off = NV.sf_offset(rows[:, None], np.arange(2048 // 16)[None, :], 2048)
    assert np.array_equal(sfh[off], rs)


def test_quantised_operands_through_the_nvfp4_gemms(gpu):
    """quantise(a), quantise(b) -> mm_nvfp4_lora with alpha = 1/(g_a g_b): the
    oracle's product of its own quantised operands (bitwise the GPU's) within
    the tolerance, and close to the bf16 product a @ b^T."""
    g = synth.gen(21)
    a = synth.bf16_normal((256, 512), 1.0, g)
    b = synth.bf16_normal((384, 512), 0.05, g)
    ga, gb = _gscale(a), _gscale(b)
    ca, sa = fp4_quantize(a.to(gpu), ga.to(gpu))
    cb, sb = fp4_quantize(b.to(gpu), gb.to(gpu))
    alpha = torch.tensor([1.0 / (float(ga[0]) * float(gb[0]))], dtype=torch.float32)
    out = mm_nvfp4_lora(ca, cb, sa, sb, alpha.to(gpu))
    torch.cuda.synchronize()
    rca, rsa = Q.fp4_quantize(_x32(a), np.float32(ga[0]))
    rcb, rsb = Q.fp4_quantize(_x32(b), np.float32(gb[0]))
    assert np.array_equal(ca.cpu().numpy(), rca) and np.array_equal(sb.cpu().numpy(), rsb)
    base = NV.base_product(rca, rcb, rsa, rsb, 512)
    check_close(to_f64(out), NV.mm_nvfp4_off(base, float(alpha[0])), "quantised operands")
    exact = a.double().numpy() @ b.double().numpy().T
    rel = np.sqrt(np.mean((to_f64(out) - exact) ** 2) / np.mean(exact ** 2))
    assert rel < 0.2, rel  # NVFP4 quantisation error, not a layout mistake
    # grouped: each expert's weights quantised as its own matrix (batched call)
    counts = (100, 0, 156)
    mi = torch.tensor([0, 100, 100, 256], dtype=torch.int32)
    w = synth.bf16_normal((3, 256, 512), 0.05, g)
    gw = torch.tensor([448.0 * 6.0 / float(w[e].float().abs().max()) for e in range(3)],
                      dtype=torch.float32)
    cw, sw = fp4_quantize(w.to(gpu), gw.to(gpu))
    alphas = (1.0 / (float(ga[0]) * gw)).to(torch.float32)
    og = grouped_mm_nvfp4(ca, sa, cw, sw, mi.to(gpu), alphas.to(gpu))
    torch.cuda.synchronize()
    ref, written = oracle_grouped(rca, rsa, cw.cpu().numpy(), sw.cpu().numpy(), alphas.numpy(),
                                  mi.numpy(), 512)
    for e in range(3):
        rw, rsw = Q.fp4_quantize(_x32(w[e]), np.float32(gw[e]))
        assert np.array_equal(cw[e].cpu().numpy(), rw)
        per = 2 * 8 * 512
        assert np.array_equal(sw[e * per:(e + 1) * per].cpu().numpy(), rsw)
    check_close(to_f64(og)[written], ref[written], "grouped with quantised operands")
    assert sum(counts) == int(written.sum())
