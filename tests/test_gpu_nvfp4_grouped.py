"""GPU parity of the NVFP4 grouped GEMM against the fp64 oracle: exact
probes bitwise, random operands within the tolerance, the full-size skewed
MoE FC2 shape on sampled rows and columns."""
import numpy as np
import pytest
import torch

import synth
from moe_expert_grouped_amd import grouped_mm_bf16, grouped_mm_nvfp4, nvfp4_dequant
from oracle.formats import f64_to_bf16_bits
from oracle.nvfp4_grouped import grouped_mm_nvfp4 as oracle_grouped
from oracle.nvfp4_grouped import grouped_mm_nvfp4_rows as oracle_rows
from tests.parity import bits16, check_close, to_f64

pytestmark = pytest.mark.gpu


def np_case(c):
    return (c.a.cpu().numpy(), c.a_sf.cpu().numpy(), c.b.cpu().numpy(), c.b_sf.cpu().numpy(),
            c.alpha.cpu().numpy(), c.m_indptr.cpu().numpy())


def run(c, gpu, out_dtype=torch.bfloat16, out=None):
    print(f"grouped_mm_nvfp4: {c.name} out={out_dtype}", flush=True)
    o = grouped_mm_nvfp4(c.a.to(gpu), c.a_sf.to(gpu), c.b.to(gpu), c.b_sf.to(gpu),
                         c.m_indptr.to(gpu), c.alpha.to(gpu), out=out, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("counts,n,k", [
    ((0, 1, 200, 256, 300, 0, 513, 40), 256, 256),   # 256-row tiles only (n % 512 != 0)
    ((0, 1, 200, 256, 300, 0, 513, 40), 512, 256),   # tails <= 128 rows take 128 x 512 tiles
    ((129, 0, 7), 1024, 512),                         # two K stages per trip, several panels
])
def test_exact_probe_bitwise(gpu, counts, n, k):
    """Scales 1.0 and power-of-two alphas: every fp32 sum is exact, so each
    output type is the exact value rounded once."""
    c = synth.nvfp4_grouped_case(seed=sum(counts), counts=counts, n=n, k=k, exact=True)
    ref, written = oracle_grouped(*np_case(c), k)
    out = run(c, gpu)
    assert np.array_equal(bits16(out)[written], f64_to_bf16_bits(ref[written]))
    out32 = run(c, gpu, torch.float32)
    assert np.array_equal(to_f64(out32)[written], ref[written])


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_misaligned_out_matches_aligned_bitwise(gpu, out_dtype):
    """An output not aligned for 4-column stores (a contiguous view one element
    into its buffer) takes per-element stores: the same bits as the aligned
    output, rows outside the groups untouched."""
    c = synth.nvfp4_grouped_case(seed=41, counts=(0, 130, 1, 300, 0, 129), n=512, k=256)
    ref = run(c, gpu, out_dtype)
    rows = c.a.shape[0]
    buf = torch.full((rows * 512 + 8,), 7.0, dtype=out_dtype, device=gpu)
    out = buf[1:1 + rows * 512].view(rows, 512)
    assert out.data_ptr() % 8 != 0
    out.copy_(ref)
    written = np.zeros(rows, dtype=bool)
    ind = c.m_indptr.numpy()
    written[ind[0]:ind[-1]] = True
    out[torch.from_numpy(written).to(gpu)] = float("nan")
    run(c, gpu, out_dtype, out=out)
    assert torch.equal(out, ref)
    assert (buf[0] == 7.0).item() and bool((buf[1 + rows * 512:] == 7.0).all())


@pytest.mark.parametrize("side", ["a", "b"])
def test_scale_decode_all_codes_bitwise(gpu, side):
    """The grouped K loop's UE4M3 decode over every finite scale code, on the
    activation side and on the expert-weight side: each output is one exact
    product, so it must equal the oracle bitwise (up to the sign of zero)."""
    c = synth.nvfp4_grouped_scale_probe(side, counts=(0, 130, 1, 300, 0, 129))
    sf = c.a_sf if side == "a" else c.b_sf
    assert set(sf.unique().tolist()) == set(range(0x7F))
    ref, written = oracle_grouped(*np_case(c), c.k)
    want = f64_to_bf16_bits(ref[written])
    got = bits16(run(c, gpu))[written]
    nz = (want & 0x7FFF) != 0
    assert np.array_equal(got[nz], want[nz])
    assert np.all((got[~nz] & 0x7FFF) == 0)
    out32 = to_f64(run(c, gpu, torch.float32))[written]
    assert np.array_equal(out32, ref[written])


def test_rows_outside_groups_untouched(gpu):
    c = synth.nvfp4_grouped_case(seed=3, counts=(5, 0, 40), n=256, k=256, exact=True)
    g = synth.gen(9)
    lead, trail = 3, 130  # trailing rows reach into the next 128-row scale tile
    a = torch.cat([torch.randint(0, 256, (lead, 128), generator=g, dtype=torch.uint8), c.a,
                   torch.randint(0, 256, (trail, 128), generator=g, dtype=torch.uint8)])
    a_sf = torch.full((synth.sf_buffer_bytes(a.shape[0], 256),), 0x38, dtype=torch.uint8)
    c2 = synth.Nvfp4GroupedCase("offset rows", a, a_sf, c.b, c.b_sf, c.alpha, c.m_indptr + lead,
                                256)
    sentinel = torch.full((a.shape[0], 256), -7.0, dtype=torch.bfloat16, device=gpu)
    out = run(c2, gpu, out=sentinel)
    ref, written = oracle_grouped(*np_case(c2), 256)
    assert written.sum() == 45 and not written[:lead].any() and not written[-trail:].any()
    assert (to_f64(out)[~written] == -7.0).all()
    assert np.array_equal(bits16(out)[written], f64_to_bf16_bits(ref[written]))


def test_random_operands(gpu):
    rng = np.random.default_rng(4)
    counts = rng.integers(0, 600, 9)
    counts[3] = 0
    c = synth.nvfp4_grouped_case(seed=4, counts=counts, n=512, k=768)
    ref, written = oracle_grouped(*np_case(c), 768)
    out = run(c, gpu)
    check_close(to_f64(out)[written], ref[written], "nvfp4 grouped random")
    # the same product through the decoder and the bf16 grouped GEMM (fp32 out):
    # a different summation order, so compared within the tolerance
    a16 = nvfp4_dequant(c.a.to(gpu), c.a_sf.to(gpu), 768)
    per = c.b_sf.numel() // c.b.shape[0]
    b16 = torch.stack([nvfp4_dequant(c.b[e].to(gpu), c.b_sf[e * per:(e + 1) * per].to(gpu), 768)
                       for e in range(c.b.shape[0])])
    via = grouped_mm_bf16(a16, b16, c.m_indptr.to(gpu), out_dtype=torch.float32)
    rows = torch.repeat_interleave(c.alpha, torch.from_numpy(np.asarray(counts)))
    check_close(to_f64(out)[written], (via.cpu().double() * rows[:, None].double()).numpy(),
                "nvfp4 grouped vs decode + bf16 grouped GEMM")


@pytest.mark.slow
def test_full_size_skewed_sampled(gpu):
    """E=128 experts with the Zipf(1.1) routing of 4096 tokens x top-8
    (cum_m=32768), n=7168, k=2048, bf16 out, in the launch configuration the
    bench times; first/last row of every non-empty expert plus random rows,
    96 random columns."""
    c = synth.nvfp4_grouped_case(device=gpu)
    out = run(c, gpu)
    out2 = run(c, gpu)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), "not deterministic"
    mi = c.m_indptr.cpu().numpy()
    rng = np.random.default_rng(0)
    rows = set()
    for e in range(len(mi) - 1):
        if mi[e + 1] > mi[e]:
            rows.update({int(mi[e]), int(mi[e + 1]) - 1})
    rows.update(rng.integers(0, int(mi[-1]), 32).tolist())
    rows = sorted(rows)
    cols = np.sort(rng.choice(c.b.shape[1], 96, replace=False))
    colt = torch.from_numpy(cols).to(gpu)
    ref = oracle_rows(c.a[rows].cpu().numpy(), c.a_sf.cpu().numpy(),
                      lambda e: c.b[e].index_select(0, colt).cpu().numpy(), c.b_sf.cpu().numpy(),
                      c.alpha.cpu().numpy(), mi, c.k, c.b.shape[1], rows, cols)
    check_close(to_f64(out[rows][:, colt]), ref, "nvfp4 grouped full size (sampled)")
