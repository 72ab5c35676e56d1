"""GPU parity of the ragged grouped GEMM against the fp64 oracle."""
import numpy as np
import pytest
import torch

import synth
from moe_expert_grouped_amd import grouped_mm_bf16
from oracle.formats import f64_to_bf16_bits
from oracle.grouped_mm import grouped_mm, grouped_mm_rows
from tests.parity import bits16, check_close, to_f64

pytestmark = pytest.mark.gpu


def _run(case, dev, out_dtype=torch.bfloat16, out=None):
    a, b, mi = case.a.to(dev), case.b.to(dev), case.m_indptr.to(dev)
    o = grouped_mm_bf16(a, b, mi, out=out, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o


def _oracle(case):
    return grouped_mm(bits16(case.a), bits16(case.b), case.m_indptr.numpy())


def test_tiny_moe_fc2(gpu):
    case = synth.grouped_tiny()
    ref, written = _oracle(case)
    out = _run(case, gpu)
    check_close(to_f64(out)[written], ref[written], "tiny grouped GEMM")


@pytest.mark.parametrize("counts,n,k", [
    ((0, 1, 17, 128, 0, 255), 256, 128),          # small groups: 64x128 tiles, 2 K steps
    ((100, 0, 150, 177, 0, 229), 512, 192),       # medium: 64x128 tiles, several per group
    ((300, 0, 513, 1, 256, 0, 390), 256, 256),    # large: 256x256 tiles, ragged tails
    # large, n not a multiple of 512 (256x256 tiles), odd K-step count: last
    # pieces of 128 / 129 / 255 / 1 / 0 / 128 / 88 / 232 rows (128-row tiles
    # for pieces up to 128 rows, 256-row tiles above)
    ((128, 129, 255, 257, 0, 384, 600, 1000), 768, 192),
])
def test_integer_probe_bitwise(gpu, counts, n, k):
    case = synth.grouped_int_probe(counts=counts, n=n, k=k)
    ref, written = _oracle(case)
    out = _run(case, gpu)
    want = f64_to_bf16_bits(ref[written])
    got = bits16(out)[written]
    assert np.array_equal(got, want)
    out32 = _run(case, gpu, torch.float32)
    assert np.array_equal(to_f64(out32)[written], ref[written])


@pytest.mark.parametrize("counts,n,k", [
    # large groups with n % 512 == 0 (384-row tiles; a last piece of 129..256
    # rows as a 256-row tile, of at most 128 rows as a 128 x 512 tile): pieces
    # of 1, 127, 128, 129, 255, 256, 257, 383 rows; one K step only, an even
    # and an odd step count
    ((384, 385, 0, 640, 641, 767, 1, 128, 129, 256, 257, 383), 1024, 64),
    ((500, 1, 0, 1151), 512, 128),
    ((257, 0, 700, 64, 129, 1000), 1536, 320),
])
def test_integer_probe_bitwise_large_tiles(gpu, counts, n, k):
    """Every output type, bf16 and fp16 operands, against the exact sums."""
    from oracle.formats import f64_to_f16_bits
    assert sum(counts) >= 192 * len(counts) and n % 512 == 0
    case = synth.grouped_int_probe(seed=120 + k, counts=counts, n=n, k=k)
    ref, written = _oracle(case)
    assert np.array_equal(bits16(_run(case, gpu))[written], f64_to_bf16_bits(ref[written]))
    assert np.array_equal(to_f64(_run(case, gpu, torch.float32))[written], ref[written])
    assert np.array_equal(bits16(_run(case, gpu, torch.float16))[written],
                          f64_to_f16_bits(ref[written]))
    a16, b16 = case.a.float().half(), case.b.float().half()
    mi = case.m_indptr
    ref16, w16 = grouped_mm(bits16(a16), bits16(b16), mi.numpy(), "f16")
    out = grouped_mm_bf16(a16.to(gpu), b16.to(gpu), mi.to(gpu), out_dtype=torch.float16)
    torch.cuda.synchronize()
    assert np.array_equal(bits16(out)[w16], f64_to_f16_bits(ref16[w16]))


def test_large_tiles_rows_outside_groups_untouched_and_many_experts(gpu):
    """Large groups with n % 512 == 0: leading and trailing rows outside every
    group keep their contents (the last group's tile reads past its rows);
    300 experts, most empty, a few of one row, in one call."""
    base = synth.grouped_int_probe(seed=21, counts=(400, 0, 433, 1), n=512, k=128)
    cum = base.a.shape[0]
    a = synth.bf16_ints((5 + cum + 9, 128), -3, 3, synth.gen(22))
    case = synth.GroupedCase("offset large", a, base.b, base.m_indptr + 5)
    sentinel = torch.full((a.shape[0], 512), -7.0, dtype=torch.bfloat16, device=gpu)
    out = _run(case, gpu, out=sentinel)
    ref, written = _oracle(case)
    assert not written[:5].any() and not written[-9:].any() and written[5:5 + cum].all()
    assert (to_f64(out)[~written] == -7.0).all()
    assert np.array_equal(bits16(out)[written], f64_to_bf16_bits(ref[written]))
    rng = np.random.default_rng(23)
    counts = np.zeros(300, dtype=np.int64)
    live = rng.choice(300, 80, replace=False)
    counts[live] = rng.integers(300, 1700, 80)
    counts[live[:4]] = 1
    assert counts.sum() >= 192 * 300
    many = synth.grouped_int_probe(seed=24, counts=tuple(counts.tolist()), n=512, k=64)
    ref, written = _oracle(many)
    assert np.array_equal(bits16(_run(many, gpu))[written], f64_to_bf16_bits(ref[written]))


def test_rows_outside_groups_untouched(gpu):
    base = synth.grouped_int_probe(counts=(5, 0, 40), n=256, k=64)
    cum = base.a.shape[0]
    a = synth.bf16_ints((3 + cum + 7, 64), -3, 3, synth.gen(5))
    case = synth.GroupedCase("offset", a, base.b, base.m_indptr + 3)  # 3 leading, 7 trailing rows
    sentinel = torch.full((a.shape[0], 256), -7.0, dtype=torch.bfloat16, device=gpu)
    out = _run(case, gpu, out=sentinel)
    ref, written = _oracle(case)
    assert not written[:3].any() and not written[-7:].any() and written[3:3 + cum].all()
    assert (to_f64(out)[~written] == -7.0).all()
    assert np.array_equal(bits16(out)[written], f64_to_bf16_bits(ref[written]))


def test_uniform_full_size_bf16_and_fp32(gpu):
    case = synth.grouped_uniform(device="cpu")
    ref, written = _oracle(case)
    for dt in (torch.bfloat16, torch.float32):
        out = _run(case, gpu, dt)
        check_close(to_f64(out), ref, f"uniform E=8 tpe=128 k=4096 n=2048 {dt}")


@pytest.mark.parametrize("n", [768, 1024])  # large groups: 256x256 tiles / direct-to-LDS tiles
def test_random_ragged_shapes_all_tile_configs(gpu, n):
    g = np.random.default_rng(7 + n)
    for avg in (40, 130, 400, 700):
        E = 9
        counts = g.integers(0, 2 * avg, E)
        counts[g.integers(0, E)] = 0
        mi = torch.zeros(E + 1, dtype=torch.int32)
        mi[1:] = torch.from_numpy(np.cumsum(counts)).to(torch.int32)
        gg = synth.gen(int(avg) + n)
        a = synth.bf16_normal((int(mi[-1]), 320), 1.0, gg)
        b = synth.bf16_normal((E, n, 320), 320 ** -0.5, gg)
        case = synth.GroupedCase(f"avg{avg} n{n}", a, b, mi)
        ref, written = _oracle(case)
        out = _run(case, gpu)
        check_close(to_f64(out)[written], ref[written], f"ragged avg={avg} n={n}")


@pytest.mark.slow
def test_zipf_full_size_sampled(gpu):
    """Full-size skewed MoE FC2 (E=128, cum_m=32768, k=2048, n=7168) checked
    on sampled rows (first/last row of every non-empty expert plus random
    rows) and sampled columns, in the launch configuration the bench times."""
    case = synth.grouped_zipf(device=gpu)
    out = grouped_mm_bf16(case.a, case.b, case.m_indptr)
    out2 = grouped_mm_bf16(case.a, case.b, case.m_indptr)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), "not deterministic"
    mi = case.m_indptr.cpu().numpy()
    rng = np.random.default_rng(0)
    rows = set()
    for e in range(len(mi) - 1):
        if mi[e + 1] > mi[e]:
            rows.update({int(mi[e]), int(mi[e + 1]) - 1})
            # both sides of every 384-row tile edge inside the expert
            for r0 in range(int(mi[e]) + 384, int(mi[e + 1]), 384):
                rows.update({r0 - 1, r0})
    rows.update(rng.integers(0, int(mi[-1]), 32).tolist())
    rows = sorted(rows)
    # both sides of 256- and 512-column panel edges, plus random columns
    edges = {0, 255, 256, 511, 512, 3583, 3584, 7167}
    cols = np.sort(np.array(sorted(edges | set(rng.choice(7168, 96, replace=False).tolist()))))
    a_rows = bits16(case.a[rows])
    colt = torch.from_numpy(cols).to(gpu)
    ref = grouped_mm_rows(a_rows, lambda e, c: bits16(case.b[e].index_select(0, colt)), mi, rows,
                          cols)
    got = to_f64(out[rows][:, colt])
    check_close(got, ref, "zipf sampled")


def test_deterministic(gpu):
    case = synth.grouped_int_probe(counts=(300, 0, 513, 1), n=512, k=256, lo=-100, hi=100)
    o1 = _run(case, gpu)
    o2 = _run(case, gpu)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("counts,n,k", [
    ((0, 1, 17, 128, 0, 255), 256, 128),          # small groups: 64x128 tiles, 2 K steps
    ((300, 0, 513, 1, 256, 0, 390), 256, 256),    # large: 256x256 tiles
])
def test_fp16_inputs_integer_probe_bitwise_every_output(gpu, counts, n, k):
    """fp16 a and b (the page's other input type) with bf16, fp16 and fp32
    outputs; small-integer operands make every fp32 sum exact, so each output
    is the oracle's exact value rounded once."""
    from oracle.formats import f64_to_f16_bits
    case = synth.grouped_int_probe(seed=111, counts=counts, n=n, k=k)
    a16, b16 = case.a.float().half(), case.b.float().half()
    mi = case.m_indptr
    ref, written = grouped_mm(bits16(a16), bits16(b16), mi.numpy(), "f16")
    for out_dtype, enc in ((torch.float16, f64_to_f16_bits), (torch.bfloat16, f64_to_bf16_bits)):
        out = grouped_mm_bf16(a16.to(gpu), b16.to(gpu), mi.to(gpu), out_dtype=out_dtype)
        torch.cuda.synchronize()
        assert np.array_equal(bits16(out)[written], enc(ref[written])), out_dtype
    out = grouped_mm_bf16(a16.to(gpu), b16.to(gpu), mi.to(gpu), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(out)[written], ref[written])


def test_fp16_random_ragged_fp16_out(gpu):
    g = np.random.default_rng(17)
    for avg in (40, 400):
        E = 7
        counts = g.integers(0, 2 * avg, E)
        mi = torch.zeros(E + 1, dtype=torch.int32)
        mi[1:] = torch.from_numpy(np.cumsum(counts)).to(torch.int32)
        gg = synth.gen(int(avg) + 5)
        a = synth.bf16_normal((int(mi[-1]), 256), 1.0, gg).float().half()
        b = synth.bf16_normal((E, 512, 256), 256 ** -0.5, gg).float().half()
        ref, written = grouped_mm(bits16(a), bits16(b), mi.numpy(), "f16")
        out = grouped_mm_bf16(a.to(gpu), b.to(gpu), mi.to(gpu), out_dtype=torch.float16)
        torch.cuda.synchronize()
        check_close(to_f64(out)[written], ref[written], f"fp16 ragged avg={avg}")


def test_limits_of_the_walk(gpu):
    """1024 experts (the largest batch), most of them empty, one row in some,
    n=256 (the smallest n), and a long K (k=8192) with a single-row group."""
    rng = np.random.default_rng(11)
    counts = np.zeros(1024, dtype=np.int64)
    live = rng.choice(1024, 40, replace=False)
    counts[live] = rng.integers(1, 300, 40)
    counts[live[:5]] = 1
    case = synth.grouped_int_probe(seed=12, counts=tuple(counts.tolist()), n=256, k=64)
    ref, written = _oracle(case)
    out = _run(case, gpu)
    assert np.array_equal(bits16(out)[written], f64_to_bf16_bits(ref[written]))
    big = synth.grouped_int_probe(seed=13, counts=(1, 0, 2), n=256, k=8192, lo=-1, hi=1)
    ref, written = _oracle(big)
    out32 = _run(big, gpu, torch.float32)
    assert np.array_equal(to_f64(out32)[written], ref[written])
