"""The C-ABI library loads, exports every symbol its header declares, and
rejects invalid arguments on the host before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

from moe_expert_grouped_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_symbols():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", f)).read()
            names |= set(re.findall(r"MI_API\s+[\w\s\*]+?\b(mi_\w+)\s*\(", txt))
    return names


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    syms = header_symbols()
    assert syms == set(_lib.EXPORTS)
    for s in syms:
        assert hasattr(L, s), s
    assert L.mi_abi_version() == 9


def _err(status):
    with pytest.raises(ValueError) as ei:
        _lib.check(status)
    return str(ei.value)


NULL = None
FAKE = 0x100000  # never dereferenced: validation fails before any launch


def test_grouped_mm_validation():
    L = _lib.lib()
    msg = _err(L.mi_grouped_mm_bf16(FAKE, 64, 64, _lib.MI_BF16, FAKE, 2, 100, FAKE, FAKE, _lib.MI_BF16, NULL))
    assert "n % 256" in msg
    msg = _err(L.mi_grouped_mm_bf16(FAKE, 64, 96, _lib.MI_BF16, FAKE, 2, 256, FAKE, FAKE, _lib.MI_BF16, NULL))
    assert "k % 64" in msg
    msg = _err(L.mi_grouped_mm_bf16(FAKE, 64, 64, _lib.MI_BF16, FAKE, 0, 256, FAKE, FAKE, _lib.MI_BF16, NULL))
    assert "batch_size" in msg
    msg = _err(L.mi_grouped_mm_bf16(FAKE, 64, 64, _lib.MI_BF16, FAKE, 2, 256, NULL, FAKE, _lib.MI_BF16, NULL))
    assert "m_indptr" in msg
    msg = _err(L.mi_grouped_mm_bf16(FAKE, 64, 64, _lib.MI_F32, FAKE, 2, 256, FAKE, FAKE,
                                    _lib.MI_BF16, NULL))
    assert "bf16 or fp16" in msg
    # k past the buffer-descriptor range of a 512-row b panel is valid but unsupported
    st = L.mi_grouped_mm_bf16(FAKE, 64, 1 << 22, _lib.MI_BF16, FAKE, 2, 256, FAKE, FAKE,
                              _lib.MI_BF16, NULL)
    assert st == _lib.MI_EUNSUPPORTED
    with pytest.raises(NotImplementedError, match="k < 4194304"):
        _lib.check(st)
    msg = _err(L.mi_grouped_mm_bf16(FAKE, 64, 64, _lib.MI_BF16, FAKE, 2, 256, FAKE, FAKE + 8,
                                    _lib.MI_BF16, NULL))
    assert "out must be 16-byte aligned" in msg
    # an empty a is a no-op that returns before touching the device
    assert L.mi_grouped_mm_bf16(NULL, 0, 64, _lib.MI_BF16, FAKE, 2, 256, FAKE, NULL, _lib.MI_BF16, NULL) == 0


def _nv(**kw):
    args = dict(a=FAKE, b=FAKE, a_sf=FAKE, a_sf_bytes=1 << 30, b_sf=FAKE, b_sf_bytes=1 << 30,
                alpha=FAKE, m=128, n=256, k=512, d=NULL, rank=0, lora_b=NULL, lora_scale=NULL,
                b_folded=NULL, fold_flags=NULL, bias=NULL, out=FAKE, stream=NULL)
    args.update(kw)
    return _lib.lib().mi_mm_nvfp4_lora(*args.values())


def test_nvfp4_validation_names_the_rule():
    assert "multiple of 256" in _err(_nv(k=320))
    assert "M >= 1" in _err(_nv(m=0))
    assert "N >= 1" in _err(_nv(n=0))
    both = _err(_nv(d=FAKE, rank=16, lora_b=FAKE, lora_scale=FAKE, b_folded=FAKE,
                    fold_flags=FAKE))
    assert "not both" in both
    assert "requires d" in _err(_nv(b_folded=FAKE, fold_flags=FAKE, rank=16))
    assert "rank" in _err(_nv(d=FAKE, rank=12, lora_b=FAKE, lora_scale=FAKE))
    assert "a_sf holds" in _err(_nv(a_sf_bytes=100))


def test_fold_and_dequant_validation():
    L = _lib.lib()
    assert "null" in _err(L.mi_prepare_lora_fold(NULL, 16, 16, FAKE, FAKE, FAKE, FAKE, NULL))
    assert "alias" in _err(L.mi_prepare_lora_fold(FAKE, 16, 16, FAKE, FAKE, FAKE, FAKE, NULL))
    assert "K % 64" in _err(L.mi_nvfp4_dequant_bf16(FAKE, FAKE, 1 << 20, 4, 96, FAKE, NULL))


def _delta(**kw):
    args = dict(act=FAKE, padded_rows=64, inter=128, perm=FAKE, wa=FAKE, sa=1024, wb=FAKE,
                sb=1024, ids=FAKE, w=FAKE, lids=FAKE, T=16, k=2, E=4, L=2, r=16, H=256,
                ldt=_lib.MI_BF16, scale=2.0, odt=_lib.MI_BF16, out=FAKE, ws=FAKE,
                wsb=1 << 30, stream=NULL)
    args.update(kw)
    return _lib.lib().mi_moe_fc2_lora_delta(*args.values())


def test_delta_validation():
    assert "rank" in _err(_delta(r=12))
    assert "top_k" in _err(_delta(k=0))
    assert "workspace" in _err(_delta(wsb=16))
    assert "strides" in _err(_delta(sa=1001))
    with pytest.raises(NotImplementedError):
        _lib.check(_delta(H=200))
    # a B_down block of 2^32 bytes or more does not fit the kernels' 32-bit range
    with pytest.raises(NotImplementedError, match="below 4 GiB"):
        _lib.check(_delta(H=1 << 27, r=16))
    with pytest.raises(NotImplementedError, match="below 4 GiB"):
        _lib.check(_delta(H=1 << 25, r=64))
    assert "lora_dtype must be bf16 or fp16" in _err(_delta(ldt=_lib.MI_F32))
    L = _lib.lib()
    fin = lambda fc2, fdt, **kw: L.mi_moe_fc2_finalize_lora(fc2, fdt, *dict(
        dict(act=FAKE, padded_rows=64, inter=128, perm=FAKE, wa=FAKE, sa=1024, wb=FAKE, sb=1024,
             ids=FAKE, w=FAKE, lids=FAKE, T=16, k=2, E=4, L=2, r=16, H=256, ldt=_lib.MI_BF16,
             scale=2.0, odt=_lib.MI_BF16, out=FAKE, ws=FAKE, wsb=1 << 30, stream=NULL),
        **kw).values())
    assert "fc2_out dtype" in _err(fin(FAKE, 7))
    assert "fc2_out is null" in _err(fin(NULL, _lib.MI_BF16))
    assert "rank" in _err(fin(FAKE, _lib.MI_F32, r=12))
    assert L.mi_moe_fc2_lora_delta_workspace_size(8192, 8, 64, 8, 16) > 8192 * 8 * 16 * 4
    assert L.mi_moe_fc2_lora_delta_workspace_size(8, 0, 4, 2, 8) == 0


def test_route_permutation_and_permute_rows_validation():
    L = _lib.lib()
    ws = L.mi_moe_route_workspace_size(65536, 64)
    assert ws == 64 * 64 * 4 + 256  # chunks of 1024 slots x experts x int32, plus slack
    assert L.mi_moe_route_workspace_size(0, 64) == 256
    assert L.mi_moe_route_workspace_size(-1, 64) == 0
    rp = lambda **kw: L.mi_moe_route_permutation(*{**dict(
        ids=FAKE, T=8192, k=8, E=64, indptr=FAKE, perm=FAKE, inv=NULL, ws=FAKE, wsb=ws,
        stream=NULL), **kw}.values())
    assert "num_experts must be in [1, 1024]" in _err(rp(E=1025))
    assert "num_experts must be in [1, 1024]" in _err(rp(E=0))
    assert "[0, 2^31)" in _err(rp(k=0))
    assert "[0, 2^31)" in _err(rp(T=1 << 28))
    assert "workspace needs" in _err(rp(wsb=ws - 1))
    assert "workspace needs" in _err(rp(ws=NULL))
    assert "m_indptr is null" in _err(rp(indptr=NULL))
    assert "is null" in _err(rp(perm=NULL))
    pr = lambda **kw: L.mi_moe_permute_rows(*{**dict(
        x=FAKE, T=16, rb=8192, perm=FAKE, k=8, out=FAKE, rows=128, stream=NULL), **kw}.values())
    assert "multiple of 16" in _err(pr(rb=8200))
    assert "multiple of 16" in _err(pr(rb=0))
    assert "16-byte aligned" in _err(pr(x=FAKE + 8))
    assert "null pointer" in _err(pr(perm=NULL))
    assert "out_rows" in _err(pr(rows=-1))
    assert "[0, 2^31)" in _err(pr(k=0))
    # nothing to copy: returns before touching the device
    assert pr(T=0, x=NULL, perm=NULL, out=NULL) == 0
    assert pr(rows=0, out=NULL) == 0


def test_grouped_nvfp4_validation():
    L = _lib.lib()
    per = 56 * 32 * 512  # n=7168 -> 56 row tiles, k=2048 -> 32 column tiles
    g = lambda **kw: L.mi_grouped_mm_nvfp4(*{**dict(
        a=FAKE, a_sf=FAKE, a_sf_bytes=1 << 30, m=32768, k=2048, b=FAKE, b_sf=FAKE,
        b_sf_bytes=128 * per, batch=128, n=7168, mi=FAKE, alpha=FAKE, out=FAKE,
        odt=_lib.MI_BF16, stream=NULL), **kw}.values())
    assert "n % 256" in _err(g(n=7000))
    assert "multiple of 256" in _err(g(k=2000))
    assert "batch_size" in _err(g(batch=0))
    assert "batch_size" in _err(g(batch=1025))
    assert "bf16 or fp32" in _err(g(odt=_lib.MI_F16))
    assert "experts' 128x4 layouts need" in _err(g(b_sf_bytes=128 * per - 1))
    assert "a_sf holds" in _err(g(a_sf_bytes=1000))
    assert "non-null" in _err(g(alpha=NULL))
    assert "16-byte aligned" in _err(g(a=FAKE + 8))
    assert "4-byte aligned" in _err(g(b_sf=FAKE + 2))
    assert g(m=0, a=NULL, a_sf=NULL, out=NULL) == 0  # no rows: nothing to do


def test_swiglu_validation():
    L = _lib.lib()
    g = lambda **kw: L.mi_grouped_mm_swiglu(*{**dict(
        a=FAKE, m=4096, k=2048, adt=_lib.MI_BF16, b=FAKE, batch=8, inter=1024, mi=FAKE,
        delta=NULL, alpha=NULL, beta=NULL, limit=NULL, out=FAKE, odt=_lib.MI_BF16,
        stream=NULL), **kw}.values())
    assert "% 128" in _err(g(inter=1000))
    assert "k % 64" in _err(g(k=100))
    assert "batch_size" in _err(g(batch=0))
    assert "bf16 or fp16" in _err(g(adt=_lib.MI_F32))
    assert "8-byte aligned" in _err(g(delta=FAKE + 4))
    assert "16-byte aligned" in _err(g(out=FAKE + 8))
    assert "null" in _err(g(mi=NULL))
    assert g(m=0, a=NULL, out=NULL) == 0


def test_fp4_quantize_validation():
    L = _lib.lib()
    q = lambda **kw: L.mi_fp4_quantize(*{**dict(
        x=FAKE, batch=1, rows=300, k=512, dt=_lib.MI_BF16, g=FAKE, codes=FAKE, sf=FAKE,
        sfb=1 << 30, stream=NULL), **kw}.values())
    assert "multiple of 64" in _err(q(k=96))
    assert "multiple of 64" in _err(q(k=0))
    assert "batch" in _err(q(batch=0))
    assert "bf16, fp16 or fp32" in _err(q(dt=7))
    assert "sf holds" in _err(q(sfb=3 * 8 * 512 - 1))
    assert q(sfb=3 * 8 * 512, rows=0, x=NULL, codes=NULL, sf=NULL) == 0  # no rows: no-op
    assert "null" in _err(q(g=NULL))
    assert "16-byte aligned" in _err(q(x=FAKE + 8))
    assert "4-byte aligned" in _err(q(sf=FAKE + 2))


def test_fc1_delta_validation():
    L = _lib.lib()
    f = lambda **kw: L.mi_moe_fc1_lora_delta(*{**dict(
        act=FAKE, padded_rows=64, hidden=128, perm=FAKE, wa=FAKE, sa=1024, wb=FAKE, sb=1024,
        ids=FAKE, lids=FAKE, T=16, k=2, E=4, L=2, r=16, out_features=256, ldt=_lib.MI_BF16,
        scale=2.0, odt=_lib.MI_BF16, out=FAKE, ws=FAKE, wsb=1 << 30, stream=NULL),
        **kw}.values())
    assert "moe_fc1_lora_delta" in _err(f(r=12)) and "rank" in _err(f(r=12))
    assert "top_k" in _err(f(k=0))
    assert "workspace" in _err(f(wsb=16))
    assert "strides" in _err(f(sb=1001))
    with pytest.raises(NotImplementedError):
        _lib.check(f(out_features=200))
    with pytest.raises(NotImplementedError, match="below 4 GiB"):
        _lib.check(f(out_features=1 << 27))
    assert "activation width" in _err(f(hidden=12))
    assert "16-byte aligned" in _err(f(out=FAKE + 8))
    assert f(T=0, act=NULL, perm=NULL, ids=NULL, lids=NULL, out=NULL, ws=NULL) == 0
    assert L.mi_moe_fc1_lora_delta_workspace_size(8192, 8, 64, 8, 16) == \
        L.mi_moe_fc2_lora_delta_workspace_size(8192, 8, 64, 8, 16)
