"""The allocation-free FC2 delta entry point against the workspace one, called
through the C ABI: bitwise the same output on two calls in a row, the
second on a smaller problem (the scratch array keeps the first call's
contents), and the host-side refusal of a problem larger than the array."""
import ctypes

import pytest
import torch

import synth
from moe_expert_grouped_amd import _lib, bgmv_moe_gemm2_lora_delta, fill_w_ptr

pytestmark = pytest.mark.gpu


def _noalloc(case, wa, sa, wb, sb, out):
    L = _lib.lib()
    dev = case.act.device
    stream = torch.cuda.current_stream(dev).cuda_stream
    T, top_k = case.topk_ids.shape
    return L.mi_moe_fc2_lora_delta_noalloc(
        case.act.data_ptr(), case.act.shape[0], case.act.shape[1], case.perm.data_ptr(),
        wa.data_ptr(), sa, wb.data_ptr(), sb, case.topk_ids.data_ptr(),
        case.topk_weights.data_ptr(), case.lora_ids.data_ptr(), T, top_k, wa.numel(), case.L,
        case.rank, case.H, _lib.MI_BF16, ctypes.c_float(case.scale), _lib.MI_BF16,
        out.data_ptr(), ctypes.c_void_p(stream))


def _case_pair(case):
    wa, wb = fill_w_ptr(case.A), fill_w_ptr(case.B)
    sa = case.E * case.rank * case.I
    sb = case.E * case.H * case.rank
    return wa, sa, wb, sb


def _small(gpu):
    c = synth.delta_tiny()
    return synth.DeltaCase(c.name, c.act.to(gpu), c.perm.to(gpu), c.A.to(gpu), c.B.to(gpu),
                           c.topk_ids.to(gpu), c.topk_weights.to(gpu), c.lora_ids.to(gpu),
                           c.scale)


def test_noalloc_matches_workspace_entry_point(gpu):
    big = synth.delta_at_scale(device=gpu)
    small = _small(gpu)
    for case in (big, small):  # two calls in a row, the second smaller
        print(f"delta noalloc vs workspace: {case.name}", flush=True)
        wa, sa, wb, sb = _case_pair(case)
        ref = bgmv_moe_gemm2_lora_delta(case.act, case.perm, wa, sa, wb, sb, case.topk_ids,
                                        case.topk_weights, case.lora_ids, case.rank, case.H,
                                        num_adapters=case.L, scale=case.scale)
        out = torch.full_like(ref, 3.0)
        _lib.check(_noalloc(case, wa, sa, wb, sb, out))
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), case.name
    # a problem whose workspace exceeds the array is refused before any launch
    L = _lib.lib()
    T, top_k, E, nl, r = 65536, 8, 64, 8, 16
    assert L.mi_moe_fc2_lora_delta_workspace_size(T, top_k, E, nl, r) > (32 << 20)
    big_ids = torch.zeros((T, top_k), dtype=torch.int32, device=gpu)
    st = L.mi_moe_fc2_lora_delta_noalloc(
        big.act.data_ptr(), big.act.shape[0], big.act.shape[1], big_ids.data_ptr(),
        big.A.data_ptr(), 0, big.B.data_ptr(), 0, big_ids.data_ptr(), big_ids.data_ptr(),
        big_ids.data_ptr(), T, top_k, E, nl, r, big.H, _lib.MI_BF16, ctypes.c_float(1.0),
        _lib.MI_BF16, big.act.data_ptr(), None)
    with pytest.raises(NotImplementedError, match="fixed array holds"):
        _lib.check(st)
