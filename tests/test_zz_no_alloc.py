"""The allocation-free tree verify (attn_verify_tree_noalloc, scratch held by
the library) gives exactly the results of attn_verify_tree with a caller
workspace: the same kernels run on the same inputs.  Two calls in a row, the
second on a smaller batch, so the second reuses the scratch the first left
behind; both compared element by element (bit-identical) and to the oracle."""

import ctypes

import numpy as np
import pytest
import torch

import masked_flash_attention_mask_amd as ma
from masked_flash_attention_mask_amd import _lib as L
import workloads as W
from helpers import TOL_BF16, device_inputs, lse_err, max_abs_err, oracle

pytestmark = pytest.mark.gpu


def _calls(w, form, max_q, max_kv):
    dev = device_inputs(w)
    mi = w.masks[form]
    data = mi.data if mi.kind == "dense" else mi.data.view(np.int64)
    mask = torch.from_numpy(np.ascontiguousarray(data)).cuda()
    # the existing entry point, with a caller workspace
    o_ws, l_ws = ma.attn_verify_tree(dev["q"], dev["k"], dev["v"], dev["pt"], dev["cu"], dev["kv"], mask, mi.kind,
                                     max_q, max_kv, w.scale, out_dtype=torch.float32)
    # the allocation-free one, straight through the C ABI
    total_q, hq, d = dev["q"].shape
    o_na = torch.full_like(o_ws, float("nan"))
    l_na = torch.full_like(l_ws, float("nan"))
    st = (ctypes.c_int64 * 3)(*dev["k"].stride()[:3])
    status = L.LIB.attn_verify_tree_noalloc(
        dev["q"].data_ptr(), total_q, hq, dev["k"].data_ptr(), dev["v"].data_ptr(), dev["k"].shape[2], d,
        dev["k"].shape[1], st, dev["pt"].data_ptr(), dev["pt"].shape[1], dev["cu"].data_ptr(), dev["kv"].data_ptr(),
        w.batch, max_q, max_kv, L.KIND[mi.kind], mask.data_ptr(), mask.numel(), L.BF16, L.F32, float(w.scale),
        o_na.data_ptr(), l_na.data_ptr(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert status == L.MA_OK, L.LIB.ma_last_error()
    torch.cuda.synchronize()
    return o_ws, l_ws, o_na, l_na


@pytest.mark.parametrize("form", ["tree_packed", "tree_dense"])
def test_noalloc_matches_workspace_entry_point(form):
    big = W.config2(seed=81, batch=6, nodes=64, ctx_lo=900, ctx_hi=3000)
    small = W.config2(seed=82, batch=3, nodes=40, ctx_lo=100, ctx_hi=600)
    for w, label in ((big, "first call"), (small, "second, smaller call")):
        print("[case] noalloc", form, label, flush=True)
        max_q, max_kv = int(w.q_lens.max()), int(w.kv_lens.max())
        o_ws, l_ws, o_na, l_na = _calls(w, form, max_q, max_kv)
        assert torch.equal(o_ws, o_na), label
        assert torch.equal(l_ws, l_na), label
        ref_o, ref_l = oracle(w, form)
        assert max_abs_err(o_na, ref_o) <= TOL_BF16
        assert lse_err(l_na, ref_l) <= 1e-2


def test_noalloc_refuses_bounds_beyond_its_scratch():
    # 64 sequences of 64 queries over 32 heads and 1M keys need far more than
    # 64 MiB of split partials: a size error before any launch
    need = ma.attn_verify_tree_workspace(64, 64, 1 << 20, 32, 8, 128)
    assert need > 64 << 20
    st = (ctypes.c_int64 * 3)(2048, 128, 128)
    fake = ctypes.c_void_p(16)
    status = L.LIB.attn_verify_tree_noalloc(fake, 64 * 64, 32, fake, fake, 8, 128, 16, st, fake, 65536, fake, fake,
                                            64, 64, 1 << 20, L.KIND["packed"], fake, 1 << 30, L.BF16, L.F32, 0.1,
                                            fake, None, None)
    assert status == L.MA_ERR_SIZE
    assert "scratch" in L.LIB.ma_last_error().decode()
