"""GPU parity of speculative tree verify (device lengths, on-the-fly mask
classification, split K/V with a fixed-order merge) against the oracle."""

import numpy as np
import pytest
import torch

import masked_flash_attention_mask_amd as ma
import workloads as W
from helpers import TOL_BF16, bf16_out_err, device_inputs, lse_err, max_abs_err, oracle

pytestmark = pytest.mark.gpu


def _run(w, dev, form, out_dtype=torch.float32):
    mi = w.masks[form]
    data = mi.data if mi.kind == "dense" else mi.data.view(np.int64)
    mask = torch.from_numpy(np.ascontiguousarray(data)).cuda()
    out, lse = ma.attn_verify_tree(dev["q"], dev["k"], dev["v"], dev["pt"], dev["cu"], dev["kv"], mask, mi.kind,
                                   int(w.q_lens.max()), int(w.kv_lens.max()), w.scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, lse


def test_config2_full():
    w = W.config2()
    print("[case] cfg2 full", flush=True)
    dev = device_inputs(w)
    o_p, l_p = _run(w, dev, "tree_packed")
    o_d, l_d = _run(w, dev, "tree_dense")
    assert torch.equal(o_p, o_d) and torch.equal(l_p, l_d)
    ref_o, ref_l = oracle(w, "tree_packed")
    assert max_abs_err(o_p, ref_o) <= TOL_BF16
    assert lse_err(l_p, ref_l) <= 1e-2
    o2, l2 = _run(w, dev, "tree_packed")
    assert torch.equal(o_p, o2) and torch.equal(l_p, l2)
    ob, _ = _run(w, dev, "tree_packed", out_dtype=torch.bfloat16)
    assert bf16_out_err(ob, ref_o) <= TOL_BF16


@pytest.mark.parametrize("nodes,ctx_lo,ctx_hi,hq,hkv,d", [
    (7, 10, 100, 4, 4, 64), (64, 1, 64, 8, 2, 128), (33, 200, 900, 6, 2, 128), (64, 300, 1500, 4, 2, 256)])
def test_verify_small_shapes(nodes, ctx_lo, ctx_hi, hq, hkv, d):
    w = W.config2(seed=nodes + d, batch=3, nodes=nodes, ctx_lo=ctx_lo, ctx_hi=ctx_hi, hq=hq, hkv=hkv, d=d)
    print("[case] verify", nodes, ctx_lo, ctx_hi, hq, hkv, d, flush=True)
    dev = device_inputs(w)
    ref_o, ref_l = oracle(w, "tree_packed")
    for form in ("tree_packed", "tree_dense"):
        o, l = _run(w, dev, form)
        assert max_abs_err(o, ref_o) <= TOL_BF16
        assert lse_err(l, ref_l) <= 1e-2


def test_verify_matches_prefill_over_device_plan():
    w = W.config2(seed=21, batch=2, ctx_lo=100, ctx_hi=700)
    dev = device_inputs(w)
    o1, _ = _run(w, dev, "tree_packed")
    mask = torch.from_numpy(w.masks["tree_packed"].data.view(np.int64)).cuda()
    plan = ma.mask_compile("packed", w.cu_seqlens_q, w.kv_lens, mask=mask, tile_q=64)
    o2, _ = ma.attn_prefill_masked(plan, dev["q"], dev["k"], dev["v"], dev["pt"], w.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert (o1 - o2).abs().max().item() <= 2e-3
