"""GPU parity of speculative tree verify (device lengths, on-the-fly mask
classification, split K/V with a fixed-order merge) against the oracle."""

import numpy as np
import pytest
import torch

import masked_flash_attention_mask_amd as ma
import workloads as W
from helpers import TOL_BF16, bf16_out_err, device_inputs, lse_err, max_abs_err, oracle, parity_report

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
    parity_report("cfg2 tree packed = dense, every element", max_abs_err=max_abs_err(o_p, ref_o),
                  lse_err=lse_err(l_p, ref_l))
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


@pytest.mark.parametrize("form", ["tree_packed", "tree_dense"])
def test_short_mask_reads_missing_elements_as_masked(form):
    """A mask buffer shorter than its sequences need (lengths are on the
    device, the host cannot check the exact size): elements at or past
    mask_numel read as 0, so the result equals the oracle over the same mask
    with those elements cleared (rows that lose every key give O = 0 and
    LSE = -inf)."""
    w = W.config2(seed=77, batch=3, nodes=20, ctx_lo=50, ctx_hi=200, hq=8, hkv=2, d=128)
    print("[case] short mask", form, flush=True)
    dev = device_inputs(w)
    mi = w.masks[form]
    keep = mi.data.size - mi.data.size // 5          # drop the last fifth of the buffer
    short = mi.data[:keep]
    data = short if mi.kind == "dense" else short.view(np.int64)
    mask = torch.from_numpy(np.ascontiguousarray(data)).cuda()
    out, lse = ma.attn_verify_tree(dev["q"], dev["k"], dev["v"], dev["pt"], dev["cu"], dev["kv"], mask, mi.kind,
                                   int(w.q_lens.max()), int(w.kv_lens.max()), w.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    cleared = mi.data.copy()
    cleared[keep:] = 0
    w.masks["cleared"] = W.gen.MaskInput(mi.kind, data=cleared)
    ref_o, ref_l = oracle(w, "cleared")
    assert max_abs_err(out, ref_o) <= TOL_BF16
    assert lse_err(lse, ref_l) <= 1e-2
    # the last sequence lost whole rows: they are empty
    assert torch.isneginf(lse[-1]).all() and (out[-1] == 0).all()


@pytest.mark.parametrize("max_q,form", [(32, "packed"), (48, "packed"), (48, "dense")])
def test_rows_past_max_q_are_left_alone(max_q, form):
    """max_q is a host bound the device lengths may break (the host checks
    only total_q <= batch * max_q): a sequence with more queries has its first
    max_q rows computed, the others left untouched, and nothing past the
    workspace or the launch's splits is touched.  max_q 32 takes the split
    kernel (4 x 32 rows per workgroup), 48 the balanced one (4 x 48 > 128)."""
    q_lens, kv_lens = [64, 10, 12], [700, 300, 950]
    rng = W.rng_for(91)
    w = W.gen._build("maxq", rng, "bf16", q_lens, kv_lens, 8, 2, 128, permute=True)
    rows = []
    for ql, kl in zip(q_lens, kv_lens):
        m = np.zeros((ql, kl), dtype=bool)
        m[:, :kl - ql] = True
        m[:, kl - ql:] = rng.random((ql, ql)) < 0.5
        m[np.arange(ql), kl - ql + np.arange(ql)] = True
        rows.append(m)
    w.masks["dense"] = W.gen.MaskInput("dense", data=np.concatenate([r.astype(np.uint8).reshape(-1) for r in rows]))
    w.masks["packed"] = W.gen.MaskInput("packed", data=np.concatenate([W.pack_rows(r).reshape(-1) for r in rows]))
    print("[case] rows past max_q", max_q, form, flush=True)
    dev = device_inputs(w)
    mi = w.masks[form]
    data = mi.data if mi.kind == "dense" else mi.data.view(np.int64)
    mask = torch.from_numpy(np.ascontiguousarray(data)).cuda()
    out = torch.full(dev["q"].shape, 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full(dev["q"].shape[:2], 7.0, dtype=torch.float32, device="cuda")
    ma.attn_verify_tree(dev["q"], dev["k"], dev["v"], dev["pt"], dev["cu"], dev["kv"], mask, mi.kind,
                        max_q, int(w.kv_lens.max()), w.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle(w, form)
    t = np.concatenate([np.arange(n) for n in q_lens])
    keep = t < max_q
    done = torch.from_numpy(keep).cuda()
    assert max_abs_err(out[done], ref_o[keep]) <= TOL_BF16
    assert lse_err(lse[done], ref_l[keep]) <= 1e-2
    assert (out[~done] == 7.0).all() and (lse[~done] == 7.0).all()
