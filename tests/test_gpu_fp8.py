"""GPU parity of the fp8 (e4m3) prefill against the fp64 oracle run on the
exact decoded inputs, with a per-element bound derived from rounding the
probabilities to e4m3 (tests/helpers.fp8_bound); every mask kind, d 64 and
128, GQA, ragged sequences; the benchmark shape at full size, sampled."""

import numpy as np
import pytest
import torch

import masked_flash_attention_mask_amd as ma
import workloads as W
from helpers import compile_plan, fp8_bound, fp8_dequantized, oracle, oracle_masks, repage
from oracle import attention as OA

pytestmark = pytest.mark.gpu

MASKS = ("causal", "window", "prefix_lm", "ranges", "dense", "packed")


def _say(*a):
    print("[case]", *a, flush=True)


def _dev8(w, f8):
    dev = {k: torch.from_numpy(np.ascontiguousarray(f8[k])).cuda() for k in ("q8", "k8", "v8")}
    dev["pt"] = torch.from_numpy(w.page_table).cuda().contiguous()
    return dev


def _run(w, f8, dev, name, out_dtype=torch.float32):
    plan = compile_plan(w, name)
    out, lse = ma.attn_prefill_masked_fp8(plan, dev["q8"], dev["k8"], dev["v8"], dev["pt"], w.scale, f8["q_s"],
                                          f8["k_s"], f8["v_s"], out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, lse


def _check(w, wd, name, out, lse, heads=None, rows=None):
    """Compare against the oracle on the dequantized inputs, element by
    element within fp8_bound, for the given heads and per-sequence rows."""
    ref_o, ref_l = oracle(wd, name, heads=heads, rows=rows)
    g = out.float().cpu().numpy().astype(np.float64)
    masks = oracle_masks(wd, name)
    group = wd.hq // wd.hkv
    worst = 0.0
    lg_all = lse.cpu().numpy().astype(np.float64)
    for b in range(wd.batch):
        if rows is not None and b not in rows:
            continue
        q0, ql, kl = int(wd.cu_seqlens_q[b]), int(wd.q_lens[b]), int(wd.kv_lens[b])
        rs = np.arange(ql) if rows is None else np.asarray(rows[b])
        if rs.size == 0:
            continue   # a sequence without queries
        mk = masks(b)
        for h in (range(wd.hq) if heads is None else heads):
            k = OA.gather_paged(wd.k_cache, wd.page_table[b], kl, h // group)
            v = OA.gather_paged(wd.v_cache, wd.page_table[b], kl, h // group)
            o = ref_o[q0 + rs, h]
            ob, lb = fp8_bound(wd.q[q0 + rs, h], k, v, mk[rs], wd.scale, o)
            err = np.abs(g[q0 + rs, h] - o)
            assert np.isfinite(g[q0 + rs, h]).all(), (name, b, h)
            assert (err <= ob).all(), (name, b, h, float((err / ob).max()))
            worst = max(worst, float((err / ob).max()))
            lg, lr = lg_all[q0 + rs, h], ref_l[q0 + rs, h]
            assert np.array_equal(np.isneginf(lg), np.isneginf(lr)), (name, b, h)
            fin = np.isfinite(lr)
            assert (np.abs(lg[fin] - lr[fin]) <= lb[fin]).all(), (name, b, h)
    return worst


@pytest.mark.parametrize("d", [64, 128, 256])
def test_fp8_mask_kinds(d):
    w = W.backward_small(seed=90 + d, d=d, hq=4, hkv=2)
    f8 = W.fp8_inputs(w)
    wd = fp8_dequantized(w, f8)
    dev = _dev8(w, f8)
    for name in MASKS:
        _say("fp8", d, name)
        out, lse = _run(w, f8, dev, name)
        worst = _check(w, wd, name, out, lse)
        _say("worst err / bound", worst)


def test_fp8_bf16_output_and_determinism():
    w = W.backward_small(seed=95, d=128, hq=4, hkv=2)
    f8 = W.fp8_inputs(w)
    dev = _dev8(w, f8)
    o1, l1 = _run(w, f8, dev, "ranges", out_dtype=torch.bfloat16)
    o2, l2 = _run(w, f8, dev, "ranges", out_dtype=torch.bfloat16)
    of, lf = _run(w, f8, dev, "ranges")
    assert o1.dtype == torch.bfloat16 and torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(l1, lf)
    assert (o1.float() - of).abs().max().item() <= 2.0 ** -8 * of.abs().max().item() + 1e-6


def test_fp8_validation():
    w = W.backward_small(seed=96, d=128, hq=4, hkv=2)
    f8 = W.fp8_inputs(w)
    dev = _dev8(w, f8)
    plan = compile_plan(w, "causal")
    with pytest.raises(ma.MaskAttnError):
        ma.attn_prefill_masked_fp8(plan, dev["q8"], dev["k8"], dev["v8"], dev["pt"], w.scale, 0.0, 1.0, 1.0)
    plan64 = compile_plan(w, "causal", tile_q=64)
    with pytest.raises(ma.MaskAttnError):
        ma.attn_prefill_masked_fp8(plan64, dev["q8"], dev["k8"], dev["v8"], dev["pt"], w.scale, 1.0, 1.0, 1.0)
    small = dev["k8"].reshape(-1, 4, *dev["k8"].shape[2:])          # 4-key pages
    pt4 = torch.arange(small.shape[0], dtype=torch.int32, device="cuda").reshape(1, -1).repeat(w.batch, 1)
    with pytest.raises(ma.MaskAttnError):
        ma.attn_prefill_masked_fp8(plan, dev["q8"], small, small, pt4.contiguous(), w.scale, 1.0, 1.0, 1.0)


def test_fp8_full_size_sampled():
    """The benchmark shape (16384 tokens, chunk-causal cs 2, 16 heads, d 128)
    in fp8, oracle on sampled heads and rows."""
    w = W.config4(chunk_sizes=(2,))
    f8 = W.fp8_inputs(w)
    wd = fp8_dequantized(w, f8)
    dev = _dev8(w, f8)
    _say("fp8 full size")
    out, lse = _run(w, f8, dev, "chunk2")
    n = int(w.kv_lens[0])
    rows = {0: np.array([0, 1, 127, 128, 1023, 1024, 1025, 5000, 8191, n - 2, n - 1])}
    worst = _check(w, wd, "chunk2", out, lse, heads=[0, 11], rows=rows)
    _say("worst err / bound", worst)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_fp8_page_sizes_bit_identical(d):
    """Pages of the minimum size (one gather instruction's rows: 4 keys at
    d 256, 8 at d 128, 16 at d 64), 16, 32 and 64 keys (one page per wave's run from 16
    keys on): the page layout does not enter the arithmetic, so the outputs
    are bit-identical; the first is also held to the oracle bound."""
    base = W.backward_small(seed=97 + d, d=d, hq=4, hkv=2)
    f8 = W.fp8_inputs(base)
    name = "ranges"
    outs = {}
    for ps in sorted({1024 // d, 16, 32, 64}):
        w = base if ps == base.page_size else repage(base, ps, 700 + ps)
        g8 = W.fp8_inputs(w)
        assert g8["k_s"] == f8["k_s"] and g8["v_s"] == f8["v_s"]   # same values, other layout
        _say("fp8 page size", d, ps)
        out, lse = _run(w, g8, _dev8(w, g8), name)
        outs[ps] = (out.cpu(), lse.cpu())
    first = 1024 // d
    for ps in outs:
        assert torch.equal(outs[ps][0], outs[first][0]) and torch.equal(outs[ps][1], outs[first][1]), ps
    _check(base, fp8_dequantized(base, f8), name, outs[16][0], outs[16][1])


def test_fp8_gemma2_global_sampled():
    """The Gemma2-like global layer (16384 tokens, causal, 8 query heads over
    4 K/V heads, d 256, random page order) in fp8, oracle on sampled heads
    and rows."""
    w = W.config3b(1)
    f8 = W.fp8_inputs(w)
    wd = fp8_dequantized(w, f8)
    dev = _dev8(w, f8)
    _say("fp8 d 256 global layer")
    out, lse = _run(w, f8, dev, "causal")
    n = int(w.kv_lens[0])
    rows = {0: np.array([0, 1, 63, 64, 127, 128, 4095, 4096, 9000, n - 2, n - 1])}
    worst = _check(w, wd, "causal", out, lse, heads=[0, 5], rows=rows)
    _say("worst err / bound", worst)
