"""GPU parity of masked decode (HIP path through the C ABI) against the fp64
oracle: ragged q_len 1..8 against ragged paged contexts (tails, one-key
contexts, contexts long enough to split), every mask kind, GQA and MHA."""

import numpy as np
import pytest
import torch

import masked_flash_attention_mask_amd as ma
import workloads as W
from helpers import TOL_BF16, bf16_out_err, device_inputs, lse_err, max_abs_err, oracle, repage
from oracle import masks as OM

pytestmark = pytest.mark.gpu

Q_LENS = [1, 1, 3, 8, 2]
KV_LENS = [1, 64, 700, 2100, 130]


def _say(*a):
    print("[case]", *a, flush=True)


def _workload(seed, d, hq, hkv):
    rng = W.rng_for(seed)
    w = W.gen._build(f"decode{seed}", rng, "bf16", Q_LENS, KV_LENS, hq, hkv, d, permute=True)
    mrng = np.random.default_rng(seed + 1)
    prefix = np.array([mrng.integers(0, k + 1) for k in KV_LENS], np.int32)
    dense = []
    for q, k in zip(Q_LENS, KV_LENS):
        m = mrng.random((q, k)) < 0.3
        m[:, k - 1] = True                   # every row sees its last key
        dense.append(m)
    w.masks["causal"] = W.MaskInput("causal")
    w.masks["window"] = W.MaskInput("window", window=37)
    w.masks["wide_window"] = W.MaskInput("window", window=5000)
    w.masks["prefix"] = W.MaskInput("prefix_lm", prefix_len=prefix)
    w.masks["dense"] = W.MaskInput("dense", data=np.concatenate([m.astype(np.uint8).reshape(-1) for m in dense]))
    w.masks["packed"] = W.MaskInput("packed", data=np.concatenate([W.pack_rows(m).reshape(-1) for m in dense]))
    causal = [OM.causal(q, k) for q, k in zip(Q_LENS, KV_LENS)]
    w.masks["causal_dense"] = W.MaskInput(
        "dense", data=np.concatenate([m.astype(np.uint8).reshape(-1) for m in causal]))
    return w


def _decode(w, dev, name, out_dtype=torch.float32):
    mi = w.masks[name]
    kw = {}
    if mi.kind == "window":
        kw["window"] = mi.window
    elif mi.kind == "prefix_lm":
        kw["prefix_len"] = torch.from_numpy(mi.prefix_len).cuda()
    elif mi.kind in ("dense", "packed"):
        data = mi.data if mi.kind == "dense" else mi.data.view(np.int64)
        kw["mask"] = torch.from_numpy(np.ascontiguousarray(data)).cuda()
    out, lse = ma.attn_decode(dev["q"], dev["k"], dev["v"], dev["pt"], dev["cu"], dev["kv"], max(Q_LENS),
                              max(KV_LENS), w.scale, mask_kind=mi.kind, out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("d,hq,hkv", [(64, 8, 2), (128, 8, 2), (128, 4, 4), (256, 4, 1)])
def test_decode_mask_kinds(d, hq, hkv):
    w = _workload(700 + d + hq, d, hq, hkv)
    dev = device_inputs(w)
    for name in ("causal", "window", "wide_window", "prefix", "dense", "packed"):
        _say("decode", d, hq, hkv, name)
        out, lse = _decode(w, dev, name)
        ref_o, ref_l = oracle(w, name)
        err = max_abs_err(out, ref_o)
        assert err <= TOL_BF16, (name, err)
        assert lse_err(lse, ref_l) <= 1e-2, name


def _rounding_bound(w, name):
    """Per output element, the most two roundings of the probabilities to
    bf16 can move O apart.  With weights w_j = p_j / sum p (fp64 oracle) and
    each probability rounded to p_j (1 + e_j), |e_j| <= u = 2^-9, the output
    sum_j p_j (1 + e_j) v_j / sum_j p_j (1 + e_j) differs from the exact O by
    sum_j w_j e_j (v_j - O) / (1 + sum_j w_j e_j), at most
    u / (1 - u) * sum_j w_j |v_j - O|; two kernels that round against
    different references are at most twice that apart.  Plus 1e-5 for the
    fp32 sums and exponentials."""
    from oracle import attention as OA
    from helpers import oracle_masks
    u = 2.0 ** -9
    masks = oracle_masks(w, name)
    bound = np.zeros(w.q.shape, dtype=np.float64)
    for b in range(w.batch):
        q0, q1, kl = int(w.cu_seqlens_q[b]), int(w.cu_seqlens_q[b + 1]), int(w.kv_lens[b])
        mk = masks(b)
        for h in range(w.hq):
            g = h // (w.hq // w.hkv)
            k = OA.gather_paged(w.k_cache, w.page_table[b], kl, g)
            v = OA.gather_paged(w.v_cache, w.page_table[b], kl, g)
            s = w.scale * (np.asarray(w.q[q0:q1, h], np.float64) @ k.T)
            s = np.where(mk, s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            wt = p / p.sum(axis=1, keepdims=True)
            o = wt @ v
            spread = np.einsum("tj,tjd->td", wt, np.abs(v[None, :, :] - o[:, None, :]))
            bound[q0:q1, h] = 2 * u / (1 - u) * spread + 1e-5
    return bound


def test_decode_equivalent_forms_agree():
    """Equal masks in forms that take the same kernel give identical outputs:
    a window wider than every context vs causal (both positional), dense vs
    packed (both read mask words). Positional masks at d <= 128 spread one
    split's tiles over the workgroup's waves and merge the waves' partial
    states, while the word-reading forms walk the tiles in order, so causal
    vs its dense rows agrees only to the rounding of the bf16 probabilities
    (each wave rounds them against its own running maximum): every element
    within the bound two such roundings allow (_rounding_bound)."""
    w = _workload(801, 128, 8, 2)
    dev = device_inputs(w)
    c, lc = _decode(w, dev, "causal")
    o, lo = _decode(w, dev, "wide_window")
    assert torch.equal(o, c) and torch.equal(lo, lc)
    o, lo = _decode(w, dev, "causal_dense")
    diff = np.abs(o.cpu().numpy().astype(np.float64) - c.cpu().numpy().astype(np.float64))
    bound = _rounding_bound(w, "causal")
    e_l = lse_err(lo, lc.cpu().numpy().astype(np.float64))
    _say("causal vs causal_dense: worst diff / bound", float((diff / bound).max()), "lse", e_l)
    assert (diff <= bound).all(), float((diff / bound).max())
    assert e_l <= 1e-4, e_l
    o1, l1 = _decode(w, dev, "dense")
    o2, l2 = _decode(w, dev, "packed")
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("d", [64, 128])
def test_decode_page_sizes(d):
    """Positional-mask decode over pages of 1 to 256 keys in a random order
    (spare pages NaN).  Pages holding a whole gather instruction's rows
    (512 / d keys) take the wave-split kernel, smaller ones the kernel whose
    waves share each tile; every page size matches the oracle, and the
    wave-split results do not depend on the page size."""
    w = _workload(803, d, 8, 2)
    names = ("causal", "window", "prefix")
    ref = {n: oracle(w, n) for n in names}
    first = {}
    for ps in (1, 4, 16, 64, 256):
        wp = repage(w, ps, 900 + ps)
        dev = device_inputs(wp)
        for n in names:
            _say("decode pages", d, ps, n)
            o, lse = _decode(wp, dev, n)
            assert max_abs_err(o, ref[n][0]) <= TOL_BF16, (ps, n)
            assert lse_err(lse, ref[n][1]) <= 1e-2, (ps, n)
            if ps >= 512 // d:
                if n in first:
                    assert torch.equal(o, first[n][0]) and torch.equal(lse, first[n][1]), (ps, n)
                else:
                    first[n] = (o, lse)


def test_decode_bf16_output_and_window_bites():
    w = _workload(802, 128, 8, 2)
    dev = device_inputs(w)
    ob, _ = _decode(w, dev, "window", out_dtype=torch.bfloat16)
    assert ob.dtype == torch.bfloat16
    ref_o, _ = oracle(w, "window")
    assert bf16_out_err(ob, ref_o) <= TOL_BF16
    # the 37-key window changes the long sequences' outputs
    oc, _ = _decode(w, dev, "causal")
    ow, _ = _decode(w, dev, "window")
    rows = slice(int(w.cu_seqlens_q[3]), int(w.cu_seqlens_q[4]))
    assert (oc[rows] - ow[rows]).abs().max().item() > 0.05


def test_decode_workspace_and_validation():
    assert ma.attn_decode_workspace(8, 1, 32768, 32, 8, 128) > 0
    assert ma.attn_decode_workspace(8, 1, 64, 32, 8, 128) == 0
    w = _workload(803, 64, 4, 2)
    dev = device_inputs(w)
    with pytest.raises(ma.MaskAttnError):
        ma.attn_decode(dev["q"], dev["k"], dev["v"], dev["pt"], dev["cu"], dev["kv"], max(Q_LENS), max(KV_LENS),
                       w.scale, mask_kind="window", window=0)
    with pytest.raises(ma.MaskAttnError):
        ma.attn_decode(dev["q"], dev["k"], dev["v"], dev["pt"], dev["cu"], dev["kv"], max(Q_LENS), max(KV_LENS),
                       w.scale, mask_kind="prefix_lm")


def test_decode_full_size_sampled():
    """The decode workload at full size (16 sequences, contexts 4k-16k, 4
    queries each): causal and a 4096-key window, oracle on sampled heads."""
    w = W.decode(q_len=4)
    dev = device_inputs(w)
    max_kv = int(w.kv_lens.max())
    rows = {b: np.arange(4) for b in (0, 5, 15)}
    for name in ("causal", "window"):
        _say("decode full", name)
        win = w.masks[name].window if name == "window" else 0
        out, lse = ma.attn_decode(dev["q"], dev["k"], dev["v"], dev["pt"], dev["cu"], dev["kv"], 4, max_kv,
                                  w.scale, mask_kind=name, window=win)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle(w, name, heads=[0, 13, 31], rows=rows)
        assert max_abs_err(out, ref_o) <= TOL_BF16, name
        assert lse_err(lse, ref_l) <= 1e-2, name
