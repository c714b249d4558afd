"""GPU parity of the balanced tree-verify path (work split over the device
lengths into equal tile ranges, four-stage pipeline, cut units merged in tile
order) against the oracle: ragged batches with empty sequences, more than 64
sequences, one-tile and long contexts, GQA groups wider than a unit, head dims
64 and 128, pages whose gathers take each form, dense and packed masks (the
dense rows become packed words first, so the two give identical bits)."""

import numpy as np
import pytest
import torch

import masked_flash_attention_mask_amd as ma
import workloads as W
from helpers import OM, TOL_BF16, bf16_out_err, device_inputs, lse_err, max_abs_err, oracle, repage

pytestmark = pytest.mark.gpu


def _workload(seed, q_lens, kv_lens, hq, hkv, d, p_visible=0.6):
    """Ragged queries at the end of their contexts; each query row sees every
    context key before the queries and a Bernoulli(p_visible) subset of the
    query keys, itself always (tree-like rows, some rows longer than others)."""
    rng = W.rng_for(seed)
    w = W.gen._build(f"bal{seed}", rng, "bf16", q_lens, kv_lens, hq, hkv, d, permute=True)
    rows = []
    for ql, kl in zip(q_lens, kv_lens):
        m = np.zeros((ql, kl), dtype=bool)
        ctx = kl - ql          # negative: more queries than keys
        lo = max(ctx, 0)
        m[:, :lo] = True
        if ql and kl:
            m[:, lo:] = rng.random((ql, kl - lo)) < p_visible
            t = np.arange(ql)
            own = ctx + t >= 0
            m[t[own], ctx + t[own]] = True
        rows.append(m)
    w.masks["dense"] = W.gen.MaskInput("dense", data=np.concatenate([r.astype(np.uint8).reshape(-1) for r in rows]))
    w.masks["packed"] = W.gen.MaskInput("packed", data=np.concatenate(
        [W.pack_rows(r).reshape(-1) for r in rows]) if rows else np.zeros(0, np.uint64))
    return w


def _run(w, dev, form, max_q, out_dtype=torch.float32):
    mi = w.masks[form]
    data = mi.data if mi.kind == "dense" else mi.data.view(np.int64)
    mask = torch.from_numpy(np.ascontiguousarray(data)).cuda()
    out, lse = ma.attn_verify_tree(dev["q"], dev["k"], dev["v"], dev["pt"], dev["cu"], dev["kv"], mask, mi.kind,
                                   max_q, int(w.kv_lens.max()), w.scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, lse


CASES = [
    # (seed, q_lens, kv_lens, hq, hkv, d, page)
    (1, [40] * 70, None, 8, 2, 128, 16),                              # 70 sequences, short contexts
    (2, [64, 0, 64, 17], [5000, 0, 64, 2100], 16, 2, 64, 16),         # empty sequence, one-tile context
    (3, [64, 64, 50], [3000, 700, 4100], 8, 2, 128, 4),               # 4-key pages: per-lane gathers
    (4, [64, 33, 64], [1200, 3300, 200], 32, 8, 128, 8),              # 8-key pages: one page per wave
]


@pytest.mark.parametrize("case", CASES, ids=[f"seed{c[0]}" for c in CASES])
def test_balanced_verify_matches_oracle(case):
    seed, q_lens, kv_lens, hq, hkv, d, page = case
    if kv_lens is None:
        kv_lens = list(W.rng_for(100 + seed).integers(40, 400, size=len(q_lens)))
    print("[case] balanced verify", seed, hq, hkv, d, page, flush=True)
    w = _workload(seed, q_lens, kv_lens, hq, hkv, d)
    if page != w.page_size:
        w = repage(w, page, 300 + seed)
    dev = device_inputs(w)
    max_q = max(max(q_lens), 1)
    o_p, l_p = _run(w, dev, "packed", max_q)
    o_d, l_d = _run(w, dev, "dense", max_q)
    assert torch.equal(o_p, o_d) and torch.equal(l_p, l_d)
    o2, l2 = _run(w, dev, "packed", max_q)
    assert torch.equal(o_p, o2) and torch.equal(l_p, l2)          # deterministic
    ref_o, ref_l = oracle(w, "packed")
    assert max_abs_err(o_p, ref_o) <= TOL_BF16
    assert lse_err(l_p, ref_l) <= 1e-2
    # a bf16 output merges bf16 partials: against the oracle after the output
    # rounding, and within two bf16 roundings of the fp32 output
    ob, _ = _run(w, dev, "packed", max_q, out_dtype=torch.bfloat16)
    assert bf16_out_err(ob, ref_o) <= TOL_BF16
    assert (ob.float() - o_p).abs().max().item() <= 2 ** -7 * max(1.0, o_p.abs().max().item())


POS_CASES = CASES + [
    (5, [64, 64, 40], [30, 500, 40], 32, 8, 128, 16),               # more queries than keys: rows see nothing
]


@pytest.mark.parametrize("case", POS_CASES, ids=[f"seed{c[0]}" for c in POS_CASES])
def test_balanced_positional_masks(case):
    """Causal and PrefixLM rows take the balanced kernel with each row's word
    computed from its position: bit-identical to the same masks given as
    packed rows.  Sliding windows keep the split kernel (its walk starts at
    the window): within the bf16 bound of the packed rows.  All within the
    bf16 bound of the oracle."""
    seed, q_lens, kv_lens, hq, hkv, d, page = case
    if kv_lens is None:
        kv_lens = list(W.rng_for(100 + seed).integers(40, 400, size=len(q_lens)))
    print("[case] balanced positional", seed, hq, hkv, d, page, flush=True)
    w = _workload(seed, q_lens, kv_lens, hq, hkv, d)
    if page != w.page_size:
        w = repage(w, page, 300 + seed)
    dev = device_inputs(w)
    max_q, max_kv = max(max(q_lens), 1), int(max(kv_lens))
    prefix = np.array([int(W.rng_for(700 + seed).integers(0, k + 1)) for k in kv_lens], dtype=np.int32)
    w.masks["causal"] = W.gen.MaskInput("causal")
    w.masks["prefix"] = W.gen.MaskInput("prefix_lm", prefix_len=prefix)
    w.masks["window"] = W.gen.MaskInput("window", window=37)
    w.masks["wide_window"] = W.gen.MaskInput("window", window=700)
    for name, build in (("causal", lambda q, k, b: OM.causal(q, k)),
                        ("prefix", lambda q, k, b: OM.prefix_lm(q, k, int(prefix[b]))),
                        ("window", lambda q, k, b: OM.sliding_window(q, k, 37)),
                        ("wide_window", lambda q, k, b: OM.sliding_window(q, k, 700))):
        mi = w.masks[name]
        pl = torch.from_numpy(prefix).cuda() if mi.kind == "prefix_lm" else None
        o_pos, l_pos = ma.attn_decode(dev["q"], dev["k"], dev["v"], dev["pt"], dev["cu"], dev["kv"], max_q, max_kv,
                                      w.scale, mask_kind=mi.kind, window=mi.window, prefix_len=pl,
                                      out_dtype=torch.float32)
        rows = [build(int(q), int(k), b) for b, (q, k) in enumerate(zip(q_lens, kv_lens))]
        packed = np.concatenate([W.pack_rows(r).reshape(-1) for r in rows])
        mask = torch.from_numpy(np.ascontiguousarray(packed.view(np.int64))).cuda()
        o_pk, l_pk = ma.attn_verify_tree(dev["q"], dev["k"], dev["v"], dev["pt"], dev["cu"], dev["kv"], mask, "packed",
                                         max_q, max_kv, w.scale, out_dtype=torch.float32)
        torch.cuda.synchronize()
        if mi.kind != "window":
            assert torch.equal(o_pos, o_pk) and torch.equal(l_pos, l_pk), name
        else:
            # another kernel, other roundings
            assert (o_pos - o_pk).abs().max().item() <= TOL_BF16, name
        ref_o, ref_l = oracle(w, name)
        assert max_abs_err(o_pos, ref_o) <= TOL_BF16, name
        assert lse_err(l_pos, ref_l) <= 1e-2, name
