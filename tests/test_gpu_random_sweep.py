"""Seeded random sweep of the GPU paths against the oracle: ragged batches
(sequences without queries or without keys included), GQA layouts, head
sizes, page sizes, tile heights and every mask input, drawn from fixed seeds
so that corners the hand-written cases miss get a chance to show: prefill,
its backward and its fp8 form, tree verify and decode.  Each case prints its
parameters before it runs."""

import numpy as np
import pytest
import torch

import masked_flash_attention_mask_amd as ma
import workloads as W
from helpers import (TOL_BF16, TOL_GRAD, compile_plan, device_inputs, fp8_dequantized, grad_err, lse_err, max_abs_err,
                     oracle, oracle_masks, repage, run_prefill)
from oracle import backward as OB
from test_gpu_fp8 import _check as fp8_check, _dev8, _run as fp8_run

pytestmark = pytest.mark.gpu

HEADS = [(4, 2), (8, 8), (6, 3), (8, 1)]
KINDS = ["causal", "window", "prefix", "ranges", "dense", "packed", "block_sparse", "dense_window"]


def _say(*a):
    print("[case]", *a, flush=True)


def _ranges(rng, q, k):
    out = []
    if q == 0 or k == 0:
        return out
    for _ in range(int(rng.integers(0, 4))):
        q0 = int(rng.integers(0, q))
        q1 = int(rng.integers(q0 + 1, q + 1))
        k0 = int(rng.integers(0, k))
        k1 = int(rng.integers(k0 + 1, k + 1))
        t = int(rng.integers(0, 5))
        out.append((q0, q1, k0, k1, t, int(rng.integers(1, 9)) if t == W.R_CHUNK_CAUSAL else 0))
    return out


def _bsr(rng, q_lens, kv_lens, br, bc):
    """Block-row CSR over all sequences' block rows, Bernoulli(0.4) blocks in
    shuffled column order (sequences without rows or keys give none)."""
    indptr, indices = [0], []
    for q, k in zip(q_lens, kv_lens):
        nrb, ncb = -(-q // br), -(-k // bc)
        for _ in range(nrb):
            cols = list(np.flatnonzero(rng.random(ncb) < 0.4))
            rng.shuffle(cols)
            indices += cols
            indptr.append(len(indices))
    return np.array(indptr, np.int32), np.array(indices, np.int32)


def _prefill_case(seed, min_window=1):
    rng = np.random.default_rng(1000 + seed)
    b = int(rng.integers(1, 5))
    q_lens = [int(x) for x in rng.integers(0, 260, b)]
    kv_lens = [int(x) for x in rng.integers(0, 600, b)]
    if sum(q_lens) == 0:
        q_lens[0] = 17
    hq, hkv = HEADS[int(rng.integers(len(HEADS)))]
    d = int(rng.choice([64, 128, 256]))
    tile_q = int(rng.choice([64, 128]))
    page = int(rng.choice([1, 4, 16, 64]))
    kind = KINDS[seed % len(KINDS)]
    w = W.gen._build(f"sweep{seed}", W.rng_for(2000 + seed), "bf16", q_lens, kv_lens, hq, hkv, d, permute=True)
    if kind == "causal":
        mi = W.MaskInput("causal")
    elif kind == "window":
        mi = W.MaskInput("window", window=int(rng.integers(min_window, 300)))
    elif kind == "prefix":
        mi = W.MaskInput("prefix_lm", prefix_len=np.array([int(rng.integers(0, k + 1)) for k in kv_lens], np.int32))
    elif kind == "ranges":
        mi = W.MaskInput("ranges", ranges=[_ranges(rng, q, k) for q, k in zip(q_lens, kv_lens)])
    elif kind == "block_sparse":
        br, bc = [(64, 64), (16, 48), (128, 128)][int(rng.integers(3))]
        mi = W.MaskInput("block_sparse", bsr=(br, bc) + _bsr(rng, q_lens, kv_lens, br, bc))
    else:
        rows = [rng.random((q, k)) < float(rng.uniform(0.05, 0.95)) for q, k in zip(q_lens, kv_lens)]
        window = int(rng.integers(min_window, 200)) if kind == "dense_window" else 0
        if kind == "packed":
            mi = W.MaskInput("packed", data=np.concatenate(
                [W.pack_rows(r).reshape(-1) for r in rows] + [np.zeros(0, np.uint64)]))
        else:
            mi = W.MaskInput("dense", data=np.concatenate([r.astype(np.uint8).reshape(-1) for r in rows]),
                             window=window)
    w.masks["m"] = mi
    if page != w.page_size:
        w = repage(w, page, 3000 + seed)
    return w, dict(seed=seed, q_lens=q_lens, kv_lens=kv_lens, hq=hq, hkv=hkv, d=d, tile_q=tile_q, page=page,
                   kind=kind)


@pytest.mark.parametrize("seed", range(32))
def test_prefill_random_sweep(seed):
    w, desc = _prefill_case(seed)
    _say("prefill sweep", desc)
    out, lse, _ = run_prefill(w, device_inputs(w), "m", tile_q=desc["tile_q"])
    ref_o, ref_l = oracle(w, "m")
    err = max_abs_err(out, ref_o)
    assert err <= TOL_BF16, (desc, err)
    assert lse_err(lse, ref_l) <= 1e-2, desc


def _verify_case(seed):
    rng = np.random.default_rng(4000 + seed)
    b = int(rng.integers(1, 10))
    max_q = int(rng.choice([8, 33, 64]))
    q_lens = [int(x) for x in rng.integers(0, max_q + 1, b)]
    if sum(q_lens) == 0:
        q_lens[0] = max_q
    ctx = [int(x) for x in rng.integers(0, 3000, b)]
    kv_lens = [c + q for c, q in zip(ctx, q_lens)]
    hq, hkv = [(8, 2), (32, 8), (4, 4), (16, 2)][int(rng.integers(4))]
    d = int(rng.choice([64, 128, 256]))
    page = int(rng.choice([4, 16, 64]))
    w = W.gen._build(f"vsweep{seed}", W.rng_for(5000 + seed), "bf16", q_lens, kv_lens, hq, hkv, d, permute=True)
    rows = []
    for q, c in zip(q_lens, ctx):
        # a random tree over the q draft nodes after the context: each node
        # sees the context, its ancestors and itself
        m = np.zeros((q, c + q), dtype=bool)
        m[:, :c] = True
        parent = [-1] + [int(rng.integers(0, n)) for n in range(1, q)]
        for n in range(q):
            a = n
            while a >= 0:
                m[n, c + a] = True
                a = parent[a]
        rows.append(m)
    w.masks["dense"] = W.MaskInput("dense", data=np.concatenate([r.astype(np.uint8).reshape(-1) for r in rows]))
    w.masks["packed"] = W.MaskInput("packed", data=np.concatenate(
        [W.pack_rows(r).reshape(-1) for r in rows] + [np.zeros(0, np.uint64)]))
    if page != w.page_size:
        w = repage(w, page, 6000 + seed)
    return w, dict(seed=seed, q_lens=q_lens, kv_lens=kv_lens, max_q=max_q, hq=hq, hkv=hkv, d=d, page=page)


@pytest.mark.parametrize("seed", range(16))
def test_verify_random_sweep(seed):
    w, desc = _verify_case(seed)
    _say("verify sweep", desc)
    dev = device_inputs(w)
    outs = {}
    for form in ("packed", "dense"):
        mi = w.masks[form]
        data = mi.data if mi.kind == "dense" else mi.data.view(np.int64)
        mask = torch.from_numpy(np.ascontiguousarray(data)).cuda()
        outs[form] = ma.attn_verify_tree(dev["q"], dev["k"], dev["v"], dev["pt"], dev["cu"], dev["kv"], mask,
                                         mi.kind, desc["max_q"], int(w.kv_lens.max()), w.scale)
        torch.cuda.synchronize()
    assert torch.equal(outs["packed"][0], outs["dense"][0]), desc
    assert torch.equal(outs["packed"][1], outs["dense"][1]), desc
    ref_o, ref_l = oracle(w, "packed")
    err = max_abs_err(outs["packed"][0], ref_o)
    assert err <= TOL_BF16, (desc, err)
    assert lse_err(outs["packed"][1], ref_l) <= 1e-2, desc
    # the same rows under masks given by position (the tree-verify shapes take
    # the balanced kernel with computed words)
    prefix = np.array([int(x) for x in np.random.default_rng(4500 + seed).integers(0, np.asarray(w.kv_lens) + 1)],
                      dtype=np.int32)
    w.masks["causal"] = W.MaskInput("causal")
    w.masks["prefix"] = W.MaskInput("prefix_lm", prefix_len=prefix)
    w.masks["window"] = W.MaskInput("window", window=int(np.random.default_rng(4600 + seed).integers(1, 1500)))
    for name in ("causal", "prefix", "window"):
        mi = w.masks[name]
        pl = torch.from_numpy(prefix).cuda() if mi.kind == "prefix_lm" else None
        o, l = ma.attn_decode(dev["q"], dev["k"], dev["v"], dev["pt"], dev["cu"], dev["kv"], desc["max_q"],
                              int(w.kv_lens.max()), w.scale, mask_kind=mi.kind, window=mi.window, prefix_len=pl)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle(w, name)
        err = max_abs_err(o, ref_o)
        assert err <= TOL_BF16, (desc, name, err)
        assert lse_err(l, ref_l) <= 1e-2, (desc, name)


@pytest.mark.parametrize("seed", range(16))
def test_backward_random_sweep(seed):
    """The prefill sweep's shapes and masks through the backward, the
    oracle's forward outputs in.  Windows of at least 2 keys: under a 1-key
    window every row has a single visible key, its exact dS and dQ are zero,
    and an error relative to the gradient's own scale means nothing."""
    w, desc = _prefill_case(seed, min_window=2)
    _say("backward sweep", desc)
    do = W.upstream_grad(w, 7000 + seed)
    dev = device_inputs(w)
    dev["do"] = torch.from_numpy(do).cuda().to(torch.bfloat16).contiguous()
    o, l = oracle(w, "m")
    out = torch.from_numpy(o.astype(np.float32)).cuda().contiguous()
    lse = torch.from_numpy(l.astype(np.float32)).cuda().contiguous()
    plan = compile_plan(w, "m", desc["tile_q"])
    dq, dk, dv = ma.attn_backward_masked(plan, dev["q"], dev["k"], dev["v"], dev["pt"], out, lse, dev["do"], w.scale)
    torch.cuda.synchronize()
    rq, rk, rv = OB.attention_backward(w.q, w.k_cache, w.v_cache, w.page_table, w.cu_seqlens_q, w.kv_lens,
                                       oracle_masks(w, "m"), w.scale, do)
    used = np.zeros(w.k_cache.shape[:2], bool)
    for b, kl in enumerate(w.kv_lens):
        j = np.arange(int(kl))
        used[w.page_table[b, j // w.page_size], j % w.page_size] = True
    keep = used[..., None, None]
    for g, r, what in ((dq, rq, "dq"), (torch.from_numpy(np.where(keep, dk.cpu().numpy(), 0.0)), rk, "dk"),
                       (torch.from_numpy(np.where(keep, dv.cpu().numpy(), 0.0)), rv, "dv")):
        err = grad_err(g, r)
        assert err <= TOL_GRAD, (desc, what, err)


@pytest.mark.parametrize("seed", range(16))
def test_fp8_random_sweep(seed):
    """The prefill sweep's shapes and masks with e4m3 inputs (pages of at
    least 16 keys, 128-row tiles), within the derived e4m3 rounding bound."""
    w, desc = _prefill_case(seed)
    if w.page_size < 16:
        w = repage(w, 16, 8000 + seed)
        desc["page"] = 16
    desc["tile_q"] = 128
    _say("fp8 sweep", desc)
    f8 = W.fp8_inputs(w)
    out, lse = fp8_run(w, f8, _dev8(w, f8), "m")
    fp8_check(w, fp8_dequantized(w, f8), "m", out, lse)


@pytest.mark.parametrize("seed", range(16))
def test_decode_random_sweep(seed):
    """The verify sweep's shapes (up to 64 queries per sequence) through
    decode under causal, window, PrefixLM, dense and packed rows."""
    w, desc = _verify_case(seed)
    rng = np.random.default_rng(9000 + seed)
    kind = ["causal", "window", "prefix", "dense", "packed"][seed % 5]
    ql, kl = [int(x) for x in w.q_lens], [int(x) for x in w.kv_lens]
    kw = {}
    if kind == "causal":
        mi = W.MaskInput("causal")
    elif kind == "window":
        mi = W.MaskInput("window", window=int(rng.integers(1, 400)))
        kw["window"] = mi.window
    elif kind == "prefix":
        mi = W.MaskInput("prefix_lm", prefix_len=np.array([int(rng.integers(0, k + 1)) for k in kl], np.int32))
        kw["prefix_len"] = torch.from_numpy(mi.prefix_len).cuda()
    else:
        rows = [rng.random((q, k)) < 0.4 for q, k in zip(ql, kl)]
        if kind == "dense":
            mi = W.MaskInput("dense", data=np.concatenate([r.astype(np.uint8).reshape(-1) for r in rows]))
            kw["mask"] = torch.from_numpy(mi.data).cuda()
        else:
            mi = W.MaskInput("packed", data=np.concatenate(
                [W.pack_rows(r).reshape(-1) for r in rows] + [np.zeros(0, np.uint64)]))
            kw["mask"] = torch.from_numpy(np.ascontiguousarray(mi.data.view(np.int64))).cuda()
    w.masks["m"] = mi
    desc["kind"] = kind
    _say("decode sweep", desc)
    dev = device_inputs(w)
    out, lse = ma.attn_decode(dev["q"], dev["k"], dev["v"], dev["pt"], dev["cu"], dev["kv"], desc["max_q"],
                              int(w.kv_lens.max()), w.scale, mask_kind=mi.kind, **kw)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle(w, "m")
    err = max_abs_err(out, ref_o)
    assert err <= TOL_BF16, (desc, err)
    assert lse_err(lse, ref_l) <= 1e-2, desc
