"""GPU parity of the masked-attention backward (HIP path through the C ABI)
against the fp64 oracle: dQ, dK and dV over ragged, paged sequences for every
mask input, GQA, both q-tile sizes, and the contract on the caches' slots."""

import numpy as np
import pytest
import torch

import masked_flash_attention_mask_amd as ma
import workloads as W
from helpers import TOL_GRAD, compile_plan, device_inputs, grad_err, oracle, oracle_masks, repage, run_prefill
from oracle import backward as OB

pytestmark = pytest.mark.gpu

MASKS = ("causal", "window", "prefix_lm", "ranges", "dense", "packed")


def _say(*a):
    print("[case]", *a, flush=True)


def _setup(d, hq=4, hkv=2, seed=7):
    w = W.backward_small(seed=seed + d, d=d, hq=hq, hkv=hkv)
    do = W.upstream_grad(w, seed + 100 + d)
    dev = device_inputs(w)
    dev["do"] = torch.from_numpy(do).cuda().to(torch.bfloat16).contiguous()
    return w, do, dev


def _fwd_oracle(w, name):
    o, lse = oracle(w, name)
    return (torch.from_numpy(o.astype(np.float32)).cuda().contiguous(),
            torch.from_numpy(lse.astype(np.float32)).cuda().contiguous())


def _bwd(w, dev, name, out, lse, tile_q=128, dk=None, dv=None):
    plan = compile_plan(w, name, tile_q)
    g = ma.attn_backward_masked(plan, dev["q"], dev["k"], dev["v"], dev["pt"], out, lse, dev["do"], w.scale,
                                dk_cache=dk, dv_cache=dv)
    torch.cuda.synchronize()
    return g


def _ref(w, do, name):
    return OB.attention_backward(w.q, w.k_cache, w.v_cache, w.page_table, w.cu_seqlens_q, w.kv_lens,
                                 oracle_masks(w, name), w.scale, do)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_backward_mask_kinds(d):
    """Oracle forward outputs in, every gradient against the oracle's."""
    w, do, dev = _setup(d)
    for name in MASKS:
        _say("backward", d, name)
        out, lse = _fwd_oracle(w, name)
        dq, dk, dv = _bwd(w, dev, name, out, lse)
        rq, rk, rv = _ref(w, do, name)
        for g, r, what in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
            err = grad_err(g, r)
            assert err <= TOL_GRAD, (name, what, err)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_backward_tile_q64_and_mha(d):
    """64-row q-tiles, and one K/V head per query head."""
    w, do, dev = _setup(d, hq=2, hkv=2, seed=17)
    for name in ("ranges", "dense"):
        _say("backward tile64", d, name)
        out, lse = _fwd_oracle(w, name)
        dq, dk, dv = _bwd(w, dev, name, out, lse, tile_q=64)
        rq, rk, rv = _ref(w, do, name)
        for g, r, what in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
            assert grad_err(g, r) <= TOL_GRAD, (name, what)


def test_backward_equal_masks_bit_identical_and_deterministic():
    """Dense bytes and packed words of one mask give identical plans, hence
    identical gradients; a second run reproduces the first bit for bit."""
    w, do, dev = _setup(128, seed=27)
    out, lse = _fwd_oracle(w, "dense")
    a = _bwd(w, dev, "dense", out, lse)
    b = _bwd(w, dev, "packed", out, lse)
    c = _bwd(w, dev, "dense", out, lse)
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y) and torch.equal(x, z)


def test_backward_slots_contract():
    """Every key below kv_len gets its slot written (0 when no query sees
    it); slots of no key keep what the caller passed."""
    w, do, dev = _setup(64, seed=37)
    name = "window"
    out, lse = _fwd_oracle(w, name)
    sentinel = 7.0
    dk0 = torch.full(dev["k"].shape, sentinel, dtype=torch.float32, device="cuda")
    dv0 = torch.full(dev["k"].shape, sentinel, dtype=torch.float32, device="cuda")
    _, dk, dv = _bwd(w, dev, name, out, lse, dk=dk0, dv=dv0)
    used = np.zeros(w.k_cache.shape[:2], bool)
    for b, kl in enumerate(w.kv_lens):
        j = np.arange(int(kl))
        used[w.page_table[b, j // w.page_size], j % w.page_size] = True
    dkn, dvn = dk.cpu().numpy(), dv.cpu().numpy()
    assert np.all(dkn[~used] == sentinel) and np.all(dvn[~used] == sentinel)
    assert not np.any(dkn[used] == sentinel) and not np.any(dvn[used] == sentinel)
    rq, rk, rv = _ref(w, do, name)
    assert grad_err(torch.from_numpy(np.where(used[..., None, None], dkn, 0.0)), rk) <= TOL_GRAD


def test_backward_empty_sequences():
    """A sequence without queries gets its keys' slots written 0, one whose
    queries have no keys gets dQ = 0 for its rows, the rest matches the
    oracle; a batch without any query row still writes dK = dV = 0 for every
    key below kv_len (dQ, dO, O, LSE and the workspace empty) and leaves the
    other slots as passed."""
    sentinel = 7.0
    for q_lens, kv_lens in (([0, 50, 40], [70, 0, 130]), ([0, 0], [5, 0])):
        _say("backward empty", q_lens, kv_lens)
        w = W.gen._build("bwd_empty", W.rng_for(60 + len(q_lens)), "bf16", q_lens, kv_lens, 4, 2, 128,
                         permute=True)
        w.masks["causal"] = W.MaskInput("causal")
        do = W.upstream_grad(w, 61)
        dev = device_inputs(w)
        dev["do"] = torch.from_numpy(do).cuda().to(torch.bfloat16).contiguous()
        out, lse = _fwd_oracle(w, "causal")
        dk0 = torch.full(dev["k"].shape, sentinel, dtype=torch.float32, device="cuda")
        dv0 = torch.full(dev["k"].shape, sentinel, dtype=torch.float32, device="cuda")
        dq, dk, dv = _bwd(w, dev, "causal", out, lse, dk=dk0, dv=dv0)
        used = np.zeros(w.k_cache.shape[:2], bool)
        for b, kl in enumerate(w.kv_lens):
            j = np.arange(int(kl))
            used[w.page_table[b, j // w.page_size], j % w.page_size] = True
        dkn, dvn = dk.cpu().numpy(), dv.cpu().numpy()
        assert np.all(dkn[~used] == sentinel) and np.all(dvn[~used] == sentinel)
        # keys of the first sequence: no query sees them
        j = np.arange(int(kv_lens[0]))
        pg, sl = w.page_table[0, j // w.page_size], j % w.page_size
        assert np.all(dkn[pg, sl] == 0) and np.all(dvn[pg, sl] == 0)
        if sum(q_lens) == 0:
            assert dq.shape[0] == 0
            continue
        assert torch.all(dq[:50] == 0)
        rq, rk, rv = _ref(w, do, "causal")
        assert grad_err(dq, rq) <= TOL_GRAD
        assert grad_err(torch.from_numpy(np.where(used[..., None, None], dkn, 0.0)), rk) <= TOL_GRAD
        assert grad_err(torch.from_numpy(np.where(used[..., None, None], dvn, 0.0)), rv) <= TOL_GRAD


def test_backward_after_gpu_forward():
    """End to end: the library's own forward (bf16 output) feeds the backward.
    D = rowsum(dO * O) then carries O's bf16 rounding, |dD| <= 2^-9
    sum |dO O| per row, and that error enters every visible dS of the row
    without cancelling; rows with few visible keys have small exact dQ, so
    dQ is held to max error <= 2^-3 of the tensor's RMS.  dK and dV sum that
    error over many rows with both signs and keep the per-row bound."""
    w, do, dev = _setup(128, seed=47)
    for name in ("causal", "ranges"):
        _say("backward e2e", name)
        out, lse, plan = run_prefill(w, dev, name, out_dtype=torch.bfloat16)
        dq, dk, dv = ma.attn_backward_masked(plan, dev["q"], dev["k"], dev["v"], dev["pt"], out, lse, dev["do"],
                                             w.scale)
        torch.cuda.synchronize()
        rq, rk, rv = _ref(w, do, name)
        for g, r, what in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
            gg = g.cpu().numpy().astype(np.float64)
            err = float(np.abs(gg - r).max() / np.sqrt((r ** 2).mean()))
            _say("e2e", name, what, "max err / rms", err, "row metric", grad_err(g, r))
            assert err <= 2.0 ** -3, (name, what, err)
            if what != "dq":
                assert grad_err(g, r) <= TOL_GRAD, (name, what)


def test_backward_rejects_unsupported():
    w, do, dev = _setup(64, seed=57)
    out, lse = _fwd_oracle(w, "causal")
    plan = compile_plan(w, "causal")
    with pytest.raises(ma.MaskAttnError):
        ma.attn_backward_masked(plan, dev["q"], dev["k"], dev["v"], dev["pt"], out, lse, dev["do"], w.scale,
                                workspace=torch.empty(8, dtype=torch.uint8, device="cuda"))


def test_backward_full_size_sampled():
    """The benchmark's backward at full size: one 16384-token sequence,
    chunk-causal (chunk 2 after a 1024-token causal prefix, one CHUNK_CAUSAL
    range), 16 heads, d 128; the library's forward (fp32 output) feeds it.
    The oracle computes exact gradients for two heads at sampled query rows
    and keys (tile and range boundaries, the ends, random picks)."""
    from oracle import masks as OM
    from oracle import attention as OA
    w = W.config4(chunk_sizes=(2,))
    dev = device_inputs(w)
    do = W.upstream_grad(w, 4001)
    dev["do"] = torch.from_numpy(do).cuda().to(torch.bfloat16).contiguous()
    name = "chunk2"
    _say("backward full size", name)
    out, lse, plan = run_prefill(w, dev, name, out_dtype=torch.float32)
    dq, dk, dv = ma.attn_backward_masked(plan, dev["q"], dev["k"], dev["v"], dev["pt"], out, lse, dev["do"], w.scale)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()
    n = int(w.kv_lens[0])
    rng = np.random.default_rng(44)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 1023, 1024, 1025, 8191, n - 2, n - 1],
                                     rng.integers(0, n, 22)]))
    keys = np.unique(np.concatenate([[0, 63, 64, 1023, 1024, 1025, 8192, n - 64, n - 1], rng.integers(0, n, 23)]))
    mask = OM.ranges(n, n, w.masks[name].ranges[0])
    page = w.page_size
    slots = (w.page_table[0, keys // page], keys % page)
    for h in (0, 9):
        _say("oracle head", h)
        k = OA.gather_paged(w.k_cache, w.page_table[0], n, h)
        v = OA.gather_paged(w.v_cache, w.page_table[0], n, h)
        rq, rk, rv = OB.attend_backward_sampled(w.q[:, h], k, v, mask, w.scale, do[:, h], rows, keys)
        gq = dq[rows, h]
        errq = float(np.abs(gq - rq).max() / np.sqrt((rq ** 2).mean()))
        _say("dq max err / rms", errq)
        assert errq <= 2.0 ** -3, (h, errq)
        for g, r, what in ((dk[slots[0], slots[1], h], rk, "dk"), (dv[slots[0], slots[1], h], rv, "dv")):
            err = grad_err(torch.from_numpy(g), r)
            _say(what, "row metric", err)
            assert err <= TOL_GRAD, (h, what, err)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_backward_page_sizes_bit_identical(d):
    """Pages of 1 and 4 keys take the per-lane gather of the dQ pass, 16 the
    per-instruction scalar base, 64 one base per wave; the page layout does not
    enter the arithmetic, so dQ and every key's dK / dV are bit-identical."""
    base, do, _ = _setup(d)
    name = "ranges"
    out, lse = _fwd_oracle(base, name)
    res = {}
    for ps in (1, 4, 16, 64):
        w = base if ps == base.page_size else repage(base, ps, 900 + ps)
        _say("backward page size", d, ps)
        dev = device_inputs(w)
        dev["do"] = torch.from_numpy(do).cuda().to(torch.bfloat16).contiguous()
        dq, dk, dv = _bwd(w, dev, name, out, lse)
        keys = []
        dkc, dvc = dk.cpu().numpy(), dv.cpu().numpy()
        for b, kl in enumerate(w.kv_lens):
            j = np.arange(int(kl))
            pg, sl = w.page_table[b, j // ps], j % ps
            keys.append((dkc[pg, sl], dvc[pg, sl]))
        res[ps] = (dq.cpu().numpy(), keys)
    rq, rk, rv = _ref(base, do, name)
    assert grad_err(torch.from_numpy(res[16][0]), rq) <= TOL_GRAD
    for ps in (1, 4, 64):
        assert np.array_equal(res[ps][0], res[16][0]), ("dq", ps)
        for b in range(len(base.kv_lens)):
            assert np.array_equal(res[ps][1][b][0], res[16][1][b][0]), ("dk", ps, b)
            assert np.array_equal(res[ps][1][b][1], res[16][1][b][1]), ("dv", ps, b)


def test_backward_gemma2_global_sampled():
    """The backward of the Gemma2-like global layer (16384 tokens, causal,
    8 query heads over 4 K/V heads, d 256, random page order) at full size;
    the library's forward (fp32 output) feeds it; the oracle takes exact
    gradients for two heads at sampled query rows and keys."""
    from oracle import masks as OM
    from oracle import attention as OA
    w = W.config3b(1)
    dev = device_inputs(w)
    do = W.upstream_grad(w, 4003)
    dev["do"] = torch.from_numpy(do).cuda().to(torch.bfloat16).contiguous()
    _say("backward d 256 global layer")
    out, lse, plan = run_prefill(w, dev, "causal", out_dtype=torch.float32)
    dq, dk, dv = ma.attn_backward_masked(plan, dev["q"], dev["k"], dev["v"], dev["pt"], out, lse, dev["do"], w.scale)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()
    n = int(w.kv_lens[0])
    rng = np.random.default_rng(46)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 4095, 4096, 8191, n - 2, n - 1], rng.integers(0, n, 15)]))
    keys = np.unique(np.concatenate([[0, 63, 64, 4095, 4096, 8192, n - 64, n - 1], rng.integers(0, n, 16)]))
    mask = OM.causal(n, n)
    page = w.page_size
    slots = (w.page_table[0, keys // page], keys % page)
    # K/V head 0 serves query heads 0 and 1: their dQ rows, and dK / dV summed
    k = OA.gather_paged(w.k_cache, w.page_table[0], n, 0)
    v = OA.gather_paged(w.v_cache, w.page_table[0], n, 0)
    rk = rv = 0
    for h in (0, 1):
        _say("oracle head", h)
        rq, rk_h, rv_h = OB.attend_backward_sampled(w.q[:, h], k, v, mask, w.scale, do[:, h], rows, keys)
        rk = rk + rk_h
        rv = rv + rv_h
        errq = float(np.abs(dq[rows, h] - rq).max() / np.sqrt((rq ** 2).mean()))
        _say("dq max err / rms", errq)
        assert errq <= 2.0 ** -3, (h, errq)
    for gr, r, what in ((dk[slots[0], slots[1], 0], rk, "dk"), (dv[slots[0], slots[1], 0], rv, "dv")):
        err = grad_err(torch.from_numpy(gr), r)
        _say(what, "row metric", err)
        assert err <= TOL_GRAD, (what, err)
