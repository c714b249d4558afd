"""GPU parity of masked prefill (HIP path through the C ABI) against the fp64
oracle on the same seeded inputs."""

import numpy as np
import pytest
import torch

import masked_flash_attention_mask_amd as ma
import workloads as W
from helpers import (TOL_BF16, TOL_F32, bf16_out_err, device_inputs, lse_err, max_abs_err, oracle, parity_report,
                     repage,
                     run_prefill)

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


# ------------------------------------------------------------------ config 1 --
@pytest.mark.parametrize("mask", ["causal", "custom", "custom_packed"])
@pytest.mark.parametrize("tile_q", [128, 64])
def test_config1_fp32(mask, tile_q):
    w = W.config1()
    _say("cfg1", mask, tile_q)
    d = device_inputs(w)
    out, lse, _ = run_prefill(w, d, mask, tile_q=tile_q)
    ref_o, ref_l = oracle(w, mask)
    parity_report(f"cfg1 {mask} tile_q {tile_q}", max_abs_err=max_abs_err(out, ref_o), lse_err=lse_err(lse, ref_l))
    assert max_abs_err(out, ref_o) <= TOL_F32
    assert lse_err(lse, ref_l) <= TOL_F32


def test_config1_host_and_device_classify_agree():
    w = W.config1()
    d = device_inputs(w)
    o1, _, p1 = run_prefill(w, d, "custom", device_mask=True)
    o2, _, p2 = run_prefill(w, d, "custom", device_mask=False)
    assert torch.equal(o1, o2)
    c1, w1 = p1.export()
    c2, w2 = p2.export()
    assert np.array_equal(c1, c2) and np.array_equal(w1, w2)


@pytest.mark.parametrize("tile_q", [64, 128])
def test_device_classify_matches_host_compile(tile_q):
    """Device-classified dense and packed masks give the host compiler's
    classes and words bit for bit: ragged rows (q_len not a multiple of the
    tile), contexts spanning several 64-tile chunks with a ragged tail, FULL,
    SKIP and PARTIAL tiles, empty and one-key rows."""
    rng = np.random.default_rng(900 + tile_q)
    q_lens, kv_lens = [300, 5, 130], [4500, 70, 8300]
    dense = []
    for q, k in zip(q_lens, kv_lens):
        m = rng.random((q, k)) < 0.2
        m[:, : min(k, 256)] = True          # FULL tiles
        m[:, k // 2: k // 2 + 700] = False   # SKIP tiles
        m[q // 2, :] = False                 # an empty row
        m[q - 1, :] = False
        m[q - 1, k - 1] = True               # a one-key row in the tail tile
        dense.append(m)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    kv = np.asarray(kv_lens, np.int32)
    flat = np.concatenate([m.astype(np.uint8).reshape(-1) for m in dense])
    packed = np.concatenate([W.pack_rows(m).reshape(-1) for m in dense])
    host = ma.mask_compile_host("dense", cu, kv, mask=flat, tile_q=tile_q)
    hc, hw = host.export()
    for kind, data in (("dense", flat), ("packed", packed.view(np.int64))):
        _say("device classify", kind, tile_q)
        p = ma.mask_compile(kind, cu, kv, mask=torch.from_numpy(np.ascontiguousarray(data)).cuda(), tile_q=tile_q)
        dc, dw = p.export()
        assert np.array_equal(dc, hc), kind
        assert np.array_equal(dw, hw), kind


@pytest.mark.parametrize("tile_q", [64, 128])
@pytest.mark.parametrize("shape", [([3, 2], [4, 1]),                  # the whole mask under 16 bytes
                                   ([5, 17, 40], [15, 33, 16]),        # rows shorter than a tile
                                   ([1, 70], [1030, 2049])])           # rows ending 6 and 1 bytes into a load
def test_device_classify_short_masks(tile_q, shape):
    """Dense rows shorter than a 16-byte load, a mask shorter than one load,
    and rows whose last bytes start a new 1 KB load: the device classes and
    words equal the host compiler's."""
    q_lens, kv_lens = shape
    rng = np.random.default_rng(950 + tile_q + len(q_lens))
    dense = [rng.random((q, k)) < 0.5 for q, k in zip(q_lens, kv_lens)]
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    kv = np.asarray(kv_lens, np.int32)
    flat = np.concatenate([m.astype(np.uint8).reshape(-1) for m in dense])
    host = ma.mask_compile_host("dense", cu, kv, mask=flat, tile_q=tile_q)
    hc, hw = host.export()
    _say("device classify short", shape, tile_q, flat.size)
    p = ma.mask_compile("dense", cu, kv, mask=torch.from_numpy(flat).cuda(), tile_q=tile_q)
    dc, dw = p.export()
    assert np.array_equal(dc, hc) and np.array_equal(dw, hw)


# ------------------------------------------- small ragged bf16 shapes, all d --
def _ragged(seed, d, hq, hkv, q_lens, kv_lens, permute=True):
    rng = W.rng_for(seed)
    return W.gen._build(f"ragged{seed}", rng, "bf16", q_lens, kv_lens, hq, hkv, d, permute=permute)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("tile_q", [128, 64])
def test_bf16_ragged_kinds(d, tile_q):
    q_lens, kv_lens = [200, 1, 64, 130], [200, 70, 300, 130]
    w = _ragged(100 + d, d, 4, 2, q_lens, kv_lens)
    w.masks["causal"] = W.MaskInput("causal")
    w.masks["window"] = W.MaskInput("window", window=37)
    w.masks["prefix"] = W.MaskInput("prefix_lm", prefix_len=np.array([50, 0, 300, 130], np.int32))
    w.masks["ranges"] = W.MaskInput("ranges", ranges=[
        [(0, 200, 0, 100, W.R_FULL, 0), (100, 200, 100, 200, W.R_CHUNK_CAUSAL, 3)],
        [],
        [(0, 64, 0, 300, W.R_CAUSAL, 0), (10, 20, 5, 250, W.R_INV_CAUSAL, 0)],
        [(0, 130, 0, 130, W.R_BI_CAUSAL, 0), (60, 130, 0, 64, W.R_FULL, 0)],
    ])
    dev = device_inputs(w)
    for mask in ("causal", "window", "prefix", "ranges"):
        _say("ragged", d, tile_q, mask)
        out, lse, _ = run_prefill(w, dev, mask, tile_q=tile_q)
        ref_o, ref_l = oracle(w, mask)
        err = max_abs_err(out, ref_o)
        assert err <= TOL_BF16, (mask, err)
        assert lse_err(lse, ref_l) <= 1e-2
    # empty rows of sequence 1 under the range mask: O = 0, LSE = -inf
    out, lse, _ = run_prefill(w, dev, "ranges", tile_q=tile_q)
    assert torch.all(out[200] == 0) and torch.all(torch.isneginf(lse[200]))


@pytest.mark.parametrize("tile_q", [128, 64])
def test_degenerate_masks(tile_q):
    """Cases that reduce to something exact: a window of 1 key leaves each
    row its own key, P = 1 and O = that key's V row bit for bit; an all-true
    custom mask and a prefix covering every key are full attention (the
    FULL range's plan, so identical outputs); an all-false custom mask
    empties every row (O = 0, LSE = -inf); a window at least as long as the
    keys is causal; causal with more queries than keys leaves the first
    q_len - kv_len rows empty (bottom-right alignment)."""
    q_lens, kv_lens = [100, 130, 70], [40, 130, 200]
    w = _ragged(600 + tile_q, 128, 4, 2, q_lens, kv_lens)
    w.masks["causal"] = W.MaskInput("causal")
    w.masks["w1"] = W.MaskInput("window", window=1)
    w.masks["w_long"] = W.MaskInput("window", window=256)
    w.masks["full"] = W.MaskInput("ranges", ranges=[[(0, q, 0, k, W.R_FULL, 0)] for q, k in zip(q_lens, kv_lens)])
    w.masks["prefix_all"] = W.MaskInput("prefix_lm", prefix_len=np.array(kv_lens, np.int32))
    n = sum(q * k for q, k in zip(q_lens, kv_lens))
    w.masks["ones"] = W.MaskInput("dense", data=np.ones(n, np.uint8))
    w.masks["zeros"] = W.MaskInput("dense", data=np.zeros(n, np.uint8))
    dev = device_inputs(w)
    res = {}
    for mask in ("causal", "w1", "w_long", "full", "prefix_all", "ones", "zeros"):
        _say("degenerate", tile_q, mask)
        res[mask] = run_prefill(w, dev, mask, tile_q=tile_q)[:2]
    for mask in ("causal", "w1", "full"):
        ref_o, ref_l = oracle(w, mask)
        assert max_abs_err(res[mask][0], ref_o) <= TOL_BF16, mask
        assert lse_err(res[mask][1], ref_l) <= 1e-2, mask
    for a, b in (("ones", "full"), ("prefix_all", "full"), ("w_long", "causal")):
        assert torch.equal(res[a][0], res[b][0]) and torch.equal(res[a][1], res[b][1]), (a, b)
    o0, l0 = res["zeros"]
    assert torch.all(o0 == 0) and torch.all(torch.isneginf(l0))
    # window 1: row t of a sequence sees key t + kv_len - q_len only
    o1 = res["w1"][0].cpu().numpy()
    t0 = 0
    for b, (q, k) in enumerate(zip(q_lens, kv_lens)):
        for t in range(q):
            key = t + k - q
            if key < 0:
                assert np.all(o1[t0 + t] == 0)
                continue
            page, slot = w.page_table[b, key // w.page_size], key % w.page_size
            v = w.v_cache[page, slot].astype(np.float32)            # [Hkv, d], bf16 values
            want = np.repeat(v, w.hq // w.hkv, axis=0)
            assert np.array_equal(o1[t0 + t], want), (b, t)
        t0 += q
    # causal with 100 queries over 40 keys: rows 0..59 see nothing
    oc, lc = res["causal"]
    assert torch.all(oc[:60] == 0) and torch.all(torch.isneginf(lc[:60]))
    assert torch.all(torch.isfinite(lc[60:100]))

@pytest.mark.parametrize("d", [64, 128, 256])
def test_empty_sequences_and_keyless_rows(d):
    """Sequences without queries, one whose 50 queries have no keys (their
    rows come out O = 0, LSE = -inf), under every host-described kind and a
    device-resident custom mask; then a batch without any query row, which
    launches nothing and accepts the empty tensors' NULL pointers."""
    q_lens, kv_lens = [0, 50, 0, 3, 40], [10, 0, 0, 70, 130]
    w = _ragged(400 + d, d, 4, 2, q_lens, kv_lens)
    w.masks["causal"] = W.MaskInput("causal")
    w.masks["window"] = W.MaskInput("window", window=9)
    w.masks["prefix"] = W.MaskInput("prefix_lm", prefix_len=np.array([4, 0, 0, 5, 64], np.int32))
    w.masks["ranges"] = W.MaskInput("ranges", ranges=[[], [], [], [(0, 3, 0, 70, W.R_FULL, 0)],
                                                       [(0, 40, 0, 130, W.R_CAUSAL, 0)]])
    rng = np.random.default_rng(d)
    dense = [rng.random((q, k)) < 0.5 for q, k in zip(q_lens, kv_lens)]
    w.masks["custom"] = W.MaskInput("dense", data=np.concatenate([m.astype(np.uint8).reshape(-1) for m in dense]))
    dev = device_inputs(w)
    for mask in ("causal", "window", "prefix", "ranges", "custom"):
        _say("empty sequences", d, mask)
        out, lse, _ = run_prefill(w, dev, mask)
        ref_o, ref_l = oracle(w, mask)
        assert max_abs_err(out, ref_o) <= TOL_BF16, mask
        assert lse_err(lse, ref_l) <= 1e-2, mask
        assert torch.all(out[:50] == 0) and torch.all(torch.isneginf(lse[:50])), mask
    e = _ragged(500 + d, d, 4, 2, [0, 0], [5, 0])
    e.masks["causal"] = W.MaskInput("causal")
    out, lse, _ = run_prefill(e, device_inputs(e), "causal")
    assert out.shape == (0, 4, d) and lse.shape == (0, 4)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_bf16_page_sizes_and_gather_modes(d):
    """Pages of 512 / d keys or more take the direct-to-LDS gather (one page
    id per instruction, or per wave once pages hold a wave's whole run of
    keys), smaller ones the register-staged gather; both tile heights.  Page
    layout does not enter the arithmetic, so every page size gives
    bit-identical outputs."""
    base = _ragged(500 + d, d, 4, 2, [150, 77], [230, 77])
    base.masks["prefix"] = W.MaskInput("prefix_lm", prefix_len=np.array([100, 7], np.int32))
    ref_o, ref_l = oracle(base, "prefix")
    for tq in (128, 64):
        outs = {}
        for ps in (1, 2, 4, 8, 16, 64):
            w = repage(base, ps, 600 + ps)
            _say("page size", d, tq, ps)
            outs[ps] = run_prefill(w, device_inputs(w), "prefix", tile_q=tq)[:2]
        assert max_abs_err(outs[1][0], ref_o) <= TOL_BF16
        assert lse_err(outs[1][1], ref_l) <= 1e-2
        for ps in (2, 4, 8, 16, 64):
            assert torch.equal(outs[ps][0], outs[1][0]) and torch.equal(outs[ps][1], outs[1][1]), (tq, ps)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_bf16_output_dtype(d):
    w = _ragged(200 + d, d, 2, 2, [150], [150])
    w.masks["causal"] = W.MaskInput("causal")
    dev = device_inputs(w)
    out, _, _ = run_prefill(w, dev, "causal", out_dtype=torch.bfloat16)
    assert out.dtype == torch.bfloat16
    ref_o, _ = oracle(w, "causal")
    assert bf16_out_err(out, ref_o) <= TOL_BF16


def _contiguous_copy(w):
    """The same workload with its K/V re-laid out in consecutive pages."""
    import copy
    c = copy.copy(w)
    pages = [(int(k) + 15) // 16 for k in w.kv_lens]
    total = sum(pages) + 2
    c.k_cache = np.full((total,) + w.k_cache.shape[1:], np.nan, np.float32)
    c.v_cache = np.full_like(c.k_cache, np.nan)
    c.page_table = np.full_like(w.page_table, total - 1)
    off = 0
    for b, kl in enumerate(w.kv_lens):
        j = np.arange(int(kl))
        src_p, src_s = w.page_table[b, j // 16], j % 16
        c.k_cache[off + j // 16, j % 16] = w.k_cache[src_p, src_s]
        c.v_cache[off + j // 16, j % 16] = w.v_cache[src_p, src_s]
        c.page_table[b, :pages[b]] = off + np.arange(pages[b])
        off += pages[b]
    return c


def test_page_permutation_invariance_and_determinism():
    a = _ragged(7, 128, 4, 1, [130, 70], [190, 70], permute=True)
    a.masks["causal"] = W.MaskInput("causal")
    b = _contiguous_copy(a)
    assert not np.array_equal(a.page_table, b.page_table)
    da, db = device_inputs(a), device_inputs(b)
    oa, la, _ = run_prefill(a, da, "causal")
    ob, lb, _ = run_prefill(b, db, "causal")
    assert torch.equal(oa, ob) and torch.equal(la, lb)
    oa2, la2, _ = run_prefill(a, da, "causal")
    assert torch.equal(oa, oa2) and torch.equal(la, la2)


def test_gqa_equals_repeated_mha():
    w = _ragged(9, 64, 8, 2, [100], [160])
    w.masks["causal"] = W.MaskInput("causal")
    m = _ragged(9, 64, 8, 2, [100], [160])
    m.k_cache = np.repeat(w.k_cache, 4, axis=2)
    m.v_cache = np.repeat(w.v_cache, 4, axis=2)
    m.hkv = 8
    m.masks["causal"] = W.MaskInput("causal")
    o1, _, _ = run_prefill(w, device_inputs(w), "causal")
    o2, _, _ = run_prefill(m, device_inputs(m), "causal")
    assert torch.equal(o1, o2)


def test_mask_probe_q_zero_v_identity():
    """Q = 0 makes every score 0; with V = I the output row is the row's mask
    divided by its popcount (the mask read back through the kernel)."""
    n, d = 96, 128
    w = _ragged(10, d, 1, 1, [n], [n], permute=False)
    w.q[:] = 0.0
    eye = np.zeros((n, 1, d), np.float32)
    eye[np.arange(n), 0, np.arange(n)] = 1.0
    for b in range(w.v_cache.shape[0] - 2):
        w.v_cache[b, :, :, :] = eye[b * 16:(b + 1) * 16]
    w.masks["probe"] = W.MaskInput("ranges", ranges=[[(0, 96, 0, 40, W.R_CHUNK_CAUSAL, 5),
                                                      (20, 96, 30, 96, W.R_CAUSAL, 0)]])
    out, _, _ = run_prefill(w, device_inputs(w), "probe")
    from oracle import masks as OM
    mk = OM.ranges(n, n, w.masks["probe"].ranges[0]).astype(np.float64)
    cnt = mk.sum(1, keepdims=True)
    want = np.where(cnt > 0, mk / np.maximum(cnt, 1), 0.0)
    got = out[:, 0, :n].double().cpu().numpy()
    assert np.abs(got - want).max() <= 1e-6     # every p is exp2(0) = 1 exactly


# ---------------------------------------------- reduced config 4 and config 5 --
def test_config4_reduced_forms_bit_identical():
    w = W.config4(seq=2048, prefix=128, hq=2)
    for cs in (2, 4, 16):
        w.masks[f"chunk{cs}"] = W.MaskInput("ranges", ranges=[W.chunk_ranges(2048, 128, cs)])
        w.masks[f"chunk{cs}_full"] = W.MaskInput("ranges", ranges=[W.chunk_ranges_expanded(2048, 128, cs)])
    dev = device_inputs(w)
    for cs in (2, 4, 16):
        _say("cfg4 reduced", cs)
        o1, l1, _ = run_prefill(w, dev, f"chunk{cs}")
        o2, l2, _ = run_prefill(w, dev, f"chunk{cs}_full")
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        ref_o, ref_l = oracle(w, f"chunk{cs}")
        assert max_abs_err(o1, ref_o) <= TOL_BF16


def test_config5_reduced_range_vs_packed():
    w = W.config5(q_len=3000, kv_len=2700, dense_keys=2048, blocks=5, block=100, hq=4, hkv=2)
    dev = device_inputs(w)
    o1, l1, _ = run_prefill(w, dev, "custom_ranges")
    o2, l2, _ = run_prefill(w, dev, "custom_packed")
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    ref_o, ref_l = oracle(w, "custom_ranges")
    assert max_abs_err(o1, ref_o) <= TOL_BF16
    assert lse_err(l1, ref_l) <= 1e-2


# ------------------------------------------------ full-size configs, sampled --
def _sample_rows(q_len, rng, n=48):
    rows = set(rng.choice(q_len, size=n, replace=False).tolist())
    rows |= {0, 1, q_len - 1, q_len // 2}
    return np.array(sorted(rows))


def test_config4_full_size_sampled():
    w = W.config4()
    dev = device_inputs(w)
    rng = np.random.default_rng(44)
    rows = {0: _sample_rows(16384, rng)}
    outs = {}
    for name in ("chunk2", "chunk2_full", "chunk16", "chunk16_full", "causal"):
        _say("cfg4 full", name)
        o, l, _ = run_prefill(w, dev, name)
        outs[name] = (o, l)
    for cs in (2, 16):
        assert torch.equal(outs[f"chunk{cs}"][0], outs[f"chunk{cs}_full"][0])
        ref_o, ref_l = oracle(w, f"chunk{cs}", heads=[0, 7, 15], rows=rows)
        parity_report(f"cfg4 chunk{cs} sampled", max_abs_err=max_abs_err(outs[f"chunk{cs}"][0], ref_o),
                      lse_err=lse_err(outs[f"chunk{cs}"][1], ref_l))
        assert max_abs_err(outs[f"chunk{cs}"][0], ref_o) <= TOL_BF16
        assert lse_err(outs[f"chunk{cs}"][1], ref_l) <= 1e-2


def test_config5_full_size_sampled():
    w = W.config5()
    dev = device_inputs(w)
    rng = np.random.default_rng(55)
    rows = _sample_rows(32768, rng, 32)
    rows = np.unique(np.concatenate([rows, [27767, 27768, 27867, 27868, 32767]]))
    o1, l1, _ = run_prefill(w, dev, "custom_ranges")
    o2, l2, _ = run_prefill(w, dev, "custom_packed")
    assert torch.equal(o1, o2)
    ref_o, ref_l = oracle(w, "custom_ranges", heads=[0, 13, 31], rows={0: rows})
    parity_report("cfg5 ranges = packed, sampled", max_abs_err=max_abs_err(o1, ref_o), lse_err=lse_err(l1, ref_l))
    assert max_abs_err(o1, ref_o) <= TOL_BF16
    assert lse_err(l1, ref_l) <= 1e-2


def test_config3a_full_size_sampled():
    w = W.config3a()
    dev = device_inputs(w)
    rng = np.random.default_rng(31)
    rows = {b: _sample_rows(4096, rng, 24) for b in range(4)}
    o1, l1, _ = run_prefill(w, dev, "prefix_lm")
    o2, _, _ = run_prefill(w, dev, "prefix_lm_ranges")
    assert torch.equal(o1, o2)
    ref_o, ref_l = oracle(w, "prefix_lm", heads=[0, 31], rows=rows)
    parity_report("cfg3a prefix_lm = ranges, sampled", max_abs_err=max_abs_err(o1, ref_o), lse_err=lse_err(l1, ref_l))
    assert max_abs_err(o1, ref_o) <= TOL_BF16
    assert lse_err(l1, ref_l) <= 1e-2


@pytest.mark.parametrize("hkv", [1, 2, 4, 8])
def test_bf16_head_group_map(hkv):
    """8 query heads over 1, 2, 4 or 8 K/V heads: with fewer query heads per
    XCD than a GQA group, the workgroups of one K/V head's query heads are
    spread over that head's XCDs by work item, the grid padded to a multiple
    of them (seven q-tiles here, so padding workgroups exist); every (q-tile,
    head) must still be computed exactly once."""
    q_lens, kv_lens = [300, 1, 129, 40], [300, 90, 129, 500]
    w = _ragged(120 + hkv, 128, 8, hkv, q_lens, kv_lens)
    w.masks["causal"] = W.MaskInput("causal")
    w.masks["window"] = W.MaskInput("window", window=70)
    dev = device_inputs(w)
    for mask in ("causal", "window"):
        _say("head group map", hkv, mask)
        out, lse, _ = run_prefill(w, dev, mask, tile_q=128)
        ref_o, ref_l = oracle(w, mask)
        assert max_abs_err(out, ref_o) <= TOL_BF16, mask
        assert lse_err(lse, ref_l) <= 1e-2, mask


def test_config3b_full_size_sampled_and_not_vacuous():
    rng = np.random.default_rng(32)
    rows = {0: _sample_rows(16384, rng, 24)}
    w0 = W.config3b(0)
    dev = device_inputs(w0)
    local, _, _ = run_prefill(w0, dev, "window")
    glob, _, _ = run_prefill(w0, dev, "causal")
    ref_o, _ = oracle(w0, "window", heads=[0, 5], rows=rows)
    parity_report("cfg3b window 4096, sampled", max_abs_err=max_abs_err(local, ref_o))
    assert max_abs_err(local, ref_o) <= TOL_BF16
    # the window bites: local and global outputs differ far beyond tolerance
    assert (local - glob).abs().max().item() > 0.1
    # an inert window (>= sequence length) reproduces the global output
    w0.masks["inert"] = W.MaskInput("window", window=16384)
    inert, _, _ = run_prefill(w0, dev, "inert")
    assert torch.equal(inert, glob)
    w1 = W.config3b(1)
    g1, _, _ = run_prefill(w1, device_inputs(w1), "causal")
    ref1, _ = oracle(w1, "causal", heads=[3], rows=rows)
    parity_report("cfg3b causal, sampled", max_abs_err=max_abs_err(g1, ref1))
    assert max_abs_err(g1, ref1) <= TOL_BF16


def test_device_classify_full_size_block_mask():
    """The 32768 x 29576 block mask with 50 triangles, classified on the GPU
    from its packed and dense forms (every k-tile chunk of every q-tile row at
    once), gives the host compiler's classes and words bit for bit."""
    w = W.config5()
    q, k = int(w.q_lens[0]), int(w.kv_lens[0])
    words = w.masks["custom_packed"].data
    host = ma.mask_compile_host("packed", w.cu_seqlens_q, w.kv_lens, mask=words)
    hc, hw = host.export()
    dense = np.unpackbits(words.view(np.uint8).reshape(q, -1), axis=1, bitorder="little")[:, :k]
    for kind, data in (("packed", words.view(np.int64)), ("dense", np.ascontiguousarray(dense).reshape(-1))):
        _say("full-size device classify", kind)
        p = ma.mask_compile(kind, w.cu_seqlens_q, w.kv_lens, mask=torch.from_numpy(np.ascontiguousarray(data)).cuda())
        dc, dw = p.export()
        assert np.array_equal(dc, hc), kind
        assert np.array_equal(dw, hw), kind
        del p
