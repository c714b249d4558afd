"""The seeded input generators against the oracle's own mask definitions
(CPU only, reduced sizes)."""

import numpy as np

import workloads as W
from oracle import masks as M


def test_config1_masks():
    w = W.config1()
    bits = w.info["bits"]
    assert bits.diagonal().all() and 0.45 < bits.mean() < 0.56
    (dense,) = M.dense_from_flat(w.masks["custom"].data, [128], [128])
    (packed,) = M.packed_from_flat(w.masks["custom_packed"].data, [128], [128])
    assert np.array_equal(dense, bits) and np.array_equal(packed, bits)
    assert w.q.dtype == np.float32 and w.scale == 1 / 8


def test_config2_tree_masks_match_oracle():
    w = W.config2(batch=3, ctx_lo=40, ctx_hi=130)
    ql, kl = w.q_lens, w.kv_lens
    dense = M.dense_from_flat(w.masks["tree_dense"].data, ql, kl)
    packed = M.packed_from_flat(w.masks["tree_packed"].data, ql, kl)
    for b in range(3):
        want = M.tree(int(w.info["ctx"][b]), w.info["parents"][b])
        assert np.array_equal(dense[b], want) and np.array_equal(packed[b], want)


def test_config2_full_size_structure():
    w = W.config2()
    assert w.batch == 8 and (w.q_lens == 64).all()
    assert ((w.info["ctx"] >= 512) & (w.info["ctx"] <= 4096)).all()
    for p in w.info["parents"]:
        assert p[0] == 0 and all(0 <= p[i] < i for i in range(1, 64))


def test_paged_layout_round_trip():
    w = W.config3a(batch=2, seq=100, hq=2, d=8)
    # keys of sequence 1 read back through the page table are finite; slots
    # past kv_len and spare pages are NaN
    for b in range(2):
        kl = int(w.kv_lens[b])
        j = np.arange(kl)
        k = w.k_cache[w.page_table[b, j // 16], j % 16]
        assert np.isfinite(k).all()
        last = w.page_table[b, (kl - 1) // 16]
        assert np.isnan(w.k_cache[last, kl % 16:]).all() if kl % 16 else True
    all_nan = np.isnan(w.k_cache).reshape(w.k_cache.shape[0], -1).all(axis=1)
    assert all_nan.sum() == 2                    # the two spare pages
    used = set(w.page_table.reshape(-1).tolist())
    assert len(used) == 14 and not all_nan[list(used)].any()
    # bf16 values are exactly representable
    assert np.array_equal(W.round_bf16(w.q), w.q)


def test_config3a_forms_equal():
    w = W.config3a(batch=2, seq=300, p_lo=20, p_hi=120, hq=1, d=8)
    for b in range(2):
        p = int(w.info["prefix_len"][b])
        a = M.prefix_lm(300, 300, p)
        r = M.ranges(300, 300, w.masks["prefix_lm_ranges"].ranges[b])
        assert np.array_equal(a, r)


def test_config4_forms_equal():
    for cs in (2, 4, 16, 7):
        a = M.ranges(600, 600, W.chunk_ranges(600, 64, cs))
        b = M.ranges(600, 600, W.chunk_ranges_expanded(600, 64, cs))
        assert np.array_equal(a, b)
    assert len(W.chunk_ranges_expanded(16384, 1024, 2)) == 1 + 7680
    assert len(W.chunk_ranges_expanded(16384, 1024, 16)) == 1 + 960


def test_config5_forms_equal_reduced():
    q, kv, dk, nb, bl = 700, 520, 320, 5, 40
    rg = W.block_triangle_ranges(q, kv, dk, nb, bl)
    pk = W.block_triangle_packed(q, kv, dk, nb, bl)
    assert np.array_equal(M.ranges(q, kv, rg), M.unpack_rows(pk, q, kv))
    # word-aligned dense block, as at full size
    rg = W.block_triangle_ranges(300, 384, 256, 2, 50)
    pk = W.block_triangle_packed(300, 384, 256, 2, 50)
    assert np.array_equal(M.ranges(300, 384, rg), M.unpack_rows(pk, 300, 384))


def test_config5_full_size_sampled_rows():
    w5 = W.block_triangle_packed(32768, 29576, 24576, 50, 100)
    rg = W.block_triangle_ranges(32768, 29576, 24576, 50, 100)
    rows = np.array([0, 27767, 27768, 27769, 27867, 27868, 32767])
    dense = M.unpack_rows(w5[rows].reshape(-1), len(rows), 29576)
    for i, t in enumerate(rows):
        want = np.zeros(29576, bool)
        for qs, qe, ks, ke, ty, cs in rg:
            if qs <= t < qe:
                blk = M.range_block(qe - qs, ke - ks, ty, cs)
                want[ks:ke] |= blk[t - qs]
        assert np.array_equal(dense[i], want)
    total = 27768 * 24576 + 5000 * 24576 + 50 * (100 * 101 // 2)
    assert total == 805558868
