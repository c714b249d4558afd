"""Host mask compiler (C ABI, no GPU) against the oracle's tile classification:
bit-exact classes and words, byte-identical plans for equivalent masks."""

import numpy as np
import pytest

import masked_flash_attention_mask_amd as ma
import masked_flash_attention_mask_amd._lib as L
import workloads as W
from oracle import masks as M
from oracle import tiles as T


def _oracle_export(dense_masks, tile_q):
    cls, words = [], []
    for m in dense_masks:
        c, w = T.classify(m, tile_q, 64)
        cls.append(c.reshape(-1))
        words.append(w.reshape(-1, tile_q))
    return np.concatenate(cls), np.concatenate(words)


def _check(plan, dense_masks, tile_q):
    c1, w1 = plan.export()
    c2, w2 = _oracle_export(dense_masks, tile_q)
    assert np.array_equal(c1, c2)
    assert np.array_equal(w1, w2)


def _cu(q_lens):
    return np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)


@pytest.mark.parametrize("tile_q", [64, 128])
def test_closed_form_kinds(tile_q):
    q_lens, kv_lens = [300, 1, 129, 64], [300, 77, 400, 64]
    cu = _cu(q_lens)
    cases = [
        ("causal", {}, [M.causal(q, k) for q, k in zip(q_lens, kv_lens)]),
        ("window", {"window": 70}, [M.sliding_window(q, k, 70) for q, k in zip(q_lens, kv_lens)]),
        ("window", {"window": 1}, [M.sliding_window(q, k, 1) for q, k in zip(q_lens, kv_lens)]),
        ("prefix_lm", {"prefix_len": [100, 0, 400, 5]},
         [M.prefix_lm(q, k, p) for q, k, p in zip(q_lens, kv_lens, [100, 0, 400, 5])]),
    ]
    for kind, kw, dense in cases:
        plan = ma.mask_compile_host(kind, cu, kv_lens, tile_q=tile_q, **kw)
        _check(plan, dense, tile_q)


def test_range_types_random():
    rng = np.random.default_rng(11)
    for trial in range(25):
        q_lens = rng.integers(1, 300, size=2)
        kv_lens = q_lens + rng.integers(0, 200, size=2)
        ranges = []
        for ql, kl in zip(q_lens, kv_lens):
            seq = []
            for _ in range(int(rng.integers(0, 6))):
                qs = int(rng.integers(0, ql)); qe = int(rng.integers(qs, ql + 1))
                ks = int(rng.integers(0, kl)); ke = int(rng.integers(ks, kl + 1))
                ty = int(rng.integers(0, 5)); cs = int(rng.integers(1, 9))
                seq.append((qs, qe, ks, ke, ty, cs))
            ranges.append(seq)
        tq = 64 if trial % 2 else 128
        plan = ma.mask_compile_host("ranges", _cu(q_lens), kv_lens, ranges=ranges, tile_q=tq)
        dense = [M.ranges(int(q), int(k), r) for q, k, r in zip(q_lens, kv_lens, ranges)]
        _check(plan, dense, tq)


def test_dense_and_packed_host():
    rng = np.random.default_rng(12)
    q_lens, kv_lens = [70, 130], [70, 200]
    dense = [rng.random((q, k)) < 0.3 for q, k in zip(q_lens, kv_lens)]
    dense[0][:, :64] = True         # a FULL tile
    dense[1][:64, 64:128] = False   # a SKIP tile
    flat = np.concatenate([d.astype(np.uint8).reshape(-1) for d in dense])
    packed = np.concatenate([W.pack_rows(d).reshape(-1) for d in dense])
    for tq in (64, 128):
        pd = ma.mask_compile_host("dense", _cu(q_lens), kv_lens, mask=flat, tile_q=tq)
        pp = ma.mask_compile_host("packed", _cu(q_lens), kv_lens, mask=packed, tile_q=tq)
        _check(pd, dense, tq)
        _check(pp, dense, tq)
        assert pd.serialize() == pp.serialize()


def test_chunk_causal_forms_byte_identical():
    """One CHUNK_CAUSAL range and its FULL expansion give the same plan bytes
    (so the deterministic kernel gives the same output bits)."""
    for seq, prefix, cs in [(2048, 128, 2), (2048, 128, 4), (2048, 128, 16), (1000, 100, 3)]:
        a = ma.mask_compile_host("ranges", [0, seq], [seq], ranges=[W.chunk_ranges(seq, prefix, cs)])
        b = ma.mask_compile_host("ranges", [0, seq], [seq], ranges=[W.chunk_ranges_expanded(seq, prefix, cs)])
        assert a.serialize() == b.serialize()
        _check(a, [M.ranges(seq, seq, W.chunk_ranges(seq, prefix, cs))], 128)


def test_equivalent_kinds_byte_identical():
    n = 700
    causal = ma.mask_compile_host("causal", [0, n], [n])
    assert causal.serialize() == ma.mask_compile_host("window", [0, n], [n], window=n).serialize()
    assert causal.serialize() == ma.mask_compile_host("prefix_lm", [0, n], [n], prefix_len=[0]).serialize()
    assert causal.serialize() == ma.mask_compile_host(
        "ranges", [0, n], [n], ranges=[[(0, n, 0, n, 4, 1)]]).serialize()
    assert causal.serialize() == ma.mask_compile_host(
        "dense", [0, n], [n], mask=M.causal(n, n).astype(np.uint8).reshape(-1)).serialize()
    pl = ma.mask_compile_host("prefix_lm", [0, n], [n], prefix_len=[300]).serialize()
    assert pl == ma.mask_compile_host("ranges", [0, n], [n],
                                      ranges=[[(0, 300, 0, 300, 0, 0), (0, n, 0, n, 1, 0)]]).serialize()


def test_workload_shapes_counts():
    """Tile counts at the full workload shapes (tile 128 x 64)."""
    def counts(plan):
        c, _ = plan.export(words=False)
        return int((c == 1).sum()), int((c == 2).sum()), int((c == 0).sum())
    n = 16384
    assert counts(ma.mask_compile_host("causal", [0, n], [n])) == (16256, 256, 16256)
    assert counts(ma.mask_compile_host("window", [0, n], [n], window=4096)) == (6944, 448, 25376)
    for cs in (2, 4, 16):
        p = ma.mask_compile_host("ranges", [0, n], [n], ranges=[W.chunk_ranges(n, 1024, cs)])
        assert counts(p) == (16256, 256, 16256)
    p5 = ma.mask_compile_host("ranges", [0, 32768], [29576],
                              ranges=[W.block_triangle_ranges(32768, 29576, 24576, 50, 100)])
    assert counts(p5) == (98304, 161, 20063)


def test_config5_range_vs_packed_host():
    rg = W.block_triangle_ranges(32768, 29576, 24576, 50, 100)
    pk = W.block_triangle_packed(32768, 29576, 24576, 50, 100).reshape(-1)
    a = ma.mask_compile_host("ranges", [0, 32768], [29576], ranges=[rg])
    b = ma.mask_compile_host("packed", [0, 32768], [29576], mask=pk)
    assert a.serialize() == b.serialize()


def test_execution_order_most_work_first():
    p = ma.mask_compile_host("causal", [0, 1024], [1024])
    data = np.frombuffer(p.serialize(), dtype=np.int32)
    # first item is the last q-tile (most tiles), last item is q-tile 0
    assert data[4 + 1] == 7
    info = p.info()
    assert info.num_qtiles == 8 and info.num_tiles == 8 * 16 and info.host_valid == 1


def _bsr_arrays(rng, q_lens, kv_lens, br, bc, p):
    indptr, indices, dense = [0], [], []
    for q, k in zip(q_lens, kv_lens):
        nrb, ncb = -(-q // br), -(-k // bc)
        blocks = rng.random((nrb, ncb)) < p
        blocks[0, :] = True if ncb else blocks[0, :]   # a dense block row (FULL tiles)
        for rb in range(nrb):
            cols = list(np.flatnonzero(blocks[rb]))
            rng.shuffle(cols)
            indices += cols
            indptr.append(len(indices))
        dense.append(np.kron(blocks, np.ones((br, bc), dtype=bool))[:q, :k])
    return np.array(indptr), np.array(indices), dense


@pytest.mark.parametrize("br,bc", [(16, 32), (64, 64), (128, 64), (7, 100), (1, 1)])
def test_block_sparse_host(br, bc):
    """Block-sparse descriptions compile to the oracle's classes and words,
    and to the same plan bytes as the equal dense mask."""
    rng = np.random.default_rng(br * 131 + bc)
    q_lens, kv_lens = [300, 5, 130], [900, 70, 130]
    indptr, indices, dense = _bsr_arrays(rng, q_lens, kv_lens, br, bc, 0.3)
    flat = np.concatenate([d.astype(np.uint8).reshape(-1) for d in dense])
    for tq in (64, 128):
        pb = ma.mask_compile_host("block_sparse", _cu(q_lens), kv_lens, bsr=(br, bc, indptr, indices), tile_q=tq)
        _check(pb, dense, tq)
        pd = ma.mask_compile_host("dense", _cu(q_lens), kv_lens, mask=flat, tile_q=tq)
        assert pb.serialize() == pd.serialize()


def test_window_intersections_host():
    """A window with a custom (dense / packed) or block-sparse mask is the
    intersection with the window band: same plan bytes as the intersected
    dense mask, and the oracle's classes and words."""
    rng = np.random.default_rng(77)
    q_lens, kv_lens = [300, 5, 130], [900, 70, 130]
    indptr, indices, bdense = _bsr_arrays(rng, q_lens, kv_lens, 32, 64, 0.5)
    custom = [rng.random((q, k)) < 0.6 for q, k in zip(q_lens, kv_lens)]
    flat = np.concatenate([d.astype(np.uint8).reshape(-1) for d in custom])
    packed = np.concatenate([W.pack_rows(d).reshape(-1) for d in custom])
    for win in (1, 37, 200, 5000):
        band = [M.window_band(q, k, win) for q, k in zip(q_lens, kv_lens)]
        want_c = [c & b for c, b in zip(custom, band)]
        want_b = [c & b for c, b in zip(bdense, band)]
        ref_c = ma.mask_compile_host("dense", _cu(q_lens), kv_lens,
                                     mask=np.concatenate([d.astype(np.uint8).reshape(-1) for d in want_c]))
        for kind, mk in (("dense", flat), ("packed", packed)):
            p = ma.mask_compile_host(kind, _cu(q_lens), kv_lens, mask=mk, window=win)
            _check(p, want_c, 128)
            assert p.serialize() == ref_c.serialize()
        pb = ma.mask_compile_host("block_sparse", _cu(q_lens), kv_lens, bsr=(32, 64, indptr, indices), window=win)
        _check(pb, want_b, 128)


def test_block_sparse_and_window_validation():
    cu, kv = [0, 10], [20]
    ok = (4, 8, [0, 1, 1, 2], [0, 2])
    ma.mask_compile_host("block_sparse", cu, kv, bsr=ok)
    bad = [
        ((0, 8, [0, 1, 1, 2], [0, 2]), ma.MaskAttnError),      # block_r 0
        ((4, 8, [0, 2, 1, 2], [0, 2]), ma.MaskAttnError),      # indptr decreases
        ((4, 8, [0, 1, 1, 2], [0, 3]), ma.MaskAttnError),      # column 3 >= ceil(20 / 8)
        ((4, 8, [1, 1, 1, 2], [0, 2]), ma.MaskAttnError),      # indptr[0] != 0
    ]
    for bsr, exc in bad:
        with pytest.raises(exc):
            ma.mask_compile_host("block_sparse", cu, kv, bsr=bsr)
    with pytest.raises(ma.MaskAttnError) as e:                 # block-sparse arrays with another kind
        ma.mask_compile_host("causal", cu, kv, bsr=ok)
    assert e.value.status == L.MA_ERR_CONFLICT
    for kind, kw in (("prefix_lm", {"prefix_len": [3]}), ("ranges", {"ranges": [[(0, 10, 0, 20, 0, 0)]]}),
                     ("causal", {})):
        with pytest.raises(ma.MaskAttnError):
            ma.mask_compile_host(kind, cu, kv, window=4, **kw)
    with pytest.raises(ma.MaskAttnError):
        ma.mask_compile_host("dense", cu, kv, mask=np.ones(200, np.uint8), window=-1)
