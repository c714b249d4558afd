"""Pins for oracle.masks against the pages' worked examples, closed forms and
brute force (CPU only)."""

import os

import numpy as np
import pytest

from oracle import masks as M

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


# --------------------------------------------------------------------------
# CHUNK_CAUSAL: worked example of MagiAttention #316
# --------------------------------------------------------------------------
def test_chunk_causal_worked_example():
    rows = _read("chunk_causal_worked_example.txt")
    compact = [r for r in rows if r[0] == "compact"][0]
    qs, qe, ks, ke, cs = map(int, compact[1:6])
    n = 200
    chunk = M.ranges(n, n, [(qs, qe, ks, ke, M.CHUNK_CAUSAL, cs)])
    # the printed FULL ranges
    for r in rows:
        if r[0] != "full":
            continue
        a, b, c, d = map(int, r[1:5])
        for t in range(a, b):
            vis = np.nonzero(chunk[t])[0]
            assert vis.min() == c and vis.max() == d - 1 and vis.size == d - c
    # the whole pattern the page elides with "...": q=[100+2c, 102+2c), k=[0, 102+2c)
    full = [(100 + 2 * c, 102 + 2 * c, 0, 102 + 2 * c, M.FULL, 0) for c in range(50)]
    assert np.array_equal(chunk, M.ranges(n, n, full))
    # rows outside q_range see nothing
    assert not chunk[:100].any()


def test_chunk_causal_not_causal_nor_bicausal():
    """The page's negative example: under CAUSAL token_i cannot see latent_i;
    under CHUNK_CAUSAL(2) it can.  BI_CAUSAL is a band, not prefix + chunk."""
    n, pre = 40, 10
    chunk = M.ranges(n, n, [(0, pre, 0, pre, M.CAUSAL, 0), (pre, n, 0, n, M.CHUNK_CAUSAL, 2)])
    caus = M.causal(n, n)
    for i in range((n - pre) // 2):
        tok, lat = pre + 2 * i, pre + 2 * i + 1
        assert chunk[tok, lat] and not caus[tok, lat]
        assert chunk[lat, tok] and chunk[tok, :tok].all()
    bi = M.ranges(n, n, [(pre, n, 0, n, M.BI_CAUSAL, 0)])
    assert not np.array_equal(bi[pre:], chunk[pre:])


@pytest.mark.parametrize("lq,lk", [(7, 7), (5, 9), (9, 12), (12, 12), (3, 20)])
def test_chunk_special_sizes(lq, lk):
    # chunk size 1 is CAUSAL (bottom-right); chunk size >= lq is FULL
    assert np.array_equal(M.range_block(lq, lk, M.CHUNK_CAUSAL, 1), M.range_block(lq, lk, M.CAUSAL))
    assert M.range_block(lq, lk, M.CHUNK_CAUSAL, lq).all()
    assert M.range_block(lq, lk, M.CHUNK_CAUSAL, lq + 5).all()


def test_chunk_brute_force():
    """Row-by-row statement of the chunk rule: the chunk containing local row
    i ends at e = min(lq, (i // cs + 1) * cs) and sees keys jj < lk - lq + e."""
    for lq, lk, cs in [(10, 10, 3), (11, 15, 4), (6, 9, 2), (13, 13, 5)]:
        blk = M.range_block(lq, lk, M.CHUNK_CAUSAL, cs)
        for i in range(lq):
            e = min(lq, (i // cs + 1) * cs)
            for jj in range(lk):
                assert blk[i, jj] == (jj < lk - lq + e)


def test_range_types_small():
    # hand-written 3x3 blocks for every type (square: no alignment question)
    F, C, I, B = (M.range_block(3, 3, t) for t in (M.FULL, M.CAUSAL, M.INV_CAUSAL, M.BI_CAUSAL))
    assert F.all()
    assert np.array_equal(C, np.array([[1, 0, 0], [1, 1, 0], [1, 1, 1]], bool))
    assert np.array_equal(I, np.array([[1, 1, 1], [0, 1, 1], [0, 0, 1]], bool))
    assert np.array_equal(B, np.eye(3, dtype=bool))
    # bottom-right CAUSAL for a wide rectangle: last row sees every key
    wide = M.range_block(2, 5, M.CAUSAL)
    assert np.array_equal(wide, np.array([[1, 1, 1, 1, 0], [1, 1, 1, 1, 1]], bool))


@pytest.mark.parametrize("lq,lk", [(1, 1), (4, 4), (7, 7), (5, 9), (9, 5), (3, 16), (16, 3)])
def test_inv_and_bi_causal_relations(lq, lk):
    """Relations the reading of INV_CAUSAL / BI_CAUSAL (MagiAttention issue
    316 names them: a band aligned the other way, and the intersection of
    both) must satisfy, on squares and rectangles: BI = CAUSAL AND INV; on a
    square INV is CAUSAL transposed; INV is top-left aligned (row i starts at
    key i, sees every key after it), CAUSAL bottom-right aligned; on squares
    and wide rectangles CAUSAL OR INV covers every entry.  (Parity stays unpinned beyond these relations: the page
    gives no matrix for either type.)"""
    C = M.range_block(lq, lk, M.CAUSAL)
    I = M.range_block(lq, lk, M.INV_CAUSAL)
    B = M.range_block(lq, lk, M.BI_CAUSAL)
    assert np.array_equal(B, C & I)
    if lq == lk:
        assert np.array_equal(I, C.T)
        assert np.array_equal(B, np.eye(lq, dtype=bool))
    i = np.arange(lq)[:, None]
    jj = np.arange(lk)[None, :]
    assert np.array_equal(I, jj >= i)                       # top-left aligned
    assert np.array_equal(C, jj <= i + (lk - lq))           # bottom-right aligned
    # on squares and wide rectangles the two half-lines of a row overlap, so
    # CAUSAL | INV covers every entry
    if lk >= lq:
        assert (C | I).all()


def test_ranges_union_and_bounds():
    m = M.ranges(4, 6, [(0, 2, 0, 2, M.FULL, 0), (1, 4, 3, 6, M.FULL, 0)])
    exp = np.zeros((4, 6), bool)
    exp[0:2, 0:2] = True
    exp[1:4, 3:6] = True
    assert np.array_equal(m, exp)
    with pytest.raises(ValueError):
        M.ranges(4, 6, [(0, 5, 0, 2, M.FULL, 0)])
    with pytest.raises(ValueError):
        M.range_block(3, 3, M.CHUNK_CAUSAL, 0)


# --------------------------------------------------------------------------
# causal, window, prefix-LM
# --------------------------------------------------------------------------
@pytest.mark.parametrize("q,k", [(16, 16), (5, 16), (1, 9)])
def test_causal_closed_form(q, k):
    m = M.causal(q, k)
    # bottom-right: row t sees exactly t + (k - q) + 1 keys, a prefix
    for t in range(q):
        n = t + k - q + 1
        assert m[t, :n].all() and not m[t, n:].any()
    if q == k:
        assert m.sum() == q * (q + 1) // 2
        assert np.array_equal(m, np.tril(np.ones((q, q), bool)))


def test_window_special_cases():
    n = 33
    assert np.array_equal(M.sliding_window(n, n, n), M.causal(n, n))
    assert np.array_equal(M.sliding_window(n, n, 10 * n), M.causal(n, n))
    assert np.array_equal(M.sliding_window(n, n, 1), np.eye(n, dtype=bool))
    for w in (1, 4, 7, 32):
        m = M.sliding_window(n, n, w)
        assert m.sum() == sum(min(w, t + 1) for t in range(n))
        for t in range(n):
            vis = np.nonzero(m[t])[0]
            assert vis.max() == t and vis.size == min(w, t + 1)
    with pytest.raises(ValueError):
        M.sliding_window(4, 4, 0)


def test_prefix_lm_special_cases():
    n = 20
    assert np.array_equal(M.prefix_lm(n, n, 0), M.causal(n, n))
    assert M.prefix_lm(n, n, n).all()
    p = 7
    m = M.prefix_lm(n, n, p)
    # bidirectional inside the prefix, causal after it
    assert m[:p, :p].all()
    assert not m[:p, p:].any()
    assert np.array_equal(m[p:], M.causal(n, n)[p:])
    # the range form used by the PrefixLM workload
    assert np.array_equal(m, M.ranges(n, n, [(0, p, 0, p, M.FULL, 0), (0, n, 0, n, M.CAUSAL, 0)]))


# --------------------------------------------------------------------------
# tree verify
# --------------------------------------------------------------------------
def test_tree_golden():
    rows = _read("tree_small.txt")
    parents = [int(x) for x in rows[0][1:]]
    anc = M.tree_ancestors(parents)
    for r in rows[1:]:
        node = int(r[1])
        want = sorted(int(x) for x in r[3:])
        assert sorted(np.nonzero(anc[node])[0].tolist()) == want
    m = M.tree(5, parents)
    assert m.shape == (7, 12) and m[:, :5].all()
    assert np.array_equal(m[:, 5:], anc)


def test_tree_vs_transitive_closure():
    """Ancestor-or-self = reflexive-transitive closure of the parent relation
    (computed by repeated boolean matrix products)."""
    rng = np.random.default_rng(0)
    for n in (1, 2, 9, 64):
        parents = [0] + [int(rng.integers(0, i)) for i in range(1, n)]
        par = np.zeros((n, n), dtype=np.int64)
        for i in range(1, n):
            par[i, parents[i]] = 1
        reach = np.eye(n, dtype=np.int64)
        for _ in range(n):
            reach = ((reach + reach @ par) > 0).astype(np.int64)
        assert np.array_equal(M.tree_ancestors(parents), reach.astype(bool))


def test_tree_inside_causal():
    rng = np.random.default_rng(1)
    parents = [0] + [int(rng.integers(0, i)) for i in range(1, 64)]
    m = M.tree(100, parents)
    assert not (m & ~M.causal(64, 164)).any()
    assert m[:, 100:].diagonal().all()


# --------------------------------------------------------------------------
# packed and flattened layouts
# --------------------------------------------------------------------------
def test_packed_golden():
    rows = dict((r[0], r[1:]) for r in _read("packed_bits.txt"))
    kv = int(rows["kv_len"][0])
    words = np.array([int(x, 16) for x in rows["words"]], dtype=np.uint64)
    dense = M.unpack_rows(words, 1, kv)
    assert sorted(np.nonzero(dense[0])[0].tolist()) == [int(x) for x in rows["visible"]]
    # padding bits are ignored
    noisy = words.copy()
    noisy[1] |= np.uint64(1) << np.uint64(60)
    assert np.array_equal(M.unpack_rows(noisy, 1, kv), dense)


def test_unpack_vs_bit_loop():
    rng = np.random.default_rng(2)
    q, kv = 5, 130
    words = rng.integers(0, 2 ** 63, size=(q, 3), dtype=np.uint64) * np.uint64(2) + np.uint64(1)
    dense = M.unpack_rows(words.reshape(-1), q, kv)
    for t in range(q):
        for j in range(kv):
            assert dense[t, j] == bool((int(words[t, j // 64]) >> (j % 64)) & 1)


def test_flat_layouts():
    # two sequences: (q=2, kv=3) then (q=1, kv=2); row-major, concatenated
    flat = np.array([1, 0, 1, 0, 1, 1, 0, 1], dtype=np.uint8)
    a, b = M.dense_from_flat(flat, [2, 1], [3, 2])
    assert np.array_equal(a, np.array([[1, 0, 1], [0, 1, 1]], bool))
    assert np.array_equal(b, np.array([[0, 1]], bool))
    with pytest.raises(ValueError):
        M.dense_from_flat(flat[:7], [2, 1], [3, 2])
    words = np.array([0b101, 0b011, 0b10], dtype=np.uint64)
    a, b = M.packed_from_flat(words, [2, 1], [3, 2])
    assert np.array_equal(a, np.array([[1, 0, 1], [1, 1, 0]], bool))
    assert np.array_equal(b, np.array([[0, 1]], bool))


# --------------------------------------------------------------------------
# Block-sparse masks and the window band


def _random_bsr(rng, q_len, kv_len, br, bc, p=0.4, repeat=True):
    nrb, ncb = -(-q_len // br), -(-kv_len // bc)
    blocks = rng.random((nrb, ncb)) < p
    indptr, indices = [0], []
    for rb in range(nrb):
        cols = list(np.flatnonzero(blocks[rb]))
        if repeat and cols:
            cols.append(cols[0])                 # a repeated block is the same block
        rng.shuffle(cols)
        indices += cols
        indptr.append(len(indices))
    return blocks, np.array(indptr), np.array(indices, dtype=np.int64)


@pytest.mark.parametrize("q_len,kv_len,br,bc", [(37, 53, 8, 16), (64, 64, 64, 64), (5, 130, 3, 7), (1, 1, 1, 1)])
def test_block_sparse_is_kron_of_blocks(q_len, kv_len, br, bc):
    """Library routine: the mask is the block matrix expanded by np.kron with
    a block of ones, cut to [q_len, kv_len]."""
    rng = np.random.default_rng(q_len * 1000 + kv_len)
    blocks, indptr, indices = _random_bsr(rng, q_len, kv_len, br, bc)
    want = np.kron(blocks, np.ones((br, bc), dtype=bool))[:q_len, :kv_len]
    assert np.array_equal(M.block_sparse(q_len, kv_len, br, bc, indptr, indices), want)


def test_block_sparse_special_cases():
    rng = np.random.default_rng(3)
    q_len, kv_len = 23, 41
    # 1 x 1 blocks list exactly the visible entries: any dense mask round-trips
    dense = rng.random((q_len, kv_len)) < 0.3
    indptr = np.concatenate([[0], np.cumsum(dense.sum(1))])
    indices = np.concatenate([np.flatnonzero(r) for r in dense])
    assert np.array_equal(M.block_sparse(q_len, kv_len, 1, 1, indptr, indices), dense)
    # every block listed: all true; none: all false
    nrb, ncb = -(-q_len // 5), -(-kv_len // 6)
    full = M.block_sparse(q_len, kv_len, 5, 6, np.arange(nrb + 1) * ncb, np.tile(np.arange(ncb), nrb))
    assert full.all()
    assert not M.block_sparse(q_len, kv_len, 5, 6, np.zeros(nrb + 1, int), np.zeros(0, int)).any()
    # a column listed twice in a block row is the same as listed once
    ip1 = np.arange(nrb + 1)
    ix1 = np.arange(nrb) % ncb
    ip2 = 2 * np.arange(nrb + 1)
    ix2 = np.repeat(ix1, 2)
    assert np.array_equal(M.block_sparse(q_len, kv_len, 5, 6, ip1, ix1), M.block_sparse(q_len, kv_len, 5, 6, ip2, ix2))


def test_window_band():
    """The band alone is the sliding-window kind's set; a window at least as
    long as the keys leaves the causal mask; window 1 is the diagonal."""
    for q_len, kv_len in [(30, 30), (7, 50)]:
        for w in (1, 5, 29, 60):
            assert np.array_equal(M.window_band(q_len, kv_len, w), M.sliding_window(q_len, kv_len, w))
        assert np.array_equal(M.window_band(q_len, kv_len, kv_len), M.causal(q_len, kv_len))
        band = M.window_band(q_len, kv_len, 1)
        assert (band.sum(1) == 1).all() and (np.argmax(band, 1) == M.positions(q_len, kv_len)).all()
