"""Dense boolean attention masks, one function per mask kind (oracle; test
infrastructure only).

Every function returns ``M`` of shape ``[q_len, kv_len]`` (numpy bool) for one
sequence, with ``M[t, j]`` true when query row ``t`` may attend to key ``j``.

Coordinates.  Query row ``t`` of a sequence sits at absolute key position
``pos(t) = t + (kv_len - q_len)``: the queries are the last ``q_len`` tokens of
the sequence whose keys are ``0 .. kv_len-1`` (ragged paged attention as in
[sglang-jax#20], highlights).  Range descriptors use per-sequence local
coordinates: ``q_start, q_end`` index query rows, ``k_start, k_end`` index keys.

Readings taken where the pages are silent (each is listed in the design notes):
  * CAUSAL with q_len != kv_len is bottom-right aligned (row t sees j <= pos(t)).
  * A range of type CAUSAL is bottom-right aligned inside its rectangle.
  * CHUNK_CAUSAL is bottom-right aligned inside its rectangle, its last chunk
    is cut at q_end and key ends are clipped to k_end; with k_end == q_end and
    shared coordinates this is exactly the formula on [MagiAttention#316],
    "Semantically equivalent to".
  * INV_CAUSAL (top-left, jj >= i) and BI_CAUSAL (CAUSAL and INV_CAUSAL): the
    page gives only the names and calls BI_CAUSAL an aligned band
    ("Why existing mask types are not enough").  Parity unpinned.
  * Sliding window W keeps W keys including the query's own position:
    pos - W < j <= pos.  [mlxcel#555] only says the window is ANDed into the
    causal mask and that W >= the sequence length changes nothing.  Parity
    unpinned beyond that.
  * Overlapping range descriptors are OR-ed.
  * Block-sparse masks ([flashinfer#724] recommends its block-sparse API for
    long sequences; the page gives no layout): blocks of block_r rows x
    block_c keys listed per block row in CSR form; a key is visible when its
    block is listed.  The last block row / column is cut at q_len / kv_len.
  * A sliding window given with a custom or block-sparse mask is ANDed with
    it (the joint use [flashinfer#724] asks about), using the band above.
"""

import numpy as np

# Range types: 0..3 as numbered in the attn_type_map list of [MagiAttention#316]
# ("Why existing mask types are not enough"); 4 is the proposed CHUNK_CAUSAL.
FULL, CAUSAL, INV_CAUSAL, BI_CAUSAL, CHUNK_CAUSAL = 0, 1, 2, 3, 4


def positions(q_len, kv_len):
    """Absolute key position of every query row: t + (kv_len - q_len)."""
    return np.arange(q_len, dtype=np.int64) + (kv_len - q_len)


def _grid(q_len, kv_len):
    pos = positions(q_len, kv_len)[:, None]
    j = np.arange(kv_len, dtype=np.int64)[None, :]
    return pos, j


def causal(q_len, kv_len):
    """Causal mask: row t sees every key at or before its own position
    ([sglang-jax#20], causal flag of the kernel)."""
    pos, j = _grid(q_len, kv_len)
    return j <= pos


def sliding_window(q_len, kv_len, window):
    """Gemma2 local mask: the causal mask ANDed with a window of `window`
    keys ending at the query's own position ([mlxcel#555], description)."""
    if window < 1:
        raise ValueError("window must be >= 1")
    pos, j = _grid(q_len, kv_len)
    return (j <= pos) & (j > pos - window)


def prefix_lm(q_len, kv_len, prefix_len):
    """PrefixLM: bidirectional inside the first `prefix_len` keys, causal after
    ([aphrodite#1526], prefixlm_mask_mod).  A key inside the prefix is visible
    to every row; any other key follows the causal rule."""
    if not 0 <= prefix_len <= kv_len:
        raise ValueError("prefix_len out of range")
    pos, j = _grid(q_len, kv_len)
    return (j <= pos) | (j < prefix_len)


def range_block(lq, lk, attn_type, chunk_size=0):
    """Mask of one (q_range, k_range, attn_type) rectangle in local
    coordinates i in [0, lq), jj in [0, lk) ([MagiAttention#316])."""
    i = np.arange(lq, dtype=np.int64)[:, None]
    jj = np.arange(lk, dtype=np.int64)[None, :]
    if attn_type == FULL:
        return np.ones((lq, lk), dtype=bool)
    if attn_type == CAUSAL:
        return jj <= i + (lk - lq)
    if attn_type == INV_CAUSAL:
        return jj >= i
    if attn_type == BI_CAUSAL:
        return (jj <= i + (lk - lq)) & (jj >= i)
    if attn_type == CHUNK_CAUSAL:
        if chunk_size < 1:
            raise ValueError("chunk_size must be >= 1")
        # chunk c = i // cs covers rows [c*cs, min(lq, (c+1)*cs)); it sees keys
        # up to the end of its own chunk, shifted to the bottom-right corner.
        chunk_end = np.minimum(lq, (i // chunk_size + 1) * chunk_size)
        return jj < lk - (lq - chunk_end)
    raise ValueError(f"unknown range type {attn_type}")


def ranges(q_len, kv_len, descs):
    """Union of range descriptors (q_start, q_end, k_start, k_end, type,
    chunk_size) for one sequence."""
    m = np.zeros((q_len, kv_len), dtype=bool)
    for qs, qe, ks, ke, ty, cs in descs:
        if not (0 <= qs <= qe <= q_len and 0 <= ks <= ke <= kv_len):
            raise ValueError("range outside the sequence")
        if qe > qs and ke > ks:
            m[qs:qe, ks:ke] |= range_block(qe - qs, ke - ks, ty, cs)
    return m


def tree_ancestors(parents):
    """Ancestor-or-self sets of a draft tree, by walking parent pointers up to
    the root.  parents[0] is ignored (node 0 is the root); parents[n] < n."""
    n = len(parents)
    anc = np.zeros((n, n), dtype=bool)
    for node in range(n):
        cur = node
        while True:
            anc[node, cur] = True
            if cur == 0:
                break
            p = int(parents[cur])
            if not 0 <= p < cur:
                raise ValueError("parent must precede its child")
            cur = p
    return anc


def tree(ctx_len, parents):
    """Speculative tree-verify mask: node n sees all ctx_len cached keys and
    the keys of its ancestors and itself, which sit at ctx_len + m
    ([flashinfer#724], tree attention through a custom mask)."""
    n = len(parents)
    m = np.zeros((n, ctx_len + n), dtype=bool)
    m[:, :ctx_len] = True
    m[:, ctx_len:] = tree_ancestors(parents)
    return m


def words_per_row(kv_len):
    return (kv_len + 63) // 64


def unpack_rows(words, q_len, kv_len):
    """Bit-packed rows -> dense bool.  Key j of a row is bit (j mod 64) of the
    row's word j // 64 (least-significant bit first); padding bits past kv_len
    are ignored.  The page only says the mask is bit-packed
    ([flashinfer#724], issue text); this bit order is our reading."""
    nw = words_per_row(kv_len)
    w = np.asarray(words, dtype=np.uint64).reshape(q_len, nw)
    out = np.zeros((q_len, nw * 64), dtype=bool)
    for b in range(64):
        out[:, b::64] = ((w >> np.uint64(b)) & np.uint64(1)).astype(bool)
    return out[:, :kv_len]


def dense_from_flat(flat, q_lens, kv_lens):
    """Split the flattened custom mask (one row-major q_len x kv_len block per
    sequence, concatenated; [sglang-jax#20], custom_mask comment) into
    per-sequence dense masks."""
    flat = np.asarray(flat).reshape(-1)
    out, off = [], 0
    for ql, kl in zip(q_lens, kv_lens):
        n = int(ql) * int(kl)
        if off + n > flat.size:
            raise ValueError("custom mask smaller than sum of q_len * kv_len")
        out.append(flat[off:off + n].reshape(int(ql), int(kl)) != 0)
        off += n
    return out


def packed_from_flat(flat, q_lens, kv_lens):
    """Same as dense_from_flat for the bit-packed form: per sequence q_len rows
    of ceil(kv_len / 64) u64 words, concatenated."""
    flat = np.asarray(flat, dtype=np.uint64).reshape(-1)
    out, off = [], 0
    for ql, kl in zip(q_lens, kv_lens):
        n = int(ql) * words_per_row(int(kl))
        if off + n > flat.size:
            raise ValueError("packed mask smaller than its rows need")
        out.append(unpack_rows(flat[off:off + n], int(ql), int(kl)))
        off += n
    return out


def block_sparse(q_len, kv_len, block_r, block_c, indptr, indices):
    """Block-sparse mask of one sequence: indptr [ceil(q_len / block_r) + 1]
    and indices (block columns) in CSR form over block rows; row t sees key
    j when block (t // block_r, j // block_c) is listed.  Written out entry
    by block entry, no blocking beyond the definition."""
    m = np.zeros((q_len, kv_len), dtype=bool)
    nrb = -(-q_len // block_r)
    for rb in range(nrb):
        r0, r1 = rb * block_r, min(q_len, (rb + 1) * block_r)
        for k in range(int(indptr[rb]), int(indptr[rb + 1])):
            c = int(indices[k])
            m[r0:r1, c * block_c:min(kv_len, (c + 1) * block_c)] = True
    return m


def window_band(q_len, kv_len, window):
    """The sliding-window band alone: pos - window < j <= pos (the set that a
    window intersects a custom or block-sparse mask with)."""
    if window < 1:
        raise ValueError("window must be >= 1")
    pos, j = _grid(q_len, kv_len)
    return (j > pos - window) & (j <= pos)
