"""fp64 masked attention over ragged sequences and paged K/V (oracle; test
infrastructure only).

Definition (the plain statement of what the flash kernel computes; the kernel
reaches the same numbers, up to rounding order, by tiles and an online
softmax):

    S[t, j] = scale * <Q[t], K[j]>                  for keys j < kv_len
    if no j has M[t, j]:   O[t] = 0,  LSE[t] = -inf
    else:                  m = max_{j: M} S[t, j]
                           p_j = M[t, j] * exp(S[t, j] - m)
                           O[t] = sum_j p_j V[j] / sum_j p_j
                           LSE[t] = m + ln(sum_j p_j)

This is softmax(Q K^T * scale + mask) V with a dense boolean mask.  Masked
entries are removed exactly (not by a large negative constant): for a row with
at least one visible key this equals the -1e30 fill of [mlxcel#555]; a row
with no visible key gives 0 rather than the mean of V.

Paged K/V: K[j] = k_cache[page_table[j // P], j % P, g] with P the page size,
and g = h // (Hq // Hkv) the K/V head of query head h (contiguous GQA groups).
Ragged queries: sequence b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]
of q[total_q, Hq, d] ([sglang-jax#20], ragged paged attention).
"""

import numpy as np

ROW_CHUNK = 512


def gather_paged(cache, page_table_row, kv_len, head):
    """Rows 0 .. kv_len-1 of one K/V head from a paged cache
    [num_pages, page_size, H_kv, d], as float64 [kv_len, d]."""
    page_size = cache.shape[1]
    j = np.arange(kv_len, dtype=np.int64)
    pages = np.asarray(page_table_row, dtype=np.int64)[j // page_size]
    return np.asarray(cache[pages, j % page_size, head, :], dtype=np.float64)


def attend(q, k, v, mask, scale):
    """One head of one sequence.  q [n, d], k and v [m, d], mask bool [n, m].
    Returns (O [n, d], LSE [n]) in float64, chunking rows by ROW_CHUNK."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    mask = np.asarray(mask, dtype=bool)
    n, d = q.shape
    o = np.zeros((n, v.shape[1]), dtype=np.float64)
    lse = np.full(n, -np.inf, dtype=np.float64)
    for r0 in range(0, n, ROW_CHUNK):
        r1 = min(n, r0 + ROW_CHUNK)
        mk = mask[r0:r1]
        has = mk.any(axis=1)
        if not has.any():
            continue
        s = scale * (q[r0:r1] @ k.T)
        s = np.where(mk, s, -np.inf)
        m = np.where(has, s.max(axis=1), 0.0)
        p = np.where(mk, np.exp(s - m[:, None]), 0.0)
        l = p.sum(axis=1)
        rows = np.nonzero(has)[0]
        o[r0 + rows] = (p[rows] @ v) / l[rows, None]
        lse[r0 + rows] = m[rows] + np.log(l[rows])
    return o, lse


def attention(q, k_cache, v_cache, page_table, cu_seqlens_q, kv_lens, masks,
              scale, heads=None, rows=None):
    """Ragged, paged, masked attention over a batch.

    q           [total_q, Hq, d] (any float dtype; upcast exactly to fp64)
    k_cache     [num_pages, page_size, Hkv, d], v_cache likewise
    page_table  [B, max_pages] int
    cu_seqlens_q [B+1], kv_lens [B]
    masks       callable b -> dense bool [q_len_b, kv_len_b], or a list
    heads       optional list of query heads to compute (default: all)
    rows        optional dict b -> array of local query rows to compute
    Returns (O [total_q, Hq, d], LSE [total_q, Hq]) float64; entries not
    computed (heads/rows not asked for) are NaN.
    """
    q = np.asarray(q)
    total_q, hq, d = q.shape
    hkv = k_cache.shape[2]
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = hq // hkv
    heads = range(hq) if heads is None else heads
    o = np.full((total_q, hq, v_cache.shape[3]), np.nan, dtype=np.float64)
    lse = np.full((total_q, hq), np.nan, dtype=np.float64)
    batch = len(kv_lens)
    for b in range(batch):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        kl = int(kv_lens[b])
        mk = masks(b) if callable(masks) else masks[b]
        sel = np.arange(q1 - q0) if rows is None or b not in rows else np.asarray(rows[b])
        if sel.size == 0:
            continue
        for h in heads:
            g = h // group
            k = gather_paged(k_cache, page_table[b], kl, g)
            v = gather_paged(v_cache, page_table[b], kl, g)
            ob, lb = attend(q[q0 + sel, h, :], k, v, mk[sel], scale)
            o[q0 + sel, h, :] = ob
            lse[q0 + sel, h] = lb
    return o, lse
