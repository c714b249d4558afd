"""fp64 gradients of masked attention over ragged sequences and paged K/V
(oracle; test infrastructure only).

Definition.  With the forward definition of oracle.attention (S = scale Q K^T
over visible keys, P[t, j] = M[t, j] exp(S[t, j] - LSE[t]) the row-normalised
probabilities, O = P V; a row with no visible key has P = 0 and O = 0) and an
upstream gradient dO, the derivatives of O = softmax(scale Q K^T + mask) V
are, per query head of one sequence:

    dV[j]    = sum_t P[t, j] dO[t]
    dP[t, j] = <dO[t], V[j]>
    D[t]     = sum_j P[t, j] dP[t, j]          (= <dO[t], O[t]>)
    dS[t, j] = P[t, j] (dP[t, j] - D[t])        (the softmax Jacobian
                                                 diag(p) - p p^T, row by row)
    dQ[t]    = scale sum_j dS[t, j] K[j]
    dK[j]    = scale sum_t dS[t, j] Q[t]

A K/V head's gradients sum those of its query heads (contiguous GQA groups).
Paged K/V: dK and dV are cache-shaped, each key's gradient at its (page,
slot); cache slots no sequence uses stay 0.  This is the same backward the
kernels compute over the plan (masked entries carry P = 0, so they add
nothing anywhere).
"""

import numpy as np

from .attention import gather_paged


def attend_backward(q, k, v, mask, scale, do):
    """One query head of one sequence: q and do [n, d], k and v [m, d], mask
    bool [n, m].  Returns (dq [n, d], dk [m, d], dv [m, d]) in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    mask = np.asarray(mask, dtype=bool)
    has = mask.any(axis=1)
    s = np.where(mask, scale * (q @ k.T), -np.inf)
    m = np.where(has, s.max(axis=1, initial=-np.inf), 0.0)
    e = np.where(mask, np.exp(s - m[:, None]), 0.0)
    l = e.sum(axis=1)
    p = np.where(has[:, None], e / np.where(has, l, 1.0)[:, None], 0.0)
    dv = p.T @ do
    dp = do @ v.T
    dd = (p * dp).sum(axis=1)
    ds = p * (dp - dd[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def attend_backward_sampled(q, k, v, mask, scale, do, rows, keys, chunk=1024):
    """attend_backward evaluated only where asked: dq for the query rows
    `rows` and dk, dv for the keys `keys` of one head (q, do [n, d]; k, v
    [m, d]; mask bool [n, m] or a callable (r0, r1) -> mask rows r0..r1-1).
    The same definition, taken over row chunks so that no n x m matrix is
    held: per chunk S, P (with the chunk's own row normaliser), dP and
    D = rowsum(P dP) are exact row by row, and the dk / dv sums over rows are
    accumulated chunk by chunk.  Returns (dq [len(rows), d], dk [len(keys),
    d], dv [len(keys), d]) in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    n = q.shape[0]
    dq = np.zeros((len(rows), k.shape[1]))
    dk = np.zeros((len(keys), q.shape[1]))
    dv = np.zeros((len(keys), do.shape[1]))
    for r0 in range(0, n, chunk):
        r1 = min(n, r0 + chunk)
        mk = mask(r0, r1) if callable(mask) else np.asarray(mask[r0:r1], dtype=bool)
        has = mk.any(axis=1)
        s = np.where(mk, scale * (q[r0:r1] @ k.T), -np.inf)
        m = np.where(has, s.max(axis=1, initial=-np.inf), 0.0)
        e = np.where(mk, np.exp(s - m[:, None]), 0.0)
        l = e.sum(axis=1)
        p = np.where(has[:, None], e / np.where(has, l, 1.0)[:, None], 0.0)
        dp = do[r0:r1] @ v.T
        dd = (p * dp).sum(axis=1)
        ds = p * (dp - dd[:, None])
        dv += p[:, keys].T @ do[r0:r1]
        dk += scale * (ds[:, keys].T @ q[r0:r1])
        sel = (rows >= r0) & (rows < r1)
        if sel.any():
            dq[sel] = scale * (ds[rows[sel] - r0] @ k)
    return dq, dk, dv


def attention_backward(q, k_cache, v_cache, page_table, cu_seqlens_q, kv_lens, masks, scale, do,
                       kv_heads=None):
    """Gradients of the ragged, paged, masked attention of oracle.attention.

    q, do       [total_q, Hq, d]
    k_cache     [num_pages, page_size, Hkv, d], v_cache likewise
    page_table  [B, max_pages];  cu_seqlens_q [B+1];  kv_lens [B]
    masks       callable b -> dense bool [q_len_b, kv_len_b], or a list
    kv_heads    optional list of K/V heads to compute (with all their query
                heads); dq of the other query heads is NaN and their dK / dV
                entries are 0
    Returns (dq [total_q, Hq, d], dk_cache, dv_cache) float64.
    """
    q = np.asarray(q)
    do = np.asarray(do)
    total_q, hq, d = q.shape
    hkv = k_cache.shape[2]
    group = hq // hkv
    page_size = k_cache.shape[1]
    kv_heads = range(hkv) if kv_heads is None else kv_heads
    dq = np.full((total_q, hq, d), np.nan, dtype=np.float64)
    dk_cache = np.zeros(k_cache.shape, dtype=np.float64)
    dv_cache = np.zeros(v_cache.shape, dtype=np.float64)
    for b in range(len(kv_lens)):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        kl = int(kv_lens[b])
        mk = masks(b) if callable(masks) else masks[b]
        j = np.arange(kl, dtype=np.int64)
        pages = np.asarray(page_table[b], dtype=np.int64)[j // page_size]
        slots = j % page_size
        for g in kv_heads:
            k = gather_paged(k_cache, page_table[b], kl, g)
            v = gather_paged(v_cache, page_table[b], kl, g)
            dk = np.zeros((kl, d))
            dv = np.zeros((kl, v.shape[1]))
            for h in range(g * group, (g + 1) * group):
                dqh, dkh, dvh = attend_backward(q[q0:q1, h, :], k, v, mk, scale, do[q0:q1, h, :])
                dq[q0:q1, h, :] = dqh
                dk += dkh
                dv += dvh
            dk_cache[pages, slots, g, :] += dk
            dv_cache[pages, slots, g, :] += dv
    return dq, dk_cache, dv_cache
