"""Pins for oracle.attention: textbook routine, closed forms and invariants
(CPU only)."""

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import masks as M


def _sdpa(q, k, v, mask=None, causal=False, scale=None):
    t = lambda x: torch.from_numpy(np.asarray(x, dtype=np.float64))[None, None]
    am = None if mask is None else torch.from_numpy(mask)[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=am, is_causal=causal, scale=scale)
    return out[0, 0].numpy()


@pytest.mark.parametrize("n,m,d", [(17, 17, 8), (33, 33, 16)])
def test_vs_sdpa_causal_and_unmasked(n, m, d):
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((x, d)) for x in (n, m, m))
    sc = 1 / np.sqrt(d)
    o, _ = A.attend(q, k, v, M.causal(n, m), sc)
    assert np.allclose(o, _sdpa(q, k, v, causal=True, scale=sc), atol=1e-12)
    o, _ = A.attend(q, k, v, np.ones((n, m), bool), sc)
    assert np.allclose(o, _sdpa(q, k, v, scale=sc), atol=1e-12)


def test_vs_sdpa_bool_mask_rectangular():
    rng = np.random.default_rng(4)
    n, m, d, dv = 9, 21, 8, 5
    q, k = rng.standard_normal((n, d)), rng.standard_normal((m, d))
    v = rng.standard_normal((m, dv))
    mask = rng.random((n, m)) < 0.4
    mask[:, 0] = True
    o, _ = A.attend(q, k, v, mask, 0.3)
    assert np.allclose(o, _sdpa(q, k, v, mask=mask, scale=0.3), atol=1e-12)


def test_lse_closed_form_and_probe():
    """Q = 0 makes every score 0: LSE = ln(#visible) and, with V = I, O[t, j] =
    M[t, j] / sum_j M[t, j] — the mask read back through the attention."""
    n, m = 6, 8
    for mask in (M.causal(n, m), M.sliding_window(n, m, 3), M.prefix_lm(n, m, 5),
                 M.ranges(n, m, [(0, 6, 0, 8, M.CHUNK_CAUSAL, 2)])):
        o, lse = A.attend(np.zeros((n, 4)), np.ones((m, 4)), np.eye(m), mask, 1.0)
        cnt = mask.sum(axis=1)
        assert np.allclose(lse, np.log(cnt), atol=1e-15)
        assert np.allclose(o, mask / cnt[:, None], atol=1e-15)


def test_single_key_and_empty_rows():
    rng = np.random.default_rng(5)
    q, k, v = rng.standard_normal((3, 4)), rng.standard_normal((5, 4)), rng.standard_normal((5, 4))
    mask = np.zeros((3, 5), bool)
    mask[0, 2] = True          # exactly one visible key
    mask[2, [1, 3]] = True
    o, lse = A.attend(q, k, v, mask, 0.5)
    assert np.array_equal(o[0], v[2])                       # bit-exact
    assert lse[0] == pytest.approx(0.5 * q[0] @ k[2], abs=1e-15)
    assert np.array_equal(o[1], np.zeros(4)) and lse[1] == -np.inf
    w = np.exp(0.5 * np.array([q[2] @ k[1], q[2] @ k[3]]))
    assert np.allclose(o[2], (w[0] * v[1] + w[1] * v[3]) / w.sum(), atol=1e-14)


def test_two_key_formula_catches_transposes():
    """Closed form for two visible keys with distinct d and dv."""
    q = np.array([[1.0, 2.0, 0.5]])
    k = np.array([[0.5, -1.0, 2.0], [1.5, 0.0, -0.5]])
    v = np.array([[1.0, 2.0], [-3.0, 4.0]])
    o, lse = A.attend(q, k, v, np.ones((1, 2), bool), 0.7)
    s = 0.7 * np.array([0.5 - 2.0 + 1.0, 1.5 + 0.0 - 0.25])
    p = np.exp(s - s.max())
    assert np.allclose(o[0], (p[0] * v[0] + p[1] * v[1]) / p.sum(), atol=1e-15)
    assert lse[0] == pytest.approx(np.log(np.exp(s).sum()), abs=1e-14)


def test_invariants_shift_convexity():
    rng = np.random.default_rng(6)
    n, m, d = 12, 30, 8
    q, k, v = rng.standard_normal((n, d)), rng.standard_normal((m, d)), rng.standard_normal((m, d))
    mask = M.sliding_window(n, m, 9)
    o, lse = A.attend(q, k, v, mask, 0.4)
    c = rng.standard_normal(d)
    o2, lse2 = A.attend(q, k + c, v, mask, 0.4)
    assert np.allclose(o, o2, atol=1e-12)
    assert np.allclose(lse2 - lse, 0.4 * q @ c, atol=1e-12)
    for t in range(n):
        vis = v[mask[t]]
        assert (o[t] >= vis.min(0) - 1e-12).all() and (o[t] <= vis.max(0) + 1e-12).all()


def _paged(rng, kv_lens, hkv, d, page, permute):
    pages = [(k + page - 1) // page for k in kv_lens]
    total = sum(pages) + 1
    perm = rng.permutation(total) if permute else np.arange(total)
    cache = np.full((total, page, hkv, d), np.nan)
    table = np.full((len(kv_lens), max(pages)), perm[-1])
    dense = []
    off = 0
    for b, kl in enumerate(kv_lens):
        vals = rng.standard_normal((kl, hkv, d))
        dense.append(vals)
        for i in range(pages[b]):
            table[b, i] = perm[off + i]
            nn = min(page, kl - i * page)
            cache[perm[off + i], :nn] = vals[i * page:i * page + nn]
        off += pages[b]
    return cache, table, dense


def test_paged_ragged_gqa():
    """Ragged batch over a permuted paged cache equals per-sequence dense
    attention; GQA equals MHA with each K/V head repeated for its group."""
    rng = np.random.default_rng(7)
    kv_lens, q_lens, hq, hkv, d, page = [37, 5, 64], [37, 2, 10], 4, 2, 8, 4
    kc, table, kd = _paged(rng, kv_lens, hkv, d, page, True)
    vc, _, vd = _paged(np.random.default_rng(8), kv_lens, hkv, d, page, True)
    # the two caches must share the same table for the test to make sense
    vc2 = np.full_like(kc, np.nan)
    for b, kl in enumerate(kv_lens):
        for j in range(kl):
            vc2[table[b, j // page], j % page] = vd[b][j]
    cu = np.concatenate([[0], np.cumsum(q_lens)])
    q = rng.standard_normal((cu[-1], hq, d))
    masks = [M.causal(ql, kl) for ql, kl in zip(q_lens, kv_lens)]
    o, lse = A.attention(q, kc, vc2, table, cu, kv_lens, masks, 0.35)
    assert not np.isnan(o).any()
    for b in range(3):
        for h in range(hq):
            g = h // (hq // hkv)
            ob, lb = A.attend(q[cu[b]:cu[b + 1], h], kd[b][:, g], vd[b][:, g], masks[b], 0.35)
            assert np.array_equal(o[cu[b]:cu[b + 1], h], ob)
            assert np.array_equal(lse[cu[b]:cu[b + 1], h], lb)
    # GQA == MHA with repeated K/V heads
    kr = np.repeat(kc, hq // hkv, axis=2)
    vr = np.repeat(vc2, hq // hkv, axis=2)
    o2, _ = A.attention(q, kr, vr, table, cu, kv_lens, masks, 0.35)
    assert np.array_equal(o, o2)
    # sampled rows / heads agree with the full result
    o3, _ = A.attention(q, kc, vc2, table, cu, kv_lens, masks, 0.35, heads=[3], rows={2: [0, 9]})
    assert np.array_equal(o3[cu[2] + np.array([0, 9]), 3], o[cu[2] + np.array([0, 9]), 3])
    assert np.isnan(o3[:, 0]).all()
