"""Pins for oracle.backward (CPU only): central finite differences of the
forward oracle, autograd of torch's fp64 scaled-dot-product attention, closed
forms and invariants."""

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import backward as B
from oracle import masks as M


def _paged_problem(seed, q_lens, kv_lens, hq, hkv, d, page, empty_row=True):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
    pages = [(k + page - 1) // page for k in kv_lens]
    total = sum(pages) + 1
    perm = rng.permutation(total)
    table = np.zeros((len(kv_lens), max(pages)), np.int64)
    off = 0
    for b, n in enumerate(pages):
        table[b, :n] = perm[off:off + n]
        off += n
    q = rng.standard_normal((cu[-1], hq, d))
    kc = rng.standard_normal((total, page, hkv, d))
    vc = rng.standard_normal((total, page, hkv, d))
    do = rng.standard_normal((cu[-1], hq, d))
    masks = []
    for ql, kl in zip(q_lens, kv_lens):
        mk = rng.random((ql, kl)) < 0.5
        mk[:, kl - 1] = True
        if empty_row and ql > 2:
            mk[1, :] = False
        masks.append(mk)
    return q, kc, vc, table, cu, np.asarray(kv_lens), masks, do


def _used_slots(table, kv_lens, page):
    used = set()
    for b, kl in enumerate(kv_lens):
        for j in range(int(kl)):
            used.add((int(table[b, j // page]), j % page))
    return used


def test_finite_differences():
    """Every gradient entry equals the central difference of
    L = sum(O * dO) through the forward oracle."""
    q_lens, kv_lens, hq, hkv, d, page = [4, 3], [6, 5], 4, 2, 3, 2
    q, kc, vc, table, cu, kv, masks, do = _paged_problem(11, q_lens, kv_lens, hq, hkv, d, page)
    sc = 0.7
    dq, dk, dv = B.attention_backward(q, kc, vc, table, cu, kv, masks, sc, do)

    def loss(qq, kk, vv):
        o, _ = A.attention(qq, kk, vv, table, cu, kv, masks, sc)
        return float(np.sum(o * do))

    eps = 1e-6
    for arr, grad, name in ((q, dq, "q"), (kc, dk, "k"), (vc, dv, "v")):
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            if name != "q" and (idx[0], idx[1]) not in _used_slots(table, kv, page):
                assert grad[idx] == 0.0
                continue
            old = arr[idx]
            arr[idx] = old + eps
            lp = loss(q, kc, vc)
            arr[idx] = old - eps
            lm = loss(q, kc, vc)
            arr[idx] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


@pytest.mark.parametrize("n,m,d", [(9, 9, 8), (12, 30, 16)])
def test_vs_torch_autograd(n, m, d):
    """The textbook routine: autograd of torch's fp64 SDPA with a boolean mask
    (every row keeps a key: SDPA gives NaN for empty rows)."""
    rng = np.random.default_rng(12)
    q, k, v, do = (rng.standard_normal((x, d)) for x in (n, m, m, n))
    mask = M.causal(n, m) | (rng.random((n, m)) < 0.2)
    sc = 1 / np.sqrt(d)
    t = lambda x: torch.tensor(x, dtype=torch.float64, requires_grad=True)
    tq, tk, tv = t(q[None, None]), t(k[None, None]), t(v[None, None])
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(mask)[None, None],
                                                           scale=sc)
    out.backward(torch.from_numpy(do)[None, None])
    dq, dk, dv = B.attend_backward(q, k, v, mask, sc, do)
    assert np.allclose(dq, tq.grad[0, 0].numpy(), atol=1e-12)
    assert np.allclose(dk, tk.grad[0, 0].numpy(), atol=1e-12)
    assert np.allclose(dv, tv.grad[0, 0].numpy(), atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(13)
    n, m, d = 6, 8, 5
    q, k, v, do = (rng.standard_normal((x, d)) for x in (n, m, m, n))
    mask = rng.random((n, m)) < 0.5
    mask[:, 0] = True
    # dO = 0: every gradient is 0
    for g in B.attend_backward(q, k, v, mask, 0.5, np.zeros_like(do)):
        assert np.all(g == 0)
    # a row that sees one key: P = 1, so its dQ is 0 and that key's dV gets dO
    one = np.zeros((1, m), bool)
    one[0, 3] = True
    dq, dk, dv = B.attend_backward(q[:1], k, v, one, 0.5, do[:1])
    assert np.allclose(dq, 0) and np.allclose(dk, 0)
    assert np.allclose(dv[3], do[0]) and np.allclose(np.delete(dv, 3, axis=0), 0)
    # an empty row contributes nothing
    empty = mask.copy()
    empty[2] = False
    dq, dk, dv = B.attend_backward(q, k, v, empty, 0.5, do)
    assert np.all(dq[2] == 0)
    dq2, dk2, dv2 = B.attend_backward(np.delete(q, 2, 0), k, v, np.delete(empty, 2, 0), 0.5, np.delete(do, 2, 0))
    assert np.allclose(dk, dk2) and np.allclose(dv, dv2)
    # Q = 0 (uniform probabilities over the visible keys): dV[j] = sum over the
    # rows that see j of dO[t] / count(t)
    dq, dk, dv = B.attend_backward(np.zeros_like(q), k, v, mask, 0.5, do)
    want = (mask / mask.sum(1, keepdims=True)).T @ do
    assert np.allclose(dv, want)


def test_invariants():
    rng = np.random.default_rng(14)
    n, m, d = 7, 9, 4
    q, k, v, do = (rng.standard_normal((x, d)) for x in (n, m, m, n))
    mask = rng.random((n, m)) < 0.6
    mask[:, -1] = True
    sc = 0.8
    dq, dk, dv = B.attend_backward(q, k, v, mask, sc, do)
    # K + c shifts each row's scores by a constant: O and dQ do not move
    c = rng.standard_normal(d)
    dq2, _, dv2 = B.attend_backward(q, k + c, v, mask, sc, do)
    assert np.allclose(dq, dq2) and np.allclose(dv, dv2)
    # V + c moves O by c in every non-empty row: dQ and dK do not move
    dq3, dk3, _ = B.attend_backward(q, k, v + c, mask, sc, do)
    assert np.allclose(dq, dq3) and np.allclose(dk, dk3)
    # the loss is linear in dO
    a1 = B.attend_backward(q, k, v, mask, sc, 2.0 * do)
    for g1, g in zip(a1, (dq, dk, dv)):
        assert np.allclose(g1, 2.0 * g)
    # sum_t dV = sum_t dO over non-empty rows (each P row sums to 1)
    assert np.allclose(dv.sum(0), do[mask.any(1)].sum(0))


def test_gqa_sums_query_heads():
    q_lens, kv_lens, hq, hkv, d, page = [5], [9], 4, 1, 6, 4
    q, kc, vc, table, cu, kv, masks, do = _paged_problem(15, q_lens, kv_lens, hq, hkv, d, page, empty_row=False)
    dq, dk, dv = B.attention_backward(q, kc, vc, table, cu, kv, masks, 0.4, do)
    k = A.gather_paged(kc, table[0], 9, 0)
    v = A.gather_paged(vc, table[0], 9, 0)
    dks, dvs = 0, 0
    for h in range(hq):
        a, b, c = B.attend_backward(q[:, h], k, v, masks[0], 0.4, do[:, h])
        assert np.allclose(dq[:, h], a)
        dks, dvs = dks + b, dvs + c
    assert np.allclose(A.gather_paged(dk, table[0], 9, 0), dks)
    assert np.allclose(A.gather_paged(dv, table[0], 9, 0), dvs)


@pytest.mark.parametrize("chunk", [1, 3, 64])
def test_sampled_equals_whole(chunk):
    """The sampled, row-chunked evaluation returns exactly the whole-matrix
    gradients at the sampled rows and keys (a mask given as a matrix and as
    a row-block callable), empty rows included."""
    rng = np.random.default_rng(16)
    n, m, d = 37, 53, 8
    q, k, v, do = (rng.standard_normal((x, d)) for x in (n, m, m, n))
    mask = rng.random((n, m)) < 0.4
    mask[5] = False
    mask[:, 0] |= M.causal(n, m)[:, 0]
    dq, dk, dv = B.attend_backward(q, k, v, mask, 0.3, do)
    rows = np.array([0, 5, 17, 36])
    keys = np.array([0, 1, 26, 52])
    for mk in (mask, lambda r0, r1: mask[r0:r1]):
        sq, sk, sv = B.attend_backward_sampled(q, k, v, mk, 0.3, do, rows, keys, chunk=chunk)
        assert np.allclose(sq, dq[rows], rtol=1e-12, atol=1e-13)
        assert np.allclose(sk, dk[keys], rtol=1e-12, atol=1e-13)
        assert np.allclose(sv, dv[keys], rtol=1e-12, atol=1e-13)
