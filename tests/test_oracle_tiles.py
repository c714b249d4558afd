"""Pins for oracle.tiles: brute force on tiny masks and interval-based closed
forms on the workload shapes (CPU only)."""

import numpy as np
import pytest

from oracle import masks as M
from oracle import tiles as T


def _brute(mask, bq, bk):
    nq, nk = mask.shape
    nqt, nkt = -(-nq // bq), -(-nk // bk)
    cls = np.zeros((nqt, nkt), np.uint8)
    words = np.zeros((nqt, nkt, bq, bk // 64), np.uint64)
    for a in range(nqt):
        for c in range(nkt):
            ones = area = 0
            for r in range(bq):
                for x in range(bk):
                    t, j = a * bq + r, c * bk + x
                    if t < nq and j < nk:
                        area += 1
                        ones += int(mask[t, j])
            cls[a, c] = T.FULL if ones == area else (T.SKIP if ones == 0 else T.PARTIAL)
            if cls[a, c] == T.PARTIAL:
                for r in range(bq):
                    for x in range(bk):
                        t, j = a * bq + r, c * bk + x
                        if t < nq and j < nk and mask[t, j]:
                            words[a, c, r, x // 64] |= np.uint64(1) << np.uint64(x % 64)
    return cls, words


@pytest.mark.parametrize("nq,nk,bq,bk", [(19, 150, 8, 64), (64, 64, 16, 64), (5, 200, 4, 128)])
def test_classify_brute_force(nq, nk, bq, bk):
    rng = np.random.default_rng(nq * nk)
    for mask in (rng.random((nq, nk)) < 0.5, M.causal(nq, nk), M.sliding_window(nq, nk, 70),
                 np.ones((nq, nk), bool), np.zeros((nq, nk), bool)):
        c1, w1 = T.classify(mask, bq, bk)
        c2, w2 = _brute(mask, bq, bk)
        assert np.array_equal(c1, c2)
        assert np.array_equal(w1, w2)


def _interval_counts(n, bq, bk, lo_of, hi_of):
    """Per-tile classes when every row t sees the single key interval
    [lo_of(t), hi_of(t)), from the intersection and union of the tile's rows'
    intervals (square n x n mask)."""
    nqt, nkt = -(-n // bq), -(-n // bk)
    full = part = skip = 0
    for a in range(nqt):
        rows = range(a * bq, min(n, (a + 1) * bq))
        inter_lo = max(lo_of(t) for t in rows)
        inter_hi = min(hi_of(t) for t in rows)
        uni_lo = min(lo_of(t) for t in rows)
        uni_hi = max(hi_of(t) for t in rows)
        for c in range(nkt):
            k0, k1 = c * bk, min(n, (c + 1) * bk)
            if inter_lo <= k0 and k1 <= inter_hi:
                full += 1
            elif k1 <= uni_lo or k0 >= uni_hi:
                skip += 1
            else:
                part += 1
    return full, part, skip


def test_causal_window_counts_match_intervals():
    n = 1536
    for mask, lo, hi in ((M.causal(n, n), lambda t: 0, lambda t: t + 1),
                         (M.sliding_window(n, n, 384), lambda t: max(0, t - 383), lambda t: t + 1),
                         (M.prefix_lm(n, n, 300), lambda t: 0, lambda t: max(300, t + 1))):
        cls, _ = T.classify(mask, 128, 64)
        assert T.counts(cls) == _interval_counts(n, 128, 64, lo, hi)


def test_workload_shape_counts():
    """Tile counts at the full 16384-token shapes (tile 128 x 64), from the
    interval rule; the causal count also has the closed form FULL = 2 * sum(a)
    over q-tiles a, PARTIAL = 2 per q-tile."""
    n = 16384
    assert _interval_counts(n, 128, 64, lambda t: 0, lambda t: t + 1) == (16256, 256, 16256)
    assert 2 * sum(range(128)) == 16256
    assert _interval_counts(n, 128, 64, lambda t: max(0, t - 4095), lambda t: t + 1) == (6944, 448, 25376)


def test_partial_words_layout():
    mask = np.zeros((3, 130), bool)
    mask[0, [0, 63]] = True
    mask[2, [64, 129]] = True
    cls, words = T.classify(mask, 4, 128)
    assert cls.tolist() == [[T.PARTIAL, T.PARTIAL]]
    assert int(words[0, 0, 0, 0]) == (1 | (1 << 63))
    assert int(words[0, 0, 2, 1]) == 1
    assert int(words[0, 1, 2, 0]) == 2          # key 129 = tile 1, bit 1
    assert int(words[0, 0, 3, 0]) == 0          # out-of-bounds row
