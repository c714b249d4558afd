"""Tile classification of a dense mask (oracle; test infrastructure only).

A plan cuts each sequence's [q_len, kv_len] mask into tiles of tile_q rows by
tile_k keys.  Tile (a, c) covers rows [a*tile_q, min(q_len, (a+1)*tile_q)) and
keys [c*tile_k, min(kv_len, (c+1)*tile_k)).  Counting in-bounds entries only,
it is FULL when every entry is visible, SKIP when none is and PARTIAL
otherwise.  A PARTIAL tile carries its mask as one row of tile_k // 64 u64
words per tile row: bit x of word w of row r is M[a*tile_q + r,
c*tile_k + 64*w + x] when that entry is in bounds and 0 when it is not.

This is the block mask that FlexAttention's build_block_mask derives from a
mask function ([aphrodite#1526]) and the block-sparse form [flashinfer#724]
recommends over a per-element custom mask, written out per tile.
"""

import numpy as np

SKIP, FULL, PARTIAL = 0, 1, 2


def classify(mask, tile_q, tile_k):
    """Returns (classes uint8 [nqt, nkt], words uint64 [nqt, nkt, tile_q,
    tile_k // 64]); words are zero for tiles that are not PARTIAL."""
    if tile_k % 64:
        raise ValueError("tile_k must be a multiple of 64")
    mask = np.asarray(mask, dtype=bool)
    nq, nk = mask.shape
    nqt = -(-nq // tile_q)
    nkt = -(-nk // tile_k)
    padded = np.zeros((nqt * tile_q, nkt * tile_k), dtype=bool)
    padded[:nq, :nk] = mask
    inb = np.zeros_like(padded)
    inb[:nq, :nk] = True
    blocks = padded.reshape(nqt, tile_q, nkt, tile_k).transpose(0, 2, 1, 3)
    inb_blocks = inb.reshape(nqt, tile_q, nkt, tile_k).transpose(0, 2, 1, 3)
    ones = blocks.sum(axis=(2, 3))
    area = inb_blocks.sum(axis=(2, 3))
    classes = np.full((nqt, nkt), PARTIAL, dtype=np.uint8)
    classes[ones == area] = FULL
    classes[ones == 0] = SKIP
    nw = tile_k // 64
    bits = blocks.reshape(nqt, nkt, tile_q, nw, 64).astype(np.uint64)
    weights = np.uint64(1) << np.arange(64, dtype=np.uint64)
    words = (bits * weights).sum(axis=-1, dtype=np.uint64)
    words[classes != PARTIAL] = 0
    return classes, words


def counts(classes):
    """(FULL, PARTIAL, SKIP) tile counts."""
    c = np.asarray(classes)
    return int((c == FULL).sum()), int((c == PARTIAL).sum()), int((c == SKIP).sum())
