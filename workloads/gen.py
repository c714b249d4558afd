"""Seeded synthetic workloads for masked prefill and tree verify.

Recipe (the same for tests, benchmark and oracle checks):
  * Generator: numpy PCG64(seed).  Structure is drawn first (lengths,
    prefix lengths, tree parents, Bernoulli mask bits, page permutation), then
    Q, K, V as float32 N(0, 1).  For bf16 workloads Q, K, V are rounded to
    bf16 (round to nearest even) and kept as the float32 values of those bf16
    numbers, so both sides read identical inputs.
  * Integer "uniform in [a, b]" is inclusive.
  * K/V live in a paged cache [num_pages, page_size, H_kv, d] (page size 16).
    Pages of a sequence are consecutive when the layout is contiguous and a
    random permutation of all pages otherwise.  Unused slots of the last page,
    two spare pages and every page-table entry past a sequence's last page
    hold / point at NaN, so a read past kv_len shows up in the output.
  * fp8 inputs (fp8_inputs): per-tensor descale = max |x| / 448 over the
    finite values of Q, of the K cache and of the V cache; each value x is
    stored as the e4m3 byte of x / descale, rounded to nearest even
    (torch's float8_e4m3fn conversion); NaN slots stay NaN bytes.
  * Mask buffers are laid out as the caller hands them over: a dense mask is
    one row-major q_len x kv_len uint8 block per sequence, concatenated; a
    packed mask is one row of ceil(kv_len / 64) uint64 words per query, key j
    in bit j % 64 of word j // 64, rows concatenated over sequences.
"""

from dataclasses import dataclass, field

import numpy as np

PAGE_SIZE = 16
# Range types as numbered in MagiAttention's attn_type_map, plus CHUNK_CAUSAL.
R_FULL, R_CAUSAL, R_INV_CAUSAL, R_BI_CAUSAL, R_CHUNK_CAUSAL = 0, 1, 2, 3, 4


@dataclass
class MaskInput:
    """One mask as handed to the library.

    kind: 'causal' | 'window' | 'prefix_lm' | 'ranges' | 'dense' | 'packed' |
          'block_sparse'
    window: the window of 'window', or one ANDed with 'dense' / 'packed' /
            'block_sparse' (0: none)
    """
    kind: str
    window: int = 0
    prefix_len: np.ndarray = None          # int32 [B]
    ranges: list = None                    # per sequence: list of 6-tuples
    data: np.ndarray = None                # dense uint8 flat / packed uint64 flat
    bsr: tuple = None                      # (block_r, block_c, indptr, indices), block rows of all sequences


@dataclass
class Workload:
    name: str
    dtype: str                   # 'f32' or 'bf16'
    hq: int
    hkv: int
    d: int
    scale: float
    page_size: int
    q: np.ndarray                # float32 [total_q, Hq, d]
    k_cache: np.ndarray          # float32 [num_pages, page_size, Hkv, d]
    v_cache: np.ndarray
    page_table: np.ndarray       # int32 [B, max_pages]
    cu_seqlens_q: np.ndarray     # int32 [B+1]
    kv_lens: np.ndarray          # int32 [B]
    masks: dict = field(default_factory=dict)
    info: dict = field(default_factory=dict)

    @property
    def batch(self):
        return len(self.kv_lens)

    @property
    def q_lens(self):
        return np.diff(self.cu_seqlens_q)


def rng_for(seed):
    return np.random.Generator(np.random.PCG64(seed))


def round_bf16(x):
    """float32 -> nearest bf16 (ties to even), returned as float32."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def pack_rows(dense):
    """bool [n, kv] -> uint64 [n, ceil(kv / 64)], key j in bit j % 64 of word
    j // 64."""
    dense = np.asarray(dense, dtype=bool)
    n, kv = dense.shape
    nw = (kv + 63) // 64
    pad = np.zeros((n, nw * 64), dtype=bool)
    pad[:, :kv] = dense
    by = np.packbits(pad, axis=1, bitorder="little")
    return np.ascontiguousarray(by).view("<u8").reshape(n, nw)


def _draw_permutation(rng, kv_lens, page_size, permute, spare=2):
    pages = [(int(k) + page_size - 1) // page_size for k in kv_lens]
    total = sum(pages) + spare
    perm = rng.permutation(total) if permute else np.arange(total)
    return pages, total, perm


def _layout(values_per_seq, kv_lens, hkv, d, page_size, pages, total, perm):
    """Scatter per-sequence [kv_len, Hkv, d] values into pages."""
    cache = np.full((total, page_size, hkv, d), np.nan, dtype=np.float32)
    max_pages = max(pages) if pages else 1
    spare_page = int(perm[total - 1])
    table = np.full((len(kv_lens), max_pages), spare_page, dtype=np.int32)
    off = 0
    for b, (vals, kl) in enumerate(zip(values_per_seq, kv_lens)):
        kl = int(kl)
        for i in range(pages[b]):
            p = int(perm[off + i])
            table[b, i] = p
            n = min(page_size, kl - i * page_size)
            cache[p, :n] = vals[i * page_size:i * page_size + n]
        off += pages[b]
    return cache, table


def _qkv(rng, total_q, kv_lens, hq, hkv, d, dtype):
    q = rng.standard_normal((total_q, hq, d), dtype=np.float32)
    total_kv = int(np.sum(kv_lens))
    k = rng.standard_normal((total_kv, hkv, d), dtype=np.float32)
    v = rng.standard_normal((total_kv, hkv, d), dtype=np.float32)
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    cuts = np.cumsum(np.asarray(kv_lens, dtype=np.int64))[:-1]
    return q, np.split(k, cuts), np.split(v, cuts)


def _build(name, rng, dtype, q_lens, kv_lens, hq, hkv, d, permute, scale=None):
    kv_lens = np.asarray(kv_lens, dtype=np.int32)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    pages, total, perm = _draw_permutation(rng, kv_lens, PAGE_SIZE, permute)
    cu = np.zeros(len(q_lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    q, ks, vs = _qkv(rng, int(cu[-1]), kv_lens, hq, hkv, d, dtype)
    kc, table = _layout(ks, kv_lens, hkv, d, PAGE_SIZE, pages, total, perm)
    vc, _ = _layout(vs, kv_lens, hkv, d, PAGE_SIZE, pages, total, perm)
    return Workload(name=name, dtype=dtype, hq=hq, hkv=hkv, d=d,
                    scale=float(scale if scale is not None else 1.0 / np.sqrt(d)),
                    page_size=PAGE_SIZE, q=q, k_cache=kc, v_cache=vc,
                    page_table=table, cu_seqlens_q=cu, kv_lens=kv_lens)


# ---------------------------------------------------------------- config 1 --
def config1(seed=1, n=128, d=64):
    """Single sequence, one head, q_len = kv_len = n, head_dim d, fp32 inputs,
    scale 1/sqrt(d).  Masks: causal, and a dense Bernoulli(0.5) custom mask
    with the diagonal forced true."""
    rng = rng_for(seed)
    bits = rng.random((n, n)) < 0.5
    bits[np.arange(n), np.arange(n)] = True
    w = _build("cfg1", rng, "f32", [n], [n], 1, 1, d, permute=False)
    w.masks["causal"] = MaskInput("causal")
    w.masks["custom"] = MaskInput("dense", data=bits.astype(np.uint8).reshape(-1))
    w.masks["custom_packed"] = MaskInput("packed", data=pack_rows(bits).reshape(-1))
    w.info["bits"] = bits
    return w


# ---------------------------------------------------------------- config 2 --
def tree_bits(ctx, parents):
    """Tree-verify mask rows for one sequence: node n sees keys [0, ctx) and
    the keys ctx + m of its ancestors m and itself.  Ancestor sets are built by
    the recursion anc[0] = {0}, anc[n] = anc[parent[n]] + {n}."""
    n = len(parents)
    anc = np.zeros((n, n), dtype=bool)
    anc[0, 0] = True
    for i in range(1, n):
        anc[i] = anc[int(parents[i])]
        anc[i, i] = True
    m = np.zeros((n, ctx + n), dtype=bool)
    m[:, :ctx] = True
    m[:, ctx:] = anc
    return m


def config2(seed=2, batch=8, nodes=64, ctx_lo=512, ctx_hi=4096, hq=32, hkv=8,
            d=128):
    """Speculative tree verify: per sequence a cached context of length
    U[ctx_lo, ctx_hi] plus a `nodes`-node draft tree (parent[n] uniform over
    0..n-1, node 0 the root) whose K/V already sit in the paged cache after
    the context.  GQA hq/hkv, bf16, random page permutation.  The mask is
    given as full dense rows and as packed rows; a causal comparator at the
    same shape is included."""
    rng = rng_for(seed)
    ctx = rng.integers(ctx_lo, ctx_hi + 1, size=batch)
    parents = [np.concatenate([[0], [rng.integers(0, i) for i in range(1, nodes)]]).astype(np.int32)
               for _ in range(batch)]
    kv = ctx + nodes
    w = _build("cfg2", rng, "bf16", [nodes] * batch, kv, hq, hkv, d, permute=True)
    rows = [tree_bits(int(c), p) for c, p in zip(ctx, parents)]
    w.masks["tree_dense"] = MaskInput("dense", data=np.concatenate([r.astype(np.uint8).reshape(-1) for r in rows]))
    w.masks["tree_packed"] = MaskInput("packed", data=np.concatenate([pack_rows(r).reshape(-1) for r in rows]))
    w.masks["causal"] = MaskInput("causal")
    w.info.update(ctx=ctx.astype(np.int32), parents=parents)
    return w


# --------------------------------------------------------------- config 3a --
def config3a(seed=31, batch=4, seq=4096, p_lo=256, p_hi=1024, hq=32, d=64):
    """PrefixLM over ragged paged KV: prefix_len uniform in [p_lo, p_hi] per
    sequence.  Given as the PREFIX_LM kind and as the range list
    {FULL [0,P) x [0,P), CAUSAL [0,seq) x [0,seq)}; causal comparator."""
    rng = rng_for(seed)
    plen = rng.integers(p_lo, p_hi + 1, size=batch).astype(np.int32)
    w = _build("cfg3a", rng, "bf16", [seq] * batch, [seq] * batch, hq, hq, d, permute=True)
    w.masks["prefix_lm"] = MaskInput("prefix_lm", prefix_len=plen)
    w.masks["prefix_lm_ranges"] = MaskInput("ranges", ranges=[
        [(0, int(p), 0, int(p), R_FULL, 0), (0, seq, 0, seq, R_CAUSAL, 0)] for p in plen])
    w.masks["causal"] = MaskInput("causal")
    w.info["prefix_len"] = plen
    return w


# --------------------------------------------------------------- config 3b --
def config3b(layer, seq=16384, window=4096, hq=8, hkv=4, d=256, seed=None):
    """Gemma2-like layer `layer` (seed 32 + layer): even layers use a sliding
    window of `window` keys, odd layers are global causal."""
    rng = rng_for(32 + layer if seed is None else seed)
    w = _build(f"cfg3b_l{layer}", rng, "bf16", [seq], [seq], hq, hkv, d, permute=True)
    if layer % 2 == 0:
        w.masks["window"] = MaskInput("window", window=window)
    w.masks["causal"] = MaskInput("causal")
    w.info.update(layer=layer, window=window)
    return w


# ---------------------------------------------------------------- config 4 --
def chunk_ranges(seq, prefix, cs):
    """One causal prefix range plus one CHUNK_CAUSAL range over the pairs."""
    return [(0, prefix, 0, prefix, R_CAUSAL, 0), (prefix, seq, 0, seq, R_CHUNK_CAUSAL, cs)]


def chunk_ranges_expanded(seq, prefix, cs):
    """The same mask written as one FULL range per chunk: chunk c covers rows
    [prefix + c*cs, prefix + (c+1)*cs) and keys [0, prefix + (c+1)*cs)."""
    out = [(0, prefix, 0, prefix, R_CAUSAL, 0)]
    start = prefix
    while start < seq:
        end = min(seq, start + cs)
        out.append((start, end, 0, end, R_FULL, 0))
        start = end
    return out


def config4(seed=4, seq=16384, prefix=1024, hq=16, d=128, chunk_sizes=(2, 4, 16)):
    """Chunk-causal interleaved (token, latent) pairs after a causal prefix,
    as one CHUNK_CAUSAL range and as its O(num_pairs) FULL expansion, for each
    chunk size; causal comparator.  Same Q/K/V for every variant."""
    rng = rng_for(seed)
    w = _build("cfg4", rng, "bf16", [seq], [seq], hq, hq, d, permute=False)
    for cs in chunk_sizes:
        w.masks[f"chunk{cs}"] = MaskInput("ranges", ranges=[chunk_ranges(seq, prefix, cs)])
        w.masks[f"chunk{cs}_full"] = MaskInput("ranges", ranges=[chunk_ranges_expanded(seq, prefix, cs)])
    w.masks["causal"] = MaskInput("causal")
    w.info.update(prefix=prefix, chunk_sizes=tuple(chunk_sizes))
    return w


# ---------------------------------------------------------------- config 5 --
def block_triangle_ranges(q_len, kv_len, dense_keys, blocks, block):
    """Every row sees keys [0, dense_keys); the last blocks*block rows form
    `blocks` blocks of `block` rows, block b adding a causal block x block
    triangle on keys [dense_keys + block*b, dense_keys + block*(b+1))."""
    first = q_len - blocks * block
    out = [(0, q_len, 0, dense_keys, R_FULL, 0)]
    for b in range(blocks):
        out.append((first + block * b, first + block * (b + 1),
                    dense_keys + block * b, dense_keys + block * (b + 1), R_CAUSAL, 0))
    return out


def block_triangle_packed(q_len, kv_len, dense_keys, blocks, block):
    """The same mask as packed rows, written directly."""
    first = q_len - blocks * block
    nw = (kv_len + 63) // 64
    w0 = dense_keys // 64                  # words that are all ones in every row
    out = np.zeros((q_len, nw), dtype=np.uint64)
    out[:, :w0] = np.uint64(0xFFFFFFFFFFFFFFFF)
    tail = np.zeros((q_len - first, kv_len - 64 * w0), dtype=bool)
    tail[:, :dense_keys - 64 * w0] = True
    tri = np.tril(np.ones((block, block), dtype=bool))
    for b in range(blocks):
        k0 = dense_keys - 64 * w0 + block * b
        tail[block * b:block * (b + 1), k0:k0 + block] = tri
    out[first:, w0:] = pack_rows(tail)
    if dense_keys > 64 * w0:
        head = np.zeros((1, kv_len - 64 * w0), dtype=bool)
        head[:, :dense_keys - 64 * w0] = True
        out[:first, w0:] = pack_rows(head)
    return out


def config5(seed=5, q_len=32768, kv_len=29576, dense_keys=24576, blocks=50, block=100,
            hq=32, hkv=8, d=128):
    """Large irregular custom mask (a dense block plus 50 small causal
    triangles), as a range list and as a packed matrix; causal comparator."""
    rng = rng_for(seed)
    w = _build("cfg5", rng, "bf16", [q_len], [kv_len], hq, hkv, d, permute=False)
    w.masks["custom_ranges"] = MaskInput("ranges", ranges=[
        block_triangle_ranges(q_len, kv_len, dense_keys, blocks, block)])
    w.masks["custom_packed"] = MaskInput("packed", data=block_triangle_packed(
        q_len, kv_len, dense_keys, blocks, block).reshape(-1))
    w.masks["causal"] = MaskInput("causal")
    w.info.update(dense_keys=dense_keys, blocks=blocks, block=block)
    return w


# ------------------------------------------------------------------- decode --
def decode(seed=6, batch=16, q_len=1, ctx_lo=4096, ctx_hi=16384, hq=32, hkv=8, d=128, window=4096):
    """Masked decode: per sequence the last q_len tokens against a paged
    context of U[ctx_lo, ctx_hi] keys (the query tokens' own K/V included),
    GQA hq/hkv, bf16, random page permutation.  Masks: causal, and a sliding
    window of `window` keys (a Gemma2-style local layer)."""
    rng = rng_for(seed)
    kv = rng.integers(ctx_lo, ctx_hi + 1, size=batch)
    w = _build("decode", rng, "bf16", [q_len] * batch, kv, hq, hkv, d, permute=True)
    w.masks["causal"] = MaskInput("causal")
    w.masks["window"] = MaskInput("window", window=window)
    return w


# ----------------------------------------------------------------- backward --
def upstream_grad(w, seed):
    """dO for a backward pass: N(0, 1) of q's shape, rounded to bf16 (kept as
    the float32 values of those bf16 numbers), drawn from PCG64(seed)."""
    g = rng_for(seed).standard_normal(w.q.shape, dtype=np.float32)
    return round_bf16(g)


def backward_small(seed=7, d=128, hq=4, hkv=2, q_lens=(300, 5, 130, 64, 1, 200),
                   kv_lens=(900, 70, 130, 1000, 1, 200)):
    """Ragged batch for backward parity: tails in every tile direction, a
    one-key sequence, q_len = kv_len and q_len << kv_len, GQA, bf16, random
    page permutation.  Masks: causal, a 37-key window, PrefixLM (prefix
    uniform in [0, kv_len]), a range list (a causal prefix of a third of the
    rows plus CHUNK_CAUSAL with chunk 16, and one INV_CAUSAL block), and a
    Bernoulli(0.3) custom mask with an empty row and a one-key row per
    sequence (q_len > 2), as dense bytes and as packed words."""
    rng = rng_for(seed)
    q_lens, kv_lens = list(q_lens), list(kv_lens)
    plen = np.array([rng.integers(0, k + 1) for k in kv_lens], np.int32)
    dense = []
    for q, k in zip(q_lens, kv_lens):
        m = rng.random((q, k)) < 0.3
        if q > 2:
            m[1, :] = False
            m[2, :] = False
            m[2, k - 1] = True
        dense.append(m)
    ranges = []
    for q, k in zip(q_lens, kv_lens):
        p = q // 3
        off = k - q
        rs = [(0, q, 0, off + p, R_CAUSAL, 0)] if p > 0 else []
        if q > p:
            rs.append((p, q, 0, k, R_CHUNK_CAUSAL, 16))
        if q >= 8 and k >= 8:
            rs.append((0, 8, k - 8, k, R_INV_CAUSAL, 0))
        ranges.append(rs)
    w = _build(f"bwd{seed}", rng, "bf16", q_lens, kv_lens, hq, hkv, d, permute=True)
    w.masks["causal"] = MaskInput("causal")
    w.masks["window"] = MaskInput("window", window=37)
    w.masks["prefix_lm"] = MaskInput("prefix_lm", prefix_len=plen)
    w.masks["ranges"] = MaskInput("ranges", ranges=ranges)
    w.masks["dense"] = MaskInput("dense", data=np.concatenate([m.astype(np.uint8).reshape(-1) for m in dense]))
    w.masks["packed"] = MaskInput("packed", data=np.concatenate([pack_rows(m).reshape(-1) for m in dense]))
    return w


# ---------------------------------------------------------- more mask inputs --
def block_sparse_csr(rng, q_lens, kv_lens, block_r, block_c, p):
    """Bernoulli(p) block structure per sequence (the first block row forced
    full), as one CSR over the block rows of all sequences (columns local to
    each sequence, in shuffled order).  Returns (indptr, indices)."""
    indptr, indices = [0], []
    for q, k in zip(q_lens, kv_lens):
        nrb, ncb = -(-int(q) // block_r), -(-int(k) // block_c)
        blocks = rng.random((nrb, ncb)) < p
        blocks[0, :] = True
        for rb in range(nrb):
            cols = list(np.flatnonzero(blocks[rb]))
            rng.shuffle(cols)
            indices += cols
            indptr.append(len(indices))
    return np.array(indptr, dtype=np.int32), np.array(indices, dtype=np.int32)


def mask_inputs(seed=9, d=128, hq=8, hkv=2, q_lens=(300, 5, 130, 700, 1), kv_lens=(900, 70, 130, 2000, 64)):
    """Ragged batch (bf16, GQA, random page order) for the block-sparse and
    window-intersected mask inputs: block-sparse masks at block sizes 64 x 64,
    128 x 128 and 16 x 48 (Bernoulli(0.35) blocks), the 64 x 64 one also with
    a 300-key window, and a Bernoulli(0.5) custom mask with a 111-key window
    (dense bytes and packed words) and without."""
    rng = rng_for(seed)
    q_lens, kv_lens = list(q_lens), list(kv_lens)
    bs = {}
    for br, bc in ((64, 64), (128, 128), (16, 48)):
        bs[(br, bc)] = block_sparse_csr(rng, q_lens, kv_lens, br, bc, 0.35)
    custom = [rng.random((q, k)) < 0.5 for q, k in zip(q_lens, kv_lens)]
    w = _build(f"maskin{seed}", rng, "bf16", q_lens, kv_lens, hq, hkv, d, permute=True)
    for (br, bc), (ip, ix) in bs.items():
        w.masks[f"bsr{br}x{bc}"] = MaskInput("block_sparse", bsr=(br, bc, ip, ix))
    ip, ix = bs[(64, 64)]
    w.masks["bsr64x64_window"] = MaskInput("block_sparse", bsr=(64, 64, ip, ix), window=300)
    flat = np.concatenate([m.astype(np.uint8).reshape(-1) for m in custom])
    packed = np.concatenate([pack_rows(m).reshape(-1) for m in custom])
    w.masks["dense"] = MaskInput("dense", data=flat)
    w.masks["dense_window"] = MaskInput("dense", data=flat, window=111)
    w.masks["packed_window"] = MaskInput("packed", data=packed, window=111)
    return w


# --------------------------------------------------------------------- fp8 --
def _e4m3_bytes(x, descale):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32) / np.float32(descale))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def fp8_inputs(w):
    """e4m3 bytes and per-tensor descale factors of a workload's Q, K cache
    and V cache: dict q8, k8, v8 (uint8, same shapes) and q_s, k_s, v_s."""
    out = {}
    for name, x in (("q", w.q), ("k", w.k_cache), ("v", w.v_cache)):
        amax = float(np.nanmax(np.abs(x)))
        ds = amax / 448.0 if amax > 0 else 1.0
        out[name + "8"] = _e4m3_bytes(x, ds)
        out[name + "_s"] = ds
    return out
