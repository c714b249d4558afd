/*
 * maskattn — masked flash-attention prefill (and its backward), speculative
 * tree verify and masked decode over ragged sequences with paged K/V, for AMD
 * Instinct MI355X (gfx950).
 *
 * C ABI of libmaskattn.so.  Plain pointers and sizes only.  "host" and
 * "device" below say where a pointer must point.  Streams are hipStream_t
 * passed as void* (NULL = the default stream).
 *
 * Sources of the operations (web pages; sections named, not quoted):
 *  - sglang-jax pull request 20, "feat: support custom mask for flash
 *    attention": ragged paged attention with a `causal` flag or a flattened
 *    custom mask; the reference implementation rejects a custom mask together
 *    with causal; the custom mask must be at least as large as the sequences
 *    it covers; a sliding window only makes sense with causal masking
 *    (review comments).
 *  - aphrodite-engine issue 1526, "[Attention] feat: support PrefixLM":
 *    prefixlm_mask_mod, bidirectional inside a per-sequence prefix, causal
 *    after it (highlights).
 *  - flashinfer issue 724, "Custom mask slows down attention.": a float mask
 *    bit-packed before the kernel, the block-sparse alternative, tree
 *    attention for speculative decoding as a custom mask, and the question
 *    whether a sliding window and a custom mask can be used jointly.
 *  - MagiAttention issue 316, "Feature request: chunk-causal mask type for
 *    Flex Flash Attention": (q_range, k_range, attn_type) lists with types
 *    FULL, CAUSAL, INV_CAUSAL, BI_CAUSAL and the proposed CHUNK_CAUSAL with a
 *    per-range chunk size ("Proposed API", "Semantically equivalent to").
 *  - mlxcel pull request 555, "feat: add Gemma2 sliding-window (local/global)
 *    attention": the window ANDed into the causal mask.
 *
 * Semantics shared by every entry point
 *  - Sequence b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and
 *    keys 0 .. kv_len[b]-1.  Query row t of the sequence sits at key position
 *    pos(t) = t + kv_len - q_len (the queries are the sequence's last q_len
 *    tokens).
 *  - Query head h reads K/V head h / (Hq / Hkv) (contiguous GQA groups).
 *  - O[t] = sum_j P[t,j] V[j] with P = softmax over the visible keys of
 *    scale * Q[t].K[j]; a row with no visible key gives O = 0 and
 *    LSE = -inf.  LSE is the natural-log sum of exp over visible keys of the
 *    scaled scores.
 *  - Mask kinds:
 *      CAUSAL          j <= pos(t)
 *      SLIDING_WINDOW  pos(t) - window < j <= pos(t)
 *      PREFIX_LM       j <= pos(t) or j < prefix_len[b]
 *      RANGES          union of the sequence's range descriptors (below)
 *      DENSE_BOOL      uint8 per (t, j), nonzero = visible; per sequence a
 *                      row-major q_len x kv_len block, sequences concatenated
 *      PACKED_U64      per query row ceil(kv_len/64) uint64 words; key j is
 *                      bit (j % 64) of word j / 64; rows concatenated over
 *                      sequences; bits past kv_len are ignored
 *      BLOCK_SPARSE    block (t / block_r, j / block_c) is listed in the
 *                      sequence's block-row CSR (below)
 *    DENSE_BOOL, PACKED_U64 and BLOCK_SPARSE accept window >= 1: the mask is
 *    then intersected with the sliding-window band pos(t) - window < j <= pos(t).
 *  - Range descriptors are in per-sequence local coordinates (query rows and
 *    keys of that sequence).  Inside a range, i = t - q_start,
 *    jj = j - k_start, Lq = q_end - q_start, Lk = k_end - k_start:
 *      FULL          every (i, jj)
 *      CAUSAL        jj <= i + Lk - Lq            (bottom-right aligned)
 *      INV_CAUSAL    jj >= i
 *      BI_CAUSAL     i <= jj <= i + Lk - Lq
 *      CHUNK_CAUSAL  jj < Lk - (Lq - min(Lq, (i / cs + 1) * cs)), cs = chunk_size
 *
 * Errors: every function returns a status; nothing else crosses the ABI.
 * Arguments are validated on the host before any HIP call.  ma_last_error()
 * returns a thread-local message describing the last failure.
 */
#ifndef MASKATTN_H
#define MASKATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MA_OK = 0,
  MA_ERR_INVALID = -1,       /* a bad argument (null pointer, bad size, range outside the sequence) */
  MA_ERR_CONFLICT = -2,      /* arguments that cannot be used together */
  MA_ERR_SIZE = -3,          /* a mask buffer smaller than its sequences need, or a short workspace */
  MA_ERR_UNSUPPORTED = -4,   /* a head_dim, dtype, tile shape or page size with no kernel */
  MA_ERR_PLAN_MISMATCH = -5, /* plan built for other lengths / tile shape than the call */
  MA_ERR_HIP = -6,           /* a HIP runtime call failed (message has the HIP error) */
  MA_ERR_NOMEM = -7          /* host or device allocation failed */
} ma_status;

/* Range types; 0..3 keep the numbering of MagiAttention's attn_type_map. */
typedef enum {
  MA_RANGE_FULL = 0,
  MA_RANGE_CAUSAL = 1,
  MA_RANGE_INV_CAUSAL = 2,
  MA_RANGE_BI_CAUSAL = 3,
  MA_RANGE_CHUNK_CAUSAL = 4
} ma_range_type;

typedef enum {
  MA_KIND_CAUSAL = 0,
  MA_KIND_SLIDING_WINDOW = 1,
  MA_KIND_PREFIX_LM = 2,
  MA_KIND_RANGES = 3,
  MA_KIND_DENSE_BOOL = 4,
  MA_KIND_PACKED_U64 = 5,
  MA_KIND_BLOCK_SPARSE = 6
} ma_mask_kind;

typedef enum { MA_F32 = 0, MA_BF16 = 1 } ma_dtype;

/* Tile classes stored in a plan. */
typedef enum { MA_TILE_SKIP = 0, MA_TILE_FULL = 1, MA_TILE_PARTIAL = 2 } ma_tile_class;

typedef struct {
  int32_t q_start, q_end; /* query rows [q_start, q_end) of the sequence */
  int32_t k_start, k_end; /* keys [k_start, k_end) */
  int32_t type;           /* ma_range_type */
  int32_t chunk_size;     /* CHUNK_CAUSAL only, >= 1 */
} ma_range;

/* A mask description for mask_compile.  All arrays not marked otherwise are
 * host memory and are only read during the call. */
typedef struct {
  int32_t kind;                 /* ma_mask_kind */
  int32_t batch;                /* number of sequences, >= 1 */
  const int32_t *cu_seqlens_q;  /* host [batch+1], nondecreasing, starts at 0 */
  const int32_t *kv_lens;       /* host [batch], kv_len >= q_len of the sequence */
  int32_t window;               /* SLIDING_WINDOW: >= 1; DENSE_BOOL / PACKED_U64 / BLOCK_SPARSE:
                                   0 or a window >= 1 intersected with the mask; others: 0 */
  const int32_t *prefix_len;    /* PREFIX_LM: host [batch], 0 <= prefix_len <= kv_len */
  const ma_range *ranges;       /* RANGES: host, range_indptr[batch] descriptors */
  const int32_t *range_indptr;  /* RANGES: host [batch+1] CSR offsets into ranges */
  const void *mask;             /* DENSE_BOOL (uint8) or PACKED_U64 (uint64) */
  int64_t mask_numel;           /* elements in `mask`; must cover every sequence exactly or more */
  int32_t mask_on_device;       /* 1: `mask` is device memory (classified on the GPU, stream-ordered) */
  int32_t tile_q;               /* 64 or 128: query rows per tile */
  int32_t tile_k;               /* 64: keys per tile */
  /* BLOCK_SPARSE: blocks of block_r query rows x block_c keys.  Sequence b
   * has nrb_b = ceil(q_len_b / block_r) block rows; the block rows of all
   * sequences are concatenated (sequence 0 first) into one CSR:
   * bsr_indptr (host, [sum_b nrb_b + 1], starts at 0, nondecreasing) and
   * bsr_indices (host, block-column indices local to the sequence, each in
   * [0, ceil(kv_len_b / block_c)); repeats allowed). */
  int32_t block_r, block_c;
  const int32_t *bsr_indptr;
  const int32_t *bsr_indices;
} ma_mask_desc;

/* A compiled plan: per (sequence, q-tile, k-tile) FULL/SKIP/PARTIAL, the
 * packed words of PARTIAL tiles, and the q-tiles in execution order (most
 * non-SKIP tiles first).  Opaque; owned by the library. */
typedef struct ma_plan ma_plan;

typedef struct {
  int32_t batch, tile_q, tile_k;
  int32_t num_qtiles;      /* q-tile rows over all sequences */
  int64_t num_tiles;       /* sum over sequences of q-tiles x k-tiles */
  int64_t num_entries;     /* non-SKIP tiles (an upper bound for device-built plans) */
  int64_t num_word_blocks; /* PARTIAL word blocks held (tile_q rows each) */
  int64_t total_q;         /* cu_seqlens_q[batch] */
  int64_t device_bytes;    /* size of the plan's device buffer (0 before upload) */
  int32_t on_device;       /* 1 when the device buffer is populated */
  int32_t host_valid;      /* 1 when a host copy exists (host-compiled plans) */
} ma_plan_info;

/* Compile a mask into a plan and make it resident on the device (one
 * stream-ordered upload, or a device classification pass for a device-resident
 * DENSE_BOOL / PACKED_U64 mask).  The mask forms are those of the pages: the
 * kernel's causal flag or flattened custom mask (sglang-jax pull request 20,
 * the custom-mask argument of the ragged paged attention kernel), the
 * per-sequence prefix (aphrodite-engine issue 1526, prefixlm_mask_mod), a
 * bit-packed mask or a block-sparse one (flashinfer issue 724, issue body and
 * the maintainer's reply), (q_range, k_range, type, chunk_size) lists
 * (MagiAttention issue 316, "Proposed API") and the sliding window ANDed into
 * the causal mask (mlxcel pull request 555, description).  Each tile of
 * tile_q x tile_k entries is FULL, SKIP or PARTIAL over its in-bounds entries
 * and only PARTIAL tiles carry words, which is how the kernels avoid reading
 * the mask per element (flashinfer issue 724: the non-coalesced mask reads it
 * blames for the slowdown).  A host-compiled plan depends on the mask only:
 * equal masks give byte-identical plans whatever descriptors described them.
 * A device-classified plan has the same tile classes and words (export) but
 * its own execution order, so its serialisation may differ from a host
 * plan's.
 * Errors: INVALID / CONFLICT (window given with another kind; a custom mask
 * combined with causal is expressed by choosing one kind) / SIZE (mask_numel
 * short of sum q_len*kv_len, or of sum q_len*ceil(kv_len/64) words) /
 * UNSUPPORTED (tile shape) / HIP / NOMEM.  *out is set only on MA_OK. */
ma_status mask_compile(const ma_mask_desc *desc, void *stream, ma_plan **out);

/* Host-only compile (no HIP call): descriptors or a host-resident mask.
 * Used to inspect plans without a GPU; attn_prefill_masked uploads such a
 * plan on first use. */
ma_status mask_compile_host(const ma_mask_desc *desc, ma_plan **out);

/* Upload a host-compiled plan (no-op when already on the device). */
ma_status mask_plan_upload(ma_plan *plan, void *stream);

ma_status mask_plan_destroy(ma_plan *plan);

ma_status mask_plan_info_get(const ma_plan *plan, ma_plan_info *out);

/* Dense export for tests: classes[num_tiles] (ma_tile_class, tiles of
 * sequence 0 first, q-tile major, k-tile minor) and, if words != NULL,
 * words[num_tiles * tile_q * tile_k/64] holding each PARTIAL tile's rows
 * (zero for other tiles).  Reads the device copy when there is no host copy
 * (synchronises the device). */
ma_status mask_plan_export(const ma_plan *plan, uint8_t *classes, uint64_t *words);

/* Canonical serialisation of the plan (execution order, tile lists and
 * words), for byte-identity checks.  Call with dst = NULL to get *bytes. */
ma_status mask_plan_serialize(const ma_plan *plan, void *dst, size_t *bytes);

/* Masked prefill over a compiled plan: ragged query sequences against paged
 * K/V under a mask (sglang-jax pull request 20, ragged paged attention with a
 * custom mask; flashinfer issue 724, the custom-mask prefill whose speed the
 * issue measures against the causal kernel).  SKIP tiles are never visited,
 * FULL tiles take no mask work, PARTIAL tiles mask each score with their
 * row's word.
 *  q        device [total_q, Hq, d], in_dtype, contiguous
 *  k_cache, v_cache  device paged caches of in_dtype; element (page, slot,
 *           head, x) at page*kv_strides[0] + slot*kv_strides[1] +
 *           head*kv_strides[2] + x (strides in elements, x contiguous)
 *  page_table device int32 [batch, max_pages]; entry (b, i) is the physical
 *           page of keys i*page_size .. (i+1)*page_size-1 of sequence b.  Only
 *           entries for keys < kv_len are read.
 *  page_size power of two >= 1
 *  out      device [total_q, Hq, d] of out_dtype; lse device fp32 [total_q,
 *           Hq] or NULL
 *  scale    positive, finite (the softmax temperature, usually 1/sqrt(d))
 * Supported: in_dtype BF16 with d in {64, 128, 256} and out_dtype BF16 or F32;
 * in_dtype F32 with d in {64, 128} and out_dtype F32.  Arithmetic: fp32
 * accumulation; bf16 inputs use bf16 matrix products, fp32 inputs fp32 ones.
 * Launches are stream-ordered; the call does not synchronise.  Results are
 * deterministic (no atomics touch accumulators).  A plan with no query rows
 * (total_q 0) launches nothing; q and out may then be NULL. */
ma_status attn_prefill_masked(const ma_plan *plan, const void *q, int64_t total_q, int32_t hq,
                              const void *k_cache, const void *v_cache, int32_t hkv, int32_t d,
                              int32_t page_size, const int64_t kv_strides[3],
                              const int32_t *page_table, int32_t max_pages, int32_t in_dtype,
                              int32_t out_dtype, float scale, void *out, float *lse, void *stream);

/* Masked prefill with fp8 inputs (OCP e4m3: 1 sign, 4 exponent bits with
 * bias 7, 3 mantissa bits, subnormals, no infinities, 0x7F / 0xFF NaN;
 * largest 448) — the fp8 path asked about in flashinfer issue 724 (closing
 * questions).  q, k_cache, v_cache hold e4m3 bytes in the layouts of
 * attn_prefill_masked (strides in elements = bytes).  Per-tensor descale
 * factors: the attention is softmax(scale * q_descale * k_descale * Q8 K8^T
 * + mask) (v_descale * V8), Q8 / K8 / V8 the decoded bytes.
 *  out_dtype BF16 or F32; d in {64, 128, 256}; plans with tile 128 x 64; page
 *  size at least 1024 / d keys (one gather instruction's rows in one page);
 *  a page's bytes (page stride) below 2^32 and page_size * slot stride below
 *  2^31.
 * Arithmetic: both products on fp8 matrix cores with fp32 accumulation; the
 * probabilities are rounded to e4m3 (round to nearest even) for P V and the
 * row sums add those rounded values.  Deterministic; stream-ordered.
 * Errors as attn_prefill_masked, plus INVALID for descale factors that are
 * not positive and finite, UNSUPPORTED for small or too large pages. */
ma_status attn_prefill_masked_fp8(const ma_plan *plan, const void *q, int64_t total_q, int32_t hq,
                                  const void *k_cache, const void *v_cache, int32_t hkv, int32_t d,
                                  int32_t page_size, const int64_t kv_strides[3], const int32_t *page_table,
                                  int32_t max_pages, float q_descale, float k_descale, float v_descale,
                                  int32_t out_dtype, float scale, void *out, float *lse, void *stream);

/* Workspace bytes attn_backward_masked needs for this plan and Hq (two fp32
 * values per (query, head)); 0 for a NULL plan or hq < 1. */
size_t attn_backward_workspace(const ma_plan *plan, int32_t hq);

/* Gradients of masked prefill over the same plan (the training-side cost of
 * masks made of many small ranges is the motivation of the feature request
 * "chunk-causal mask type for Flex Flash Attention", MagiAttention issue 316,
 * problem statement).  With P = exp(scale Q K^T - LSE) on visible entries:
 * D = rowsum(dO * O), dS = P (dO V^T - D), dQ = scale dS K, dK = scale dS^T Q,
 * dV = P^T dO; a K/V head sums its GQA group's query heads.
 *  q, k_cache, v_cache, page_table, page_size, kv_strides, max_pages: as for
 *           attn_prefill_masked (bf16 inputs)
 *  out      device [total_q, Hq, d] of out_dtype (BF16 or F32): the forward's
 *           output;  lse  device fp32 [total_q, Hq]: the forward's LSE (-inf
 *           for a row with no visible key)
 *  dout     device bf16 [total_q, Hq, d], contiguous
 *  dq       device fp32 [total_q, Hq, d]: every element written (0 for rows
 *           with no visible key)
 *  dk_cache, dv_cache  device fp32 caches with the element strides of
 *           k_cache: the slot of every key below kv_len is written once (0
 *           when no query sees the key); other slots are not touched.  No two
 *           sequences may map keys to the same slot.
 *  workspace device, >= attn_backward_workspace(plan, hq) bytes, scratch.
 * With no query rows (total_q 0) q, out, dout, lse, dq and the workspace may
 * be NULL; dK and dV are still written (zeros) for every key below kv_len.
 * Supported: d in {64, 128, 256}; plans with tile_k 64 and tile_q 64 or 128.
 * The first call on a plan builds its key-major transpose (one device
 * allocation, held until mask_plan_destroy; synchronises `stream` once);
 * later calls only launch.  Arithmetic: bf16 matrix products (P and dS
 * rounded to bf16 for theirs) with fp32 accumulation.  Deterministic: no
 * atomics; each gradient element is summed by one workgroup in a fixed order.
 * Errors: INVALID (NULL arguments, bad shapes), SIZE (workspace too small),
 * PLAN_MISMATCH (total_q or tiles), UNSUPPORTED (d, dtype), NOMEM / HIP. */
ma_status attn_backward_masked(ma_plan *plan, const void *q, int64_t total_q, int32_t hq, const void *k_cache,
                               const void *v_cache, int32_t hkv, int32_t d, int32_t page_size,
                               const int64_t kv_strides[3], const int32_t *page_table, int32_t max_pages,
                               const void *out, int32_t out_dtype, const void *dout, const float *lse,
                               float scale, float *dq, float *dk_cache, float *dv_cache, void *workspace,
                               size_t ws_bytes, void *stream);

/* Workspace bytes attn_verify_tree needs for these bounds. */
size_t attn_verify_tree_workspace(int32_t batch, int32_t max_q, int32_t max_kv, int32_t hq,
                                  int32_t hkv, int32_t d);

/* Speculative tree verify: every sequence's draft-tree queries (q_len <= 64
 * per sequence) against its cached context plus the draft tokens, under a
 * full-row custom mask (DENSE_BOOL or PACKED_U64, device memory, rows over
 * all kv_len keys) — tree attention for speculative decoding expressed as a
 * custom mask (flashinfer issue 724, the maintainer's reply; the TARGET_VERIFY
 * mode of sglang-jax pull request 20).  Lengths stay on the device (no host
 * round trip):
 *  cu_seqlens_q device int32 [batch+1], kv_lens device int32 [batch];
 *  max_q >= every q_len (<= 64), max_kv >= every kv_len (host bounds used for
 *  the launch shape and the workspace).  The host cannot check these bounds
 *  against the device lengths: a sequence with more than max_q queries has
 *  only its first max_q rows computed (its other rows of out and lse are not
 *  written), keys at or past max_kv are not visited, and nothing outside the
 *  launch's workspace, splits or buffers is read or written.
 * The GQA group of a K/V head is processed together (the group's query heads
 * share each K/V tile) and long contexts are split over several workgroups
 * whose partial results are merged in a fixed order.  Requires in_dtype BF16
 * and d in {64, 128, 256}.  workspace: device, at least
 * attn_verify_tree_workspace(...) bytes (NULL allowed
 * when that is 0), owned by the caller; its contents need no initialisation.
 * Mask size: the layout of the mask kinds above (rows of kv_len bytes, or of
 * ceil(kv_len / 64) words, per query, sequences concatenated).  Because the
 * lengths are device-resident, the host checks only that mask_numel covers
 * one element per query row (MA_ERR_SIZE otherwise); any element at or past
 * mask_numel reads as 0, i.e. its key is masked, and nothing past the
 * buffer is read. */
ma_status attn_verify_tree(const void *q, int64_t total_q, int32_t hq, const void *k_cache,
                           const void *v_cache, int32_t hkv, int32_t d, int32_t page_size,
                           const int64_t kv_strides[3], const int32_t *page_table,
                           int32_t max_pages, const int32_t *cu_seqlens_q, const int32_t *kv_lens,
                           int32_t batch, int32_t max_q, int32_t max_kv, int32_t mask_kind,
                           const void *mask, int64_t mask_numel, int32_t in_dtype,
                           int32_t out_dtype, float scale, void *workspace, size_t ws_bytes,
                           void *out, float *lse, void *stream);

/* attn_verify_tree without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The scratch it needs lives in the
 * library: one 64 MiB device array per GPU, held until the process ends
 * (its address is looked up once per device on the first call there).
 * Arguments, results and errors are those of attn_verify_tree; bounds whose
 * attn_verify_tree_workspace exceeds 64 MiB are MA_ERR_SIZE.  The call
 * allocates nothing (no hipMalloc, no hipFree) and needs no cleared memory:
 * every scratch byte a launch reads it has written first.  All calls on one
 * GPU share its scratch, so calls that can overlap on one GPU (on different
 * streams without ordering between them) race; order them, e.g. on one
 * stream. */
ma_status attn_verify_tree_noalloc(const void *q, int64_t total_q, int32_t hq, const void *k_cache,
                                   const void *v_cache, int32_t hkv, int32_t d, int32_t page_size,
                                   const int64_t kv_strides[3], const int32_t *page_table, int32_t max_pages,
                                   const int32_t *cu_seqlens_q, const int32_t *kv_lens, int32_t batch,
                                   int32_t max_q, int32_t max_kv, int32_t mask_kind, const void *mask,
                                   int64_t mask_numel, int32_t in_dtype, int32_t out_dtype, float scale, void *out,
                                   float *lse, void *stream);

/* Workspace bytes attn_decode needs for these bounds (the same bound serves
 * every mask kind; 0 when one split covers every context). */
size_t attn_decode_workspace(int32_t batch, int32_t max_q, int32_t max_kv, int32_t hq, int32_t hkv,
                             int32_t d);

/* Masked decode (sglang-jax pull request 20, review comments: custom-mask
 * tests for prefill and decode modes; mlxcel pull request 555: the sliding
 * window in single and ragged decode graphs): each sequence's last q_len
 * (1 .. 64, ragged) tokens against
 * its paged K/V, query row t at position pos = t + kv_len - q_len, under
 *  mask_kind CAUSAL         keys <= pos,
 *            SLIDING_WINDOW pos - window < key <= pos (window >= 1),
 *            PREFIX_LM      keys <= pos or key < prefix_len[b] (device
 *                           int32 [batch]),
 *            DENSE_BOOL / PACKED_U64  rows as for attn_verify_tree;
 * the same definitions as the prefill masks of the same kinds (RANGES:
 * pass the rows, MA_ERR_UNSUPPORTED otherwise).  Lengths stay on the device
 * as for attn_verify_tree, with the same max_q / max_kv bounds; a sequence
 * with more than max_q queries is outside the contract: only its first
 * max_q rows are written (positioned as if it had max_q queries) and nothing
 * outside the buffers is read or written.  The query heads of a K/V head's GQA group and
 * their queries share each gathered K/V tile; long contexts are split over
 * workgroups and merged in a fixed order; a sliding window only walks the
 * tiles it can see.  Under CAUSAL, PREFIX_LM, DENSE_BOOL and PACKED_U64, a
 * launch whose rows per unit (GQA heads x max_q) exceed 128 at d <= 128 runs
 * attn_verify_tree's balanced kernel, the positional kinds' row words
 * computed from pos (outputs bit-identical to the same mask given as
 * packed rows).  A row that sees no key gets O = 0 and LSE = -inf.
 * Requires in_dtype BF16 and d in {64, 128, 256}.  workspace: device, at
 * least attn_decode_workspace(...) bytes (NULL allowed when that is 0), owned
 * by the caller; its contents need no initialisation.  DENSE_BOOL /
 * PACKED_U64 masks follow attn_verify_tree's size rule (one element per
 * query row checked on the host, elements past mask_numel read as 0). */
ma_status attn_decode(const void *q, int64_t total_q, int32_t hq, const void *k_cache,
                      const void *v_cache, int32_t hkv, int32_t d, int32_t page_size,
                      const int64_t kv_strides[3], const int32_t *page_table, int32_t max_pages,
                      const int32_t *cu_seqlens_q, const int32_t *kv_lens, int32_t batch,
                      int32_t max_q, int32_t max_kv, int32_t mask_kind, int32_t window,
                      const int32_t *prefix_len, const void *mask, int64_t mask_numel,
                      int32_t in_dtype, int32_t out_dtype, float scale, void *workspace,
                      size_t ws_bytes, void *out, float *lse, void *stream);

/* attn_decode over e4m3 (fp8) K/V caches (flashinfer issue 724, the
 * fp8 question after its benchmark table, for the decode side: the cache is
 * the bytes decode reads).  k_cache / v_cache hold OCP e4m3 bytes in the
 * layout of attn_decode (strides in elements = bytes); the attention is that
 * of attn_decode with K = k_descale * decode(K8) and V = v_descale *
 * decode(V8) and bf16 queries.  The kernel widens each gathered tile exactly
 * to bf16 in LDS and runs the bf16 products; the descale factors enter the
 * softmax constant and the normalisation, so the result equals attn_decode
 * on the exactly decoded caches (up to the same fp32 summation order).
 * Mask kinds, lengths, splits and workspace (attn_decode_workspace) as for
 * attn_decode.  Requires d in {64, 128, 256}, pages of at least 1024 / d
 * keys, page_size * slot stride below 2^31 and the page stride below 2^32
 * (bytes).  Errors as attn_decode, plus INVALID for descale factors that are
 * not positive and finite, UNSUPPORTED for small or too large pages. */
ma_status attn_decode_kv8(const void *q, int64_t total_q, int32_t hq, const void *k_cache,
                          const void *v_cache, int32_t hkv, int32_t d, int32_t page_size,
                          const int64_t kv_strides[3], const int32_t *page_table, int32_t max_pages,
                          const int32_t *cu_seqlens_q, const int32_t *kv_lens, int32_t batch,
                          int32_t max_q, int32_t max_kv, int32_t mask_kind, int32_t window,
                          const int32_t *prefix_len, const void *mask, int64_t mask_numel,
                          int32_t out_dtype, float scale, float k_descale, float v_descale,
                          void *workspace, size_t ws_bytes, void *out, float *lse, void *stream);

const char *ma_status_string(int32_t status);
const char *ma_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MASKATTN_H */
