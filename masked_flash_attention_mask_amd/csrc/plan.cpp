// Host mask compiler: mask descriptions -> per-(q-tile, k-tile) FULL / SKIP /
// PARTIAL plan with packed words for PARTIAL tiles.
//
// The compiler never materialises a dense mask for the closed-form kinds.
// Every query row's visible keys are a short sorted list of disjoint
// intervals (one interval for causal, window and PrefixLM; the merged union
// of the covering descriptors for range lists).  Per q-tile, visible-key
// counts per k-tile come from a difference array over the row intervals, so a
// tile is classified from its count against its in-bounds area, and only
// PARTIAL tiles are rasterised into words.  The result depends on the mask
// alone, so equivalent descriptor lists (one CHUNK_CAUSAL range, or its
// O(num_pairs) FULL expansion as in MagiAttention issue 316) give
// byte-identical plans.
#include <hip/hip_runtime.h>

#include <mutex>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <numeric>

#include "internal.h"

namespace maskattn {

namespace {
thread_local std::string g_last_error;

struct Iv {
  int32_t lo, hi;  // keys [lo, hi)
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Visible keys of row i (local) inside one range descriptor, as an interval
// relative to the range's k_start; empty when hi <= lo.
Iv range_row_interval(const ma_range &r, int32_t i) {
  const int32_t lq = r.q_end - r.q_start, lk = r.k_end - r.k_start;
  int64_t lo = 0, hi = lk;
  switch (r.type) {
    case MA_RANGE_FULL:
      break;
    case MA_RANGE_CAUSAL:
      hi = std::min<int64_t>(lk, (int64_t)i + lk - lq + 1);
      break;
    case MA_RANGE_INV_CAUSAL:
      lo = i;
      break;
    case MA_RANGE_BI_CAUSAL:
      lo = i;
      hi = std::min<int64_t>(lk, (int64_t)i + lk - lq + 1);
      break;
    case MA_RANGE_CHUNK_CAUSAL: {
      const int64_t cs = r.chunk_size;
      const int64_t chunk_end = std::min<int64_t>(lq, ((int64_t)i / cs + 1) * cs);
      hi = (int64_t)lk - (lq - chunk_end);
      break;
    }
    default:
      hi = 0;
  }
  lo = std::max<int64_t>(lo, 0);
  hi = std::min<int64_t>(hi, lk);
  if (hi < lo) hi = lo;
  return Iv{(int32_t)(r.k_start + lo), (int32_t)(r.k_start + hi)};
}

// Per-row interval lists of one sequence (CSR), merged and sorted.
struct RowIntervals {
  std::vector<int32_t> ptr;
  std::vector<Iv> iv;
};

// Intersects every row's intervals with the sliding-window band
// pos - window < j <= pos (a window given with a BLOCK_SPARSE mask).
void clip_to_window(RowIntervals &R, int32_t q_len, int32_t kv_len, int32_t window) {
  const int64_t delta = (int64_t)kv_len - q_len;
  std::vector<Iv> iv;
  std::vector<int32_t> ptr(q_len + 1, 0);
  iv.reserve(R.iv.size());
  for (int32_t t = 0; t < q_len; ++t) {
    const int64_t pos = t + delta;
    const int64_t lo = pos - window + 1, hi = pos + 1;
    for (int32_t k = R.ptr[t]; k < R.ptr[t + 1]; ++k) {
      const int64_t a = std::max<int64_t>(lo, R.iv[k].lo), z = std::min<int64_t>(hi, R.iv[k].hi);
      if (z > a) iv.push_back(Iv{(int32_t)a, (int32_t)z});
    }
    ptr[t + 1] = (int32_t)iv.size();
  }
  R.iv.swap(iv);
  R.ptr.swap(ptr);
}

// First block row of sequence b in the concatenated block-row CSR.
int64_t bsr_row_base(const ma_mask_desc *d, int b) {
  int64_t base = 0;
  for (int s = 0; s < b; ++s)
    base += ceil_div((int64_t)d->cu_seqlens_q[s + 1] - d->cu_seqlens_q[s], d->block_r);
  return base;
}

void build_rows(const ma_mask_desc *d, int b, int32_t q_len, int32_t kv_len, RowIntervals &out) {
  out.ptr.assign(q_len + 1, 0);
  out.iv.clear();
  const int64_t delta = (int64_t)kv_len - q_len;
  if (d->kind == MA_KIND_BLOCK_SPARSE) {
    // Row t sees the listed blocks of its block row; adjacent or repeated
    // blocks merge.  One sorted column list per block row.
    const int64_t rb0 = bsr_row_base(d, b);
    const int32_t nrb = (int32_t)ceil_div(q_len, d->block_r);
    std::vector<Iv> blocks;
    for (int32_t rb = 0; rb < nrb; ++rb) {
      const int32_t k0 = d->bsr_indptr[rb0 + rb], k1 = d->bsr_indptr[rb0 + rb + 1];
      std::vector<int32_t> cols(d->bsr_indices + k0, d->bsr_indices + k1);
      std::sort(cols.begin(), cols.end());
      blocks.clear();
      for (int32_t c : cols) {
        const int32_t lo = (int32_t)std::min<int64_t>(kv_len, (int64_t)c * d->block_c);
        const int32_t hi = (int32_t)std::min<int64_t>(kv_len, (int64_t)(c + 1) * d->block_c);
        if (hi <= lo) continue;
        if (!blocks.empty() && blocks.back().hi >= lo)
          blocks.back().hi = std::max(blocks.back().hi, hi);
        else
          blocks.push_back(Iv{lo, hi});
      }
      const int32_t t1 = std::min<int32_t>(q_len, (rb + 1) * d->block_r);
      for (int32_t t = rb * d->block_r; t < t1; ++t) {
        out.iv.insert(out.iv.end(), blocks.begin(), blocks.end());
        out.ptr[t + 1] = (int32_t)out.iv.size();
      }
    }
    if (d->window > 0) clip_to_window(out, q_len, kv_len, d->window);
    return;
  }
  if (d->kind == MA_KIND_CAUSAL || d->kind == MA_KIND_SLIDING_WINDOW ||
      d->kind == MA_KIND_PREFIX_LM) {
    out.iv.reserve(q_len);
    for (int32_t t = 0; t < q_len; ++t) {
      const int64_t pos = t + delta;
      int64_t lo = 0, hi = std::min<int64_t>(kv_len, pos + 1);
      if (d->kind == MA_KIND_SLIDING_WINDOW) lo = std::max<int64_t>(0, pos - d->window + 1);
      if (d->kind == MA_KIND_PREFIX_LM) hi = std::min<int64_t>(kv_len, std::max<int64_t>(d->prefix_len[b], pos + 1));
      if (hi > lo) out.iv.push_back(Iv{(int32_t)lo, (int32_t)hi});
      out.ptr[t + 1] = (int32_t)out.iv.size();
    }
    return;
  }
  // RANGES: bucket every (row, interval) pair by row, then sort + merge.
  const ma_range *rg = d->ranges + d->range_indptr[b];
  const int32_t nr = d->range_indptr[b + 1] - d->range_indptr[b];
  std::vector<int32_t> cnt(q_len + 1, 0);
  for (int32_t k = 0; k < nr; ++k)
    if (rg[k].k_end > rg[k].k_start)
      for (int32_t t = rg[k].q_start; t < rg[k].q_end; ++t) cnt[t + 1]++;
  for (int32_t t = 0; t < q_len; ++t) cnt[t + 1] += cnt[t];
  std::vector<Iv> raw(cnt[q_len]);
  std::vector<int32_t> fill(cnt.begin(), cnt.end() - 1);
  for (int32_t k = 0; k < nr; ++k) {
    if (rg[k].k_end <= rg[k].k_start) continue;
    for (int32_t t = rg[k].q_start; t < rg[k].q_end; ++t)
      raw[fill[t]++] = range_row_interval(rg[k], t - rg[k].q_start);
  }
  out.iv.reserve(raw.size());
  for (int32_t t = 0; t < q_len; ++t) {
    auto first = raw.begin() + cnt[t], last = raw.begin() + cnt[t + 1];
    if (last - first > 1)
      std::sort(first, last, [](const Iv &a, const Iv &b) { return a.lo < b.lo; });
    for (auto it = first; it != last; ++it) {
      if (it->hi <= it->lo) continue;
      if ((int32_t)out.iv.size() > out.ptr[t] && out.iv.back().hi >= it->lo)
        out.iv.back().hi = std::max(out.iv.back().hi, it->hi);
      else
        out.iv.push_back(*it);
    }
    out.ptr[t + 1] = (int32_t)out.iv.size();
  }
}

inline uint64_t bits_between(int32_t lo, int32_t hi) {  // bits [lo, hi) of a word, 0 <= lo <= hi <= 64
  if (hi <= lo) return 0;
  const uint64_t upper = hi >= 64 ? ~0ull : ((1ull << hi) - 1);
  const uint64_t lower = (1ull << lo) - 1;
  return upper & ~lower;
}

struct RowPlan {
  std::vector<Entry> ents;
  std::vector<uint64_t> words;  // tile_q words per PARTIAL entry, in entry order
  int64_t cost = 0;
};

// Classify one q-tile row from interval lists.
void classify_qtile_intervals(const RowIntervals &R, int32_t r0, int32_t r1, int32_t kv_len,
                              int32_t tile_q, int32_t nkt, std::vector<int64_t> &cnt,
                              std::vector<int64_t> &diff, RowPlan &rp) {
  const int32_t BK = 64;
  cnt.assign(nkt, 0);
  diff.assign(nkt + 1, 0);
  for (int32_t t = r0; t < r1; ++t) {
    for (int32_t k = R.ptr[t]; k < R.ptr[t + 1]; ++k) {
      const Iv v = R.iv[k];
      const int32_t c0 = v.lo / BK, c1 = (v.hi - 1) / BK;
      if (c0 == c1) {
        cnt[c0] += v.hi - v.lo;
      } else {
        cnt[c0] += (int64_t)(c0 + 1) * BK - v.lo;
        cnt[c1] += v.hi - (int64_t)c1 * BK;
        if (c1 > c0 + 1) {
          diff[c0 + 1] += BK;
          diff[c1] -= BK;
        }
      }
    }
  }
  int64_t run = 0;
  const int64_t rows = r1 - r0;
  for (int32_t c = 0; c < nkt; ++c) {
    run += diff[c];
    const int64_t ones = cnt[c] + run;
    const int64_t keys = std::min<int64_t>(BK, (int64_t)kv_len - (int64_t)c * BK);
    const int64_t area = rows * keys;
    if (ones == 0) continue;
    if (ones == area) {
      rp.ents.push_back(Entry{c | (MA_TILE_FULL << kClsShift), -1});
      rp.cost += 4;
      continue;
    }
    rp.ents.push_back(Entry{c | (MA_TILE_PARTIAL << kClsShift), 0});
    rp.cost += 5;
    const size_t base = rp.words.size();
    rp.words.resize(base + tile_q, 0);
    const int32_t k0 = c * BK, k1 = k0 + BK;
    for (int32_t t = r0; t < r1; ++t) {
      uint64_t w = 0;
      for (int32_t k = R.ptr[t]; k < R.ptr[t + 1]; ++k) {
        const Iv v = R.iv[k];
        if (v.hi <= k0) continue;
        if (v.lo >= k1) break;
        w |= bits_between(std::max(v.lo, k0) - k0, std::min(v.hi, k1) - k0);
      }
      rp.words[base + (t - r0)] = w;
    }
  }
}

// Classify one q-tile row of a host-resident dense / packed mask (ANDed with
// the sliding-window band when a window is given).
void classify_qtile_matrix(const ma_mask_desc *d, int64_t moff, int32_t r0, int32_t r1,
                           int32_t q_len, int32_t kv_len, int32_t tile_q, int32_t nkt, RowPlan &rp) {
  const int32_t BK = 64;
  const int64_t nw = ceil_div(kv_len, 64);
  const int64_t delta = (int64_t)kv_len - q_len;
  std::vector<uint64_t> tw(tile_q);
  for (int32_t c = 0; c < nkt; ++c) {
    const int32_t keys = std::min<int32_t>(BK, kv_len - c * BK);
    const uint64_t inb = bits_between(0, keys);
    bool all_full = true, all_zero = true;
    for (int32_t t = r0; t < r1; ++t) {
      uint64_t w = 0;
      if (d->kind == MA_KIND_PACKED_U64) {
        w = ((const uint64_t *)d->mask)[moff + (int64_t)t * nw + c];
      } else {
        const uint8_t *row = (const uint8_t *)d->mask + moff + (int64_t)t * kv_len + (int64_t)c * BK;
        for (int32_t x = 0; x < keys; ++x) w |= (uint64_t)(row[x] != 0) << x;
      }
      w &= inb;
      if (d->window > 0) {
        const int64_t pos = t + delta;
        const int64_t lo = std::max<int64_t>(0, pos - d->window + 1 - (int64_t)c * BK);
        const int64_t hi = std::min<int64_t>(64, pos + 1 - (int64_t)c * BK);
        w &= hi > lo ? bits_between((int32_t)lo, (int32_t)hi) : 0ull;
      }
      tw[t - r0] = w;
      all_full &= (w == inb);
      all_zero &= (w == 0);
    }
    if (all_zero) continue;
    if (all_full) {
      rp.ents.push_back(Entry{c | (MA_TILE_FULL << kClsShift), -1});
      rp.cost += 4;
      continue;
    }
    rp.ents.push_back(Entry{c | (MA_TILE_PARTIAL << kClsShift), 0});
    rp.cost += 5;
    const size_t base = rp.words.size();
    rp.words.resize(base + tile_q, 0);
    for (int32_t t = r0; t < r1; ++t) rp.words[base + (t - r0)] = tw[t - r0];
  }
}

}  // namespace

ma_status set_error(ma_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

void clear_error() { g_last_error.clear(); }

const char *last_error_cstr() { return g_last_error.c_str(); }

ma_status validate_desc(const ma_mask_desc *d) {
  if (!d) return set_error(MA_ERR_INVALID, "mask description is NULL");
  if (d->batch < 1) return set_error(MA_ERR_INVALID, "batch must be >= 1 (got %d)", d->batch);
  if (!d->cu_seqlens_q || !d->kv_lens)
    return set_error(MA_ERR_INVALID, "cu_seqlens_q and kv_lens are required");
  if (d->tile_k != 64) return set_error(MA_ERR_UNSUPPORTED, "tile_k must be 64 (got %d)", d->tile_k);
  if (d->tile_q != 64 && d->tile_q != 128)
    return set_error(MA_ERR_UNSUPPORTED, "tile_q must be 64 or 128 (got %d)", d->tile_q);
  if (d->cu_seqlens_q[0] != 0) return set_error(MA_ERR_INVALID, "cu_seqlens_q[0] must be 0");
  for (int b = 0; b < d->batch; ++b) {
    const int64_t ql = (int64_t)d->cu_seqlens_q[b + 1] - d->cu_seqlens_q[b];
    if (ql < 0) return set_error(MA_ERR_INVALID, "cu_seqlens_q decreases at sequence %d", b);
    if (d->kv_lens[b] < 0) return set_error(MA_ERR_INVALID, "kv_lens[%d] < 0", b);
    if ((int64_t)d->kv_lens[b] > (int64_t)kKtMask * 64)
      return set_error(MA_ERR_UNSUPPORTED, "kv_lens[%d] too large", b);
  }
  const int kind = d->kind;
  if (kind < MA_KIND_CAUSAL || kind > MA_KIND_BLOCK_SPARSE)
    return set_error(MA_ERR_INVALID, "unknown mask kind %d", kind);
  // A sliding window is a restriction of causal masking (sglang-jax review);
  // with a custom or block-sparse mask it is an intersection (the joint use
  // asked about in flashinfer issue 724).  With PrefixLM or a range list it
  // is a conflict, as is a custom mask or range list supplied to a
  // closed-form kind.
  const bool custom = kind == MA_KIND_DENSE_BOOL || kind == MA_KIND_PACKED_U64;
  const bool window_ok = kind == MA_KIND_SLIDING_WINDOW || custom || kind == MA_KIND_BLOCK_SPARSE;
  if (!window_ok && d->window != 0)
    return set_error(MA_ERR_CONFLICT, "window is only valid with sliding-window, custom or block-sparse kinds");
  if (d->window < 0) return set_error(MA_ERR_INVALID, "window must be >= 0 (got %d)", d->window);
  if (kind != MA_KIND_BLOCK_SPARSE && (d->bsr_indptr || d->bsr_indices))
    return set_error(MA_ERR_CONFLICT, "block-sparse arrays were given with another kind");
  if (!custom && d->mask)
    return set_error(MA_ERR_CONFLICT, "a custom mask buffer was given with a non-custom kind");
  if (kind != MA_KIND_RANGES && (d->ranges || d->range_indptr))
    return set_error(MA_ERR_CONFLICT, "range descriptors were given with a non-range kind");
  if (kind != MA_KIND_PREFIX_LM && d->prefix_len)
    return set_error(MA_ERR_CONFLICT, "prefix_len was given with a non-PrefixLM kind");
  if (kind == MA_KIND_SLIDING_WINDOW && d->window < 1)
    return set_error(MA_ERR_INVALID, "window must be >= 1 (got %d)", d->window);
  if (kind == MA_KIND_PREFIX_LM) {
    if (!d->prefix_len) return set_error(MA_ERR_INVALID, "prefix_len is required for PrefixLM");
    for (int b = 0; b < d->batch; ++b)
      if (d->prefix_len[b] < 0 || d->prefix_len[b] > d->kv_lens[b])
        return set_error(MA_ERR_INVALID, "prefix_len[%d]=%d outside [0, kv_len=%d]", b,
                         d->prefix_len[b], d->kv_lens[b]);
  }
  if (kind == MA_KIND_RANGES) {
    if (!d->range_indptr) return set_error(MA_ERR_INVALID, "range_indptr is required for range lists");
    if (d->range_indptr[0] != 0) return set_error(MA_ERR_INVALID, "range_indptr[0] must be 0");
    if (d->range_indptr[d->batch] > 0 && !d->ranges)
      return set_error(MA_ERR_INVALID, "ranges is NULL");
    for (int b = 0; b < d->batch; ++b) {
      if (d->range_indptr[b + 1] < d->range_indptr[b])
        return set_error(MA_ERR_INVALID, "range_indptr decreases at sequence %d", b);
      const int32_t ql = d->cu_seqlens_q[b + 1] - d->cu_seqlens_q[b], kl = d->kv_lens[b];
      for (int32_t k = d->range_indptr[b]; k < d->range_indptr[b + 1]; ++k) {
        const ma_range &r = d->ranges[k];
        if (r.q_start < 0 || r.q_start > r.q_end || r.q_end > ql || r.k_start < 0 ||
            r.k_start > r.k_end || r.k_end > kl)
          return set_error(MA_ERR_INVALID,
                           "range %d of sequence %d ([%d,%d) x [%d,%d)) is outside [0,%d) x [0,%d)",
                           k - d->range_indptr[b], b, r.q_start, r.q_end, r.k_start, r.k_end, ql, kl);
        if (r.type < MA_RANGE_FULL || r.type > MA_RANGE_CHUNK_CAUSAL)
          return set_error(MA_ERR_INVALID, "range %d of sequence %d has unknown type %d",
                           k - d->range_indptr[b], b, r.type);
        if (r.type == MA_RANGE_CHUNK_CAUSAL && r.chunk_size < 1)
          return set_error(MA_ERR_INVALID, "chunk_size must be >= 1 (range %d of sequence %d)",
                           k - d->range_indptr[b], b);
      }
    }
  }
  if (kind == MA_KIND_BLOCK_SPARSE) {
    if (d->block_r < 1 || d->block_c < 1)
      return set_error(MA_ERR_INVALID, "block_r and block_c must be >= 1 (got %d, %d)", d->block_r, d->block_c);
    if (!d->bsr_indptr) return set_error(MA_ERR_INVALID, "bsr_indptr is required for block-sparse masks");
    if (d->bsr_indptr[0] != 0) return set_error(MA_ERR_INVALID, "bsr_indptr[0] must be 0");
    int64_t rb = 0;
    for (int b = 0; b < d->batch; ++b) {
      const int64_t ql = d->cu_seqlens_q[b + 1] - d->cu_seqlens_q[b];
      const int64_t ncb = ceil_div(d->kv_lens[b], d->block_c);
      for (int64_t r = 0; r < ceil_div(ql, d->block_r); ++r, ++rb) {
        if (d->bsr_indptr[rb + 1] < d->bsr_indptr[rb])
          return set_error(MA_ERR_INVALID, "bsr_indptr decreases at block row %lld", (long long)rb);
        if (d->bsr_indptr[rb + 1] > d->bsr_indptr[rb] && !d->bsr_indices)
          return set_error(MA_ERR_INVALID, "bsr_indices is NULL");
        for (int32_t k = d->bsr_indptr[rb]; k < d->bsr_indptr[rb + 1]; ++k)
          if (d->bsr_indices[k] < 0 || d->bsr_indices[k] >= ncb)
            return set_error(MA_ERR_INVALID, "block column %d of block row %lld (sequence %d) outside [0, %lld)",
                             d->bsr_indices[k], (long long)r, b, (long long)ncb);
      }
    }
  }
  if (custom) {
    if (!d->mask) return set_error(MA_ERR_INVALID, "custom mask buffer is NULL");
    int64_t need = 0;
    for (int b = 0; b < d->batch; ++b) {
      const int64_t ql = d->cu_seqlens_q[b + 1] - d->cu_seqlens_q[b], kl = d->kv_lens[b];
      need += kind == MA_KIND_DENSE_BOOL ? ql * kl : ql * ceil_div(kl, 64);
    }
    // The page's own check compares against the total kv length; the exact
    // requirement is one entry per (row, key) or per (row, word).
    if (d->mask_numel < need)
      return set_error(MA_ERR_SIZE, "custom mask has %lld elements, the sequences need %lld",
                       (long long)d->mask_numel, (long long)need);
  }
  return MA_OK;
}

ma_status plan_shape(const ma_mask_desc *d, ma_plan *p) {
  p->batch = d->batch;
  p->tile_q = d->tile_q;
  p->tile_k = d->tile_k;
  p->q_start.resize(d->batch);
  p->q_len.resize(d->batch);
  p->kv_len.resize(d->batch);
  p->nqt.resize(d->batch);
  p->nkt.resize(d->batch);
  p->tile_base.resize(d->batch);
  p->row_base.resize(d->batch);
  int64_t tiles = 0, rows = 0;
  for (int b = 0; b < d->batch; ++b) {
    p->q_start[b] = d->cu_seqlens_q[b];
    p->q_len[b] = d->cu_seqlens_q[b + 1] - d->cu_seqlens_q[b];
    p->kv_len[b] = d->kv_lens[b];
    p->nqt[b] = (int32_t)ceil_div(p->q_len[b], p->tile_q);
    p->nkt[b] = (int32_t)ceil_div(p->kv_len[b], p->tile_k);
    p->tile_base[b] = tiles;
    p->row_base[b] = (int32_t)rows;
    tiles += (int64_t)p->nqt[b] * p->nkt[b];
    rows += p->nqt[b];
  }
  if (rows > INT32_MAX / 2) return set_error(MA_ERR_UNSUPPORTED, "too many q-tiles");
  p->num_tiles = tiles;
  p->num_rows = (int32_t)rows;
  p->total_q = d->cu_seqlens_q[d->batch];
  return MA_OK;
}

ma_status compile_host(const ma_mask_desc *d, ma_plan *p) {
  std::vector<RowPlan> rps(p->num_rows);
  std::vector<int64_t> cnt, diff;
  RowIntervals R;
  int64_t moff = 0;
  const bool matrix = d->kind == MA_KIND_DENSE_BOOL || d->kind == MA_KIND_PACKED_U64;
  for (int b = 0; b < p->batch; ++b) {
    const int32_t ql = p->q_len[b], kl = p->kv_len[b];
    if (!matrix) build_rows(d, b, ql, kl, R);
    for (int32_t a = 0; a < p->nqt[b]; ++a) {
      const int32_t r0 = a * p->tile_q, r1 = std::min(ql, r0 + p->tile_q);
      RowPlan &rp = rps[p->row_base[b] + a];
      if (matrix)
        classify_qtile_matrix(d, moff, r0, r1, ql, kl, p->tile_q, p->nkt[b], rp);
      else
        classify_qtile_intervals(R, r0, r1, kl, p->tile_q, p->nkt[b], cnt, diff, rp);
    }
    if (matrix) moff += d->kind == MA_KIND_DENSE_BOOL ? (int64_t)ql * kl : (int64_t)ql * ceil_div(kl, 64);
  }
  // Execution order: most work first, ties by position (stable, so the order
  // is a function of the mask alone).
  std::vector<int32_t> order(p->num_rows);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t x, int32_t y) { return rps[x].cost > rps[y].cost; });
  std::vector<int32_t> row_seq(p->num_rows), row_qt(p->num_rows);
  for (int b = 0; b < p->batch; ++b)
    for (int32_t a = 0; a < p->nqt[b]; ++a) {
      row_seq[p->row_base[b] + a] = b;
      row_qt[p->row_base[b] + a] = a;
    }
  p->items.clear();
  p->entries.clear();
  p->words.clear();
  p->items.reserve(p->num_rows);
  int32_t wblk = 0;
  for (int32_t r : order) {
    RowPlan &rp = rps[r];
    Item it{row_seq[r], row_qt[r], (int32_t)p->entries.size(), 0};
    size_t wpos = 0;
    for (Entry e : rp.ents) {
      if (entry_cls(e.kt_cls) == MA_TILE_PARTIAL) {
        e.wblk = wblk++;
        p->words.insert(p->words.end(), rp.words.begin() + wpos, rp.words.begin() + wpos + p->tile_q);
        wpos += p->tile_q;
      }
      p->entries.push_back(e);
    }
    if (p->entries.size() > (size_t)INT32_MAX)
      return set_error(MA_ERR_UNSUPPORTED, "plan has too many tiles");
    it.ent_end = (int32_t)p->entries.size();
    p->items.push_back(it);
    rp = RowPlan();
  }
  p->num_wblk = wblk;
  p->host_valid = true;
  return MA_OK;
}

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Buffers of destroyed plans are kept for the next plans (device buffers per
// device, pinned host staging buffers), so that compiling a mask in steady
// state allocates nothing: a device-classified plan reserves a word block per
// tile (as much memory as the packed mask), and hipMalloc / hipHostMalloc /
// hipFree of that size cost far more than the classification itself.  A
// buffer is only returned to the cache after a device synchronisation (the
// plan's destruction waits, as hipFree did), and is reused for a request of
// at least half its size.  At most kCacheEntries buffers of each kind and
// kCacheBytes of device memory are held; the rest is freed.
namespace {
constexpr size_t kCacheEntries = 4;
constexpr size_t kCacheBytes = (size_t)2 << 30;
struct CachedBuf {
  void *ptr;
  size_t bytes;
  int dev;   // -1: pinned host memory
};
std::mutex g_cache_mu;
std::vector<CachedBuf> g_cache;

void *cache_take(size_t bytes, int dev, size_t *got) {
  std::lock_guard<std::mutex> lock(g_cache_mu);
  int best = -1;
  for (size_t i = 0; i < g_cache.size(); ++i) {
    const CachedBuf &c = g_cache[i];
    if (c.dev == dev && c.bytes >= bytes && c.bytes <= 2 * bytes + (1 << 20) &&
        (best < 0 || c.bytes < g_cache[best].bytes))
      best = (int)i;
  }
  if (best < 0) return nullptr;
  void *ptr = g_cache[best].ptr;
  *got = g_cache[best].bytes;
  g_cache.erase(g_cache.begin() + best);
  return ptr;
}

void release(void *ptr, int dev) {
  if (dev < 0) {
    (void)hipHostFree(ptr);
    return;
  }
  int cur = 0;
  (void)hipGetDevice(&cur);
  if (cur != dev) (void)hipSetDevice(dev);
  (void)hipFree(ptr);
  if (cur != dev) (void)hipSetDevice(cur);
}

// The caller has synchronised the device the buffer was last used on.
void cache_put(void *ptr, size_t bytes, int dev) {
  std::vector<CachedBuf> drop;
  {
    std::lock_guard<std::mutex> lock(g_cache_mu);
    g_cache.push_back(CachedBuf{ptr, bytes, dev});
    size_t dev_bytes = 0, n_dev = 0, n_host = 0;
    for (const CachedBuf &c : g_cache) {
      if (c.dev >= 0) {
        dev_bytes += c.bytes;
        ++n_dev;
      } else {
        ++n_host;
      }
    }
    // drop the oldest entries beyond the limits
    for (size_t i = 0; i < g_cache.size();) {
      const bool is_dev = g_cache[i].dev >= 0;
      if ((is_dev && (n_dev > kCacheEntries || dev_bytes > kCacheBytes)) || (!is_dev && n_host > kCacheEntries)) {
        if (is_dev) {
          --n_dev;
          dev_bytes -= g_cache[i].bytes;
        } else {
          --n_host;
        }
        drop.push_back(g_cache[i]);
        g_cache.erase(g_cache.begin() + i);
      } else {
        ++i;
      }
    }
  }
  for (const CachedBuf &c : drop) release(c.ptr, c.dev);
}
}  // namespace

ma_status plan_alloc_device(ma_plan *p, int64_t cap_entries, int64_t cap_wblk, size_t extra) {
  size_t off = 0;
  p->off_seqs = off;
  off = align_up(off + sizeof(SeqInfo) * p->batch, 256);
  p->off_aux = off;
  off = align_up(off + sizeof(SeqAux) * p->batch, 256);
  p->off_items = off;
  off = align_up(off + sizeof(Item) * (size_t)p->num_rows, 256);
  p->off_entries = off;
  off = align_up(off + sizeof(Entry) * (size_t)std::max<int64_t>(cap_entries, 1), 256);
  p->off_words = off;
  off = align_up(off + sizeof(uint64_t) * (size_t)p->tile_q * (size_t)std::max<int64_t>(cap_wblk, 1), 256);
  p->off_extra = off;
  off = align_up(off + extra, 256);
  if (p->dbuf && p->dbuf_bytes >= off) {
    p->dbytes = off;
    p->cap_entries = cap_entries;
    p->cap_wblk = cap_wblk;
    return MA_OK;
  }
  if (p->dbuf) {
    (void)hipFree(p->dbuf);
    p->dbuf = nullptr;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(MA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  size_t got = 0;
  p->dbuf = cache_take(off, dev, &got);
  if (!p->dbuf) {
    e = hipMalloc(&p->dbuf, off);
    if (e != hipSuccess) {
      p->dbuf = nullptr;
      return set_error(MA_ERR_NOMEM, "hipMalloc(%zu) for the plan: %s", off, hipGetErrorString(e));
    }
    got = off;
  }
  p->device_id = dev;
  p->dbytes = off;
  p->dbuf_bytes = got;
  p->cap_entries = cap_entries;
  p->cap_wblk = cap_wblk;
  return MA_OK;
}

void fill_seqinfo(const ma_plan *p, int32_t kind, std::vector<SeqInfo> &s, std::vector<SeqAux> &aux) {
  s.resize(p->batch);
  aux.resize(p->batch);
  int64_t moff = 0;
  for (int b = 0; b < p->batch; ++b) {
    s[b] = SeqInfo{p->q_start[b], p->q_len[b], p->kv_len[b], p->nkt[b]};
    aux[b] = SeqAux{p->tile_base[b], moff, p->row_base[b], p->nqt[b]};
    moff += kind == MA_KIND_DENSE_BOOL ? (int64_t)p->q_len[b] * p->kv_len[b]
                                       : (int64_t)p->q_len[b] * ceil_div(p->kv_len[b], 64);
  }
}

ma_status plan_staging(ma_plan *p, size_t bytes) {
  if (p->staging && p->staging_bytes >= bytes) return MA_OK;
  if (p->staging) {
    // an earlier upload may still read it
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return set_error(MA_ERR_HIP, "hipDeviceSynchronize: %s", hipGetErrorString(e));
    (void)hipHostFree(p->staging);
    p->staging = nullptr;
    p->staging_bytes = 0;
  }
  size_t got = 0;
  p->staging = cache_take(bytes, -1, &got);
  if (!p->staging) {
    hipError_t e = hipHostMalloc(&p->staging, bytes, hipHostMallocDefault);
    if (e != hipSuccess) {
      p->staging = nullptr;
      return set_error(MA_ERR_NOMEM, "hipHostMalloc(%zu): %s", bytes, hipGetErrorString(e));
    }
    got = bytes;
  }
  p->staging_bytes = got;
  return MA_OK;
}

ma_status plan_upload(ma_plan *p, void *stream) {
  if (p->on_device) return MA_OK;
  if (!p->host_valid) return set_error(MA_ERR_INVALID, "plan has neither a host nor a device copy");
  ma_status st = plan_alloc_device(p, (int64_t)p->entries.size(), p->num_wblk);
  if (st != MA_OK) return st;
  // Stage the whole plan in one pinned host buffer (kept by the plan until it
  // is destroyed) so one stream-ordered copy moves it and nothing waits.
  std::vector<SeqInfo> seqs;
  std::vector<SeqAux> aux;
  fill_seqinfo(p, MA_KIND_PACKED_U64, seqs, aux);
  if ((st = plan_staging(p, p->dbytes)) != MA_OK) return st;
  char *h = (char *)p->staging;
  memset(h, 0, p->dbytes);
  memcpy(h + p->off_seqs, seqs.data(), sizeof(SeqInfo) * seqs.size());
  memcpy(h + p->off_aux, aux.data(), sizeof(SeqAux) * aux.size());
  memcpy(h + p->off_items, p->items.data(), sizeof(Item) * p->items.size());
  memcpy(h + p->off_entries, p->entries.data(), sizeof(Entry) * p->entries.size());
  memcpy(h + p->off_words, p->words.data(), sizeof(uint64_t) * p->words.size());
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(p->dbuf, h, p->dbytes, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return set_error(MA_ERR_HIP, "plan upload: %s", hipGetErrorString(e));
  p->on_device = true;
  return MA_OK;
}

ma_status plan_fetch_host_view(const ma_plan *p, std::vector<Item> &items, std::vector<Entry> &entries,
                               std::vector<uint64_t> &words) {
  if (p->host_valid) {
    items = p->items;
    entries = p->entries;
    words = p->words;
    return MA_OK;
  }
  if (!p->on_device) return set_error(MA_ERR_INVALID, "plan has no data");
  std::vector<char> h(p->dbytes);
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(h.data(), p->dbuf, p->dbytes, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return set_error(MA_ERR_HIP, "plan download: %s", hipGetErrorString(e));
  items.resize(p->num_rows);
  memcpy(items.data(), h.data() + p->off_items, sizeof(Item) * p->num_rows);
  entries.resize(p->cap_entries);
  memcpy(entries.data(), h.data() + p->off_entries, sizeof(Entry) * p->cap_entries);
  words.resize((size_t)p->cap_wblk * p->tile_q);
  memcpy(words.data(), h.data() + p->off_words, sizeof(uint64_t) * words.size());
  return MA_OK;
}

ma_status plan_build_kmajor(ma_plan *p, void *stream) {
  if (p->kbuf) return MA_OK;
  std::vector<Item> items;
  std::vector<Entry> ents;
  std::vector<uint64_t> words;
  ma_status st = plan_fetch_host_view(p, items, ents, words);
  if (st != MA_OK) return st;
  // Bucket every non-SKIP tile by (sequence, k-tile).
  std::vector<int64_t> kbase(p->batch + 1, 0);
  for (int b = 0; b < p->batch; ++b) kbase[b + 1] = kbase[b] + p->nkt[b];
  const int64_t nk = kbase[p->batch];
  if (nk > INT32_MAX) return set_error(MA_ERR_UNSUPPORTED, "too many k-tiles for the backward");
  std::vector<std::vector<Entry>> bucket((size_t)nk);
  for (const Item &it : items)
    for (int32_t e = it.ent_begin; e < it.ent_end; ++e) {
      const int32_t kt = entry_kt(ents[e].kt_cls), cls = entry_cls(ents[e].kt_cls);
      bucket[(size_t)(kbase[it.seq] + kt)].push_back(Entry{it.qt | (cls << kClsShift), ents[e].wblk});
    }
  std::vector<Item> kitems;
  std::vector<Entry> kents;
  kitems.reserve((size_t)nk);
  for (int b = 0; b < p->batch; ++b)
    for (int32_t kt = 0; kt < p->nkt[b]; ++kt) {
      std::vector<Entry> &bk = bucket[(size_t)(kbase[b] + kt)];
      // Descending q-tiles: under causal-like masks the key tiles of a head
      // all end at the last q-tiles, so workgroups started together walk the
      // same query blocks at the same time and share them in L2.
      std::sort(bk.begin(), bk.end(), [](const Entry &x, const Entry &y) {
        return entry_kt(x.kt_cls) > entry_kt(y.kt_cls);
      });
      if (kents.size() + bk.size() > (size_t)INT32_MAX)
        return set_error(MA_ERR_UNSUPPORTED, "plan has too many tiles for the backward");
      Item it{b, kt, (int32_t)kents.size(), 0};
      kents.insert(kents.end(), bk.begin(), bk.end());
      it.ent_end = (int32_t)kents.size();
      kitems.push_back(it);
    }
  std::stable_sort(kitems.begin(), kitems.end(), [](const Item &x, const Item &y) {
    return (x.ent_end - x.ent_begin) > (y.ent_end - y.ent_begin);
  });
  const size_t off_ke = align_up(sizeof(Item) * std::max<size_t>(kitems.size(), 1), 256);
  const size_t bytes = off_ke + sizeof(Entry) * std::max<size_t>(kents.size(), 1);
  std::vector<char> h(bytes, 0);
  memcpy(h.data(), kitems.data(), sizeof(Item) * kitems.size());
  memcpy(h.data() + off_ke, kents.data(), sizeof(Entry) * kents.size());
  void *buf = nullptr;
  hipError_t e = hipMalloc(&buf, bytes);
  if (e != hipSuccess) return set_error(MA_ERR_NOMEM, "hipMalloc(%zu) for the k-major plan: %s", bytes, hipGetErrorString(e));
  e = hipMemcpyAsync(buf, h.data(), bytes, hipMemcpyHostToDevice, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);  // h is freed on return
  if (e != hipSuccess) {
    (void)hipFree(buf);
    return set_error(MA_ERR_HIP, "k-major plan upload: %s", hipGetErrorString(e));
  }
  p->kbuf = buf;
  p->off_kitems = 0;
  p->off_kentries = off_ke;
  p->num_kitems = (int32_t)kitems.size();
  return MA_OK;
}

void plan_free_device(ma_plan *p) {
  int cur = 0;
  (void)hipGetDevice(&cur);
  const bool other = p->device_id >= 0 && p->device_id != cur;
  if (other) (void)hipSetDevice(p->device_id);
  // nothing queued may still use the buffers once they are handed on
  (void)hipDeviceSynchronize();
  if (p->dbuf) cache_put(p->dbuf, p->dbuf_bytes ? p->dbuf_bytes : p->dbytes, p->device_id);
  if (p->kbuf) (void)hipFree(p->kbuf);
  if (p->staging) cache_put(p->staging, p->staging_bytes, -1);
  if (other) (void)hipSetDevice(cur);
  p->dbuf = nullptr;
  p->kbuf = nullptr;
  p->staging = nullptr;
  p->staging_bytes = 0;
  p->dbuf_bytes = 0;
}

}  // namespace maskattn
