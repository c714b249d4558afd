// C ABI of libmaskattn: argument validation (host only, before any HIP call),
// plan lifetime, and dispatch to the kernel launchers.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>

#include "internal.h"

namespace maskattn {
const char *last_error_cstr();
}

using namespace maskattn;

namespace {

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int log2i(int64_t x) {
  int s = 0;
  while ((1ll << s) < x) ++s;
  return s;
}

// q and out are required when there are query rows (rows = total_q > 0).
ma_status check_paged(const void *q, const void *k, const void *v, const void *out,
                      const int32_t *page_table, int32_t hq, int32_t hkv, int32_t page_size,
                      const int64_t *strides, int32_t max_pages, float scale, bool rows) {
  if (!k || !v || !page_table || !strides || (rows && (!q || !out)))
    return set_error(MA_ERR_INVALID, "q, k_cache, v_cache, page_table, kv_strides and out are required");
  if (hq < 1 || hkv < 1 || hq % hkv != 0)
    return set_error(MA_ERR_INVALID, "Hq (%d) must be a positive multiple of Hkv (%d)", hq, hkv);
  if (!is_pow2(page_size))
    return set_error(MA_ERR_UNSUPPORTED, "page_size must be a power of two (got %d)", page_size);
  if (strides[0] < 1 || strides[1] < 1 || strides[2] < 1)
    return set_error(MA_ERR_INVALID, "kv_strides must be positive");
  if (max_pages < 1) return set_error(MA_ERR_INVALID, "max_pages must be >= 1");
  if (!std::isfinite(scale) || !(scale > 0.f))
    return set_error(MA_ERR_INVALID, "scale must be positive and finite");
  return MA_OK;
}

}  // namespace

extern "C" {

const char *ma_status_string(int32_t s) {
  switch (s) {
    case MA_OK: return "ok";
    case MA_ERR_INVALID: return "invalid argument";
    case MA_ERR_CONFLICT: return "conflicting arguments";
    case MA_ERR_SIZE: return "buffer too small";
    case MA_ERR_UNSUPPORTED: return "unsupported configuration";
    case MA_ERR_PLAN_MISMATCH: return "plan does not match the call";
    case MA_ERR_HIP: return "HIP runtime error";
    case MA_ERR_NOMEM: return "out of memory";
    default: return "unknown status";
  }
}

const char *ma_last_error(void) { return last_error_cstr(); }

ma_status mask_compile_host(const ma_mask_desc *desc, ma_plan **out) {
  clear_error();
  if (!out) return set_error(MA_ERR_INVALID, "out is NULL");
  ma_status st = validate_desc(desc);
  if (st != MA_OK) return st;
  if ((desc->kind == MA_KIND_DENSE_BOOL || desc->kind == MA_KIND_PACKED_U64) && desc->mask_on_device)
    return set_error(MA_ERR_INVALID, "mask_compile_host needs a host-resident mask");
  ma_plan *p = new (std::nothrow) ma_plan();
  if (!p) return set_error(MA_ERR_NOMEM, "plan allocation failed");
  st = plan_shape(desc, p);
  if (st == MA_OK) st = compile_host(desc, p);
  if (st != MA_OK) {
    delete p;
    return st;
  }
  *out = p;
  return MA_OK;
}

ma_status mask_compile(const ma_mask_desc *desc, void *stream, ma_plan **out) {
  clear_error();
  if (!out) return set_error(MA_ERR_INVALID, "out is NULL");
  ma_status st = validate_desc(desc);
  if (st != MA_OK) return st;
  ma_plan *p = new (std::nothrow) ma_plan();
  if (!p) return set_error(MA_ERR_NOMEM, "plan allocation failed");
  st = plan_shape(desc, p);
  const bool device_mask =
      (desc->kind == MA_KIND_DENSE_BOOL || desc->kind == MA_KIND_PACKED_U64) && desc->mask_on_device;
  if (st == MA_OK) {
    if (device_mask) {
      st = launch_classify(p, desc->mask, desc->kind, desc->mask_numel, desc->window, stream);
    } else {
      st = compile_host(desc, p);
      if (st == MA_OK) st = plan_upload(p, stream);
    }
  }
  if (st != MA_OK) {
    mask_plan_destroy(p);
    return st;
  }
  *out = p;
  return MA_OK;
}

ma_status mask_plan_upload(ma_plan *plan, void *stream) {
  clear_error();
  if (!plan) return set_error(MA_ERR_INVALID, "plan is NULL");
  return plan_upload(plan, stream);
}

ma_status mask_plan_destroy(ma_plan *plan) {
  if (!plan) return MA_OK;
  if (plan->dbuf || plan->kbuf || plan->staging) plan_free_device(plan);
  delete plan;
  return MA_OK;
}

ma_status mask_plan_info_get(const ma_plan *p, ma_plan_info *o) {
  clear_error();
  if (!p || !o) return set_error(MA_ERR_INVALID, "plan and out are required");
  o->batch = p->batch;
  o->tile_q = p->tile_q;
  o->tile_k = p->tile_k;
  o->num_qtiles = p->num_rows;
  o->num_tiles = p->num_tiles;
  o->num_entries = p->host_valid ? (int64_t)p->entries.size() : p->cap_entries;
  o->num_word_blocks = p->host_valid ? p->num_wblk : p->cap_wblk;
  o->total_q = p->total_q;
  o->device_bytes = p->on_device ? (int64_t)p->dbytes : 0;
  o->on_device = p->on_device ? 1 : 0;
  o->host_valid = p->host_valid ? 1 : 0;
  return MA_OK;
}

ma_status mask_plan_export(const ma_plan *p, uint8_t *classes, uint64_t *words) {
  clear_error();
  if (!p || !classes) return set_error(MA_ERR_INVALID, "plan and classes are required");
  std::vector<Item> items;
  std::vector<Entry> ents;
  std::vector<uint64_t> w;
  ma_status st = plan_fetch_host_view(p, items, ents, w);
  if (st != MA_OK) return st;
  memset(classes, MA_TILE_SKIP, (size_t)p->num_tiles);
  const size_t tw = (size_t)p->tile_q * (p->tile_k / 64);
  if (words) memset(words, 0, sizeof(uint64_t) * tw * (size_t)p->num_tiles);
  for (const Item &it : items) {
    const int64_t base = p->tile_base[it.seq] + (int64_t)it.qt * p->nkt[it.seq];
    for (int32_t e = it.ent_begin; e < it.ent_end; ++e) {
      const int32_t kt = entry_kt(ents[e].kt_cls), cls = entry_cls(ents[e].kt_cls);
      classes[base + kt] = (uint8_t)cls;
      if (words && cls == MA_TILE_PARTIAL)
        memcpy(words + (size_t)(base + kt) * tw, w.data() + (size_t)ents[e].wblk * tw, sizeof(uint64_t) * tw);
    }
  }
  return MA_OK;
}

ma_status mask_plan_serialize(const ma_plan *p, void *dst, size_t *bytes) {
  clear_error();
  if (!p || !bytes) return set_error(MA_ERR_INVALID, "plan and bytes are required");
  std::vector<Item> items;
  std::vector<Entry> ents;
  std::vector<uint64_t> w;
  ma_status st = plan_fetch_host_view(p, items, ents, w);
  if (st != MA_OK) return st;
  // Layout: header (batch, tile_q, tile_k, num_rows), then per item in
  // execution order: seq, qt, count, and per entry (k-tile | class << 30)
  // followed by tile_q words when PARTIAL.
  std::vector<int32_t> out32;
  std::vector<uint64_t> out64;
  size_t n = 4 * sizeof(int32_t);
  for (const Item &it : items) {
    n += 3 * sizeof(int32_t);
    for (int32_t e = it.ent_begin; e < it.ent_end; ++e) {
      n += sizeof(int32_t);
      if (entry_cls(ents[e].kt_cls) == MA_TILE_PARTIAL) n += sizeof(uint64_t) * p->tile_q;
    }
  }
  if (!dst) {
    *bytes = n;
    return MA_OK;
  }
  if (*bytes < n) return set_error(MA_ERR_SIZE, "serialize buffer has %zu bytes, needs %zu", *bytes, n);
  char *o = (char *)dst;
  auto put32 = [&](int32_t v) { memcpy(o, &v, 4); o += 4; };
  put32(p->batch);
  put32(p->tile_q);
  put32(p->tile_k);
  put32(p->num_rows);
  for (const Item &it : items) {
    put32(it.seq);
    put32(it.qt);
    put32(it.ent_end - it.ent_begin);
    for (int32_t e = it.ent_begin; e < it.ent_end; ++e) {
      put32(ents[e].kt_cls);
      if (entry_cls(ents[e].kt_cls) == MA_TILE_PARTIAL) {
        memcpy(o, w.data() + (size_t)ents[e].wblk * p->tile_q, sizeof(uint64_t) * p->tile_q);
        o += sizeof(uint64_t) * p->tile_q;
      }
    }
  }
  *bytes = n;
  return MA_OK;
}

ma_status attn_prefill_masked(const ma_plan *plan, const void *q, int64_t total_q, int32_t hq,
                              const void *k_cache, const void *v_cache, int32_t hkv, int32_t d,
                              int32_t page_size, const int64_t kv_strides[3],
                              const int32_t *page_table, int32_t max_pages, int32_t in_dtype,
                              int32_t out_dtype, float scale, void *out, float *lse, void *stream) {
  clear_error();
  if (!plan) return set_error(MA_ERR_INVALID, "plan is NULL");
  ma_status st = check_paged(q, k_cache, v_cache, out, page_table, hq, hkv, page_size, kv_strides,
                             max_pages, scale, total_q > 0);
  if (st != MA_OK) return st;
  if (total_q != plan->total_q)
    return set_error(MA_ERR_PLAN_MISMATCH, "total_q %lld differs from the plan's %lld",
                     (long long)total_q, (long long)plan->total_q);
  if (plan->tile_k != 64) return set_error(MA_ERR_PLAN_MISMATCH, "plan tile_k %d has no kernel", plan->tile_k);
  for (int b = 0; b < plan->batch; ++b)
    if ((int64_t)max_pages * page_size < plan->kv_len[b])
      return set_error(MA_ERR_INVALID, "page table (max_pages %d x page_size %d) shorter than kv_len %d",
                       max_pages, page_size, plan->kv_len[b]);
  if (in_dtype == MA_BF16) {
    if (d != 64 && d != 128 && d != 256)
      return set_error(MA_ERR_UNSUPPORTED, "bf16 head_dim %d (supported: 64, 128, 256)", d);
    if (out_dtype != MA_BF16 && out_dtype != MA_F32)
      return set_error(MA_ERR_UNSUPPORTED, "out dtype %d", out_dtype);
  } else if (in_dtype == MA_F32) {
    if (d != 64 && d != 128) return set_error(MA_ERR_UNSUPPORTED, "fp32 head_dim %d (supported: 64, 128)", d);
    if (out_dtype != MA_F32) return set_error(MA_ERR_UNSUPPORTED, "fp32 inputs need fp32 output");
  } else {
    return set_error(MA_ERR_UNSUPPORTED, "input dtype %d", in_dtype);
  }
  if (kv_strides[2] < d) return set_error(MA_ERR_INVALID, "head stride %lld < head_dim", (long long)kv_strides[2]);
  if (total_q == 0 || plan->num_rows == 0) return MA_OK;
  if (!plan->on_device) {
    st = plan_upload(const_cast<ma_plan *>(plan), stream);
    if (st != MA_OK) return st;
  }
  PrefillArgs a{};
  a.plan = plan;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.hq = hq;
  a.hkv = hkv;
  a.d = d;
  a.page_shift = log2i(page_size);
  a.s_page = kv_strides[0];
  a.s_slot = kv_strides[1];
  a.s_head = kv_strides[2];
  a.page_table = page_table;
  a.max_pages = max_pages;
  a.in_dtype = in_dtype;
  a.out_dtype = out_dtype;
  a.scale = scale;
  a.out = out;
  a.lse = lse;
  a.stream = stream;
  return launch_prefill(a);
}

ma_status attn_prefill_masked_fp8(const ma_plan *plan, const void *q, int64_t total_q, int32_t hq,
                                  const void *k_cache, const void *v_cache, int32_t hkv, int32_t d,
                                  int32_t page_size, const int64_t kv_strides[3], const int32_t *page_table,
                                  int32_t max_pages, float q_descale, float k_descale, float v_descale,
                                  int32_t out_dtype, float scale, void *out, float *lse, void *stream) {
  clear_error();
  if (!plan) return set_error(MA_ERR_INVALID, "plan is NULL");
  ma_status st = check_paged(q, k_cache, v_cache, out, page_table, hq, hkv, page_size, kv_strides,
                             max_pages, scale, total_q > 0);
  if (st != MA_OK) return st;
  for (float f : {q_descale, k_descale, v_descale})
    if (!std::isfinite(f) || !(f > 0.f)) return set_error(MA_ERR_INVALID, "descale factors must be positive and finite");
  if (total_q != plan->total_q)
    return set_error(MA_ERR_PLAN_MISMATCH, "total_q %lld differs from the plan's %lld",
                     (long long)total_q, (long long)plan->total_q);
  if (plan->tile_k != 64 || plan->tile_q != 128)
    return set_error(MA_ERR_PLAN_MISMATCH, "fp8 prefill needs a 128 x 64 tile plan (got %d x %d)", plan->tile_q,
                     plan->tile_k);
  for (int b = 0; b < plan->batch; ++b)
    if ((int64_t)max_pages * page_size < plan->kv_len[b])
      return set_error(MA_ERR_INVALID, "page table (max_pages %d x page_size %d) shorter than kv_len %d",
                       max_pages, page_size, plan->kv_len[b]);
  if (d != 64 && d != 128 && d != 256)
    return set_error(MA_ERR_UNSUPPORTED, "fp8 head_dim %d (supported: 64, 128, 256)", d);
  if (out_dtype != MA_BF16 && out_dtype != MA_F32) return set_error(MA_ERR_UNSUPPORTED, "out dtype %d", out_dtype);
  if (kv_strides[2] < d) return set_error(MA_ERR_INVALID, "head stride %lld < head_dim", (long long)kv_strides[2]);
  if (page_size < fp8_rows_per_gather(d))
    return set_error(MA_ERR_UNSUPPORTED, "fp8 prefill needs pages of at least %d keys at head_dim %d",
                     fp8_rows_per_gather(d), d);
  if ((int64_t)page_size * kv_strides[1] >= ((int64_t)1 << 31) || kv_strides[0] >= ((int64_t)1 << 32))
    return set_error(MA_ERR_UNSUPPORTED, "a page's bytes exceed a 32-bit offset");
  if (total_q == 0 || plan->num_rows == 0) return MA_OK;
  if (!plan->on_device) {
    st = plan_upload(const_cast<ma_plan *>(plan), stream);
    if (st != MA_OK) return st;
  }
  Fp8Args a{};
  a.plan = plan;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.hq = hq;
  a.hkv = hkv;
  a.d = d;
  a.page_shift = log2i(page_size);
  a.s_page = kv_strides[0];
  a.s_slot = kv_strides[1];
  a.s_head = kv_strides[2];
  a.page_table = page_table;
  a.max_pages = max_pages;
  a.out_dtype = out_dtype;
  a.scale = scale;
  a.q_descale = q_descale;
  a.k_descale = k_descale;
  a.v_descale = v_descale;
  a.out = out;
  a.lse = lse;
  a.stream = stream;
  return launch_prefill_fp8(a);
}

size_t attn_backward_workspace(const ma_plan *plan, int32_t hq) {
  if (!plan || hq < 1) return 0;
  return backward_workspace(plan->total_q, hq);
}

ma_status attn_backward_masked(ma_plan *plan, const void *q, int64_t total_q, int32_t hq, const void *k_cache,
                               const void *v_cache, int32_t hkv, int32_t d, int32_t page_size,
                               const int64_t kv_strides[3], const int32_t *page_table, int32_t max_pages,
                               const void *out, int32_t out_dtype, const void *dout, const float *lse,
                               float scale, float *dq, float *dk_cache, float *dv_cache, void *workspace,
                               size_t ws_bytes, void *stream) {
  clear_error();
  if (!plan) return set_error(MA_ERR_INVALID, "plan is NULL");
  ma_status st = check_paged(q, k_cache, v_cache, out, page_table, hq, hkv, page_size, kv_strides,
                             max_pages, scale, total_q > 0);
  if (st != MA_OK) return st;
  if (!dk_cache || !dv_cache || (total_q > 0 && (!dout || !lse || !dq)))
    return set_error(MA_ERR_INVALID, "dout, lse, dq, dk_cache and dv_cache are required");
  if (total_q != plan->total_q)
    return set_error(MA_ERR_PLAN_MISMATCH, "total_q %lld differs from the plan's %lld",
                     (long long)total_q, (long long)plan->total_q);
  if (plan->tile_k != 64 || (plan->tile_q != 64 && plan->tile_q != 128))
    return set_error(MA_ERR_PLAN_MISMATCH, "plan tiles %dx%d have no backward kernel", plan->tile_q, plan->tile_k);
  for (int b = 0; b < plan->batch; ++b)
    if ((int64_t)max_pages * page_size < plan->kv_len[b])
      return set_error(MA_ERR_INVALID, "page table (max_pages %d x page_size %d) shorter than kv_len %d",
                       max_pages, page_size, plan->kv_len[b]);
  if (d != 64 && d != 128 && d != 256)
    return set_error(MA_ERR_UNSUPPORTED, "backward head_dim %d (supported: 64, 128, 256)", d);
  if (out_dtype != MA_BF16 && out_dtype != MA_F32)
    return set_error(MA_ERR_UNSUPPORTED, "out dtype %d", out_dtype);
  if (kv_strides[2] < d) return set_error(MA_ERR_INVALID, "head stride %lld < head_dim", (long long)kv_strides[2]);
  // No early return for a plan without query rows: dK / dV of its keys are
  // still written (zeros); the passes over query rows then have empty grids.
  const size_t need = backward_workspace(total_q, hq);
  if (need > 0 && (!workspace || ws_bytes < need))
    return set_error(MA_ERR_SIZE, "workspace of %zu bytes is below the %zu required", ws_bytes, need);
  if (!plan->on_device) {
    st = plan_upload(plan, stream);
    if (st != MA_OK) return st;
  }
  BackwardArgs a{};
  a.plan = plan;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.o = out;
  a.dout = dout;
  a.lse = lse;
  a.hq = hq;
  a.hkv = hkv;
  a.d = d;
  a.page_shift = log2i(page_size);
  a.total_q = total_q;
  a.s_page = kv_strides[0];
  a.s_slot = kv_strides[1];
  a.s_head = kv_strides[2];
  a.page_table = page_table;
  a.max_pages = max_pages;
  a.o_dtype = out_dtype;
  a.scale = scale;
  a.dq = dq;
  a.dk = dk_cache;
  a.dv = dv_cache;
  a.workspace = workspace;
  a.stream = stream;
  return launch_backward(a);
}

size_t attn_verify_tree_workspace(int32_t batch, int32_t max_q, int32_t max_kv, int32_t hq,
                                  int32_t hkv, int32_t d) {
  if (batch < 1 || max_q < 1 || max_kv < 1 || hq < 1 || hkv < 1 || d < 1) return 0;
  return verify_workspace(batch, max_q, max_kv, hq, hkv, d);
}

// Checks shared by tree verify and decode (small-q launches).
static ma_status check_small_q(const void *q, const void *k_cache, const void *v_cache, void *out,
                               const int32_t *page_table, int32_t hq, int32_t hkv, int32_t page_size,
                               const int64_t kv_strides[3], int32_t max_pages, float scale,
                               const int32_t *cu_seqlens_q, const int32_t *kv_lens, int32_t batch,
                               int32_t max_q, int32_t max_kv, int32_t in_dtype, int32_t out_dtype, int32_t d,
                               int64_t total_q) {
  // q and out are always required here: the rows are counted on the device
  ma_status st = check_paged(q, k_cache, v_cache, out, page_table, hq, hkv, page_size, kv_strides,
                             max_pages, scale, true);
  if (st != MA_OK) return st;
  if (!cu_seqlens_q || !kv_lens) return set_error(MA_ERR_INVALID, "cu_seqlens_q and kv_lens are required");
  if (batch < 1) return set_error(MA_ERR_INVALID, "batch must be >= 1");
  if (max_q < 1 || max_q > 64) return set_error(MA_ERR_UNSUPPORTED, "max_q must be in [1, 64] (got %d)", max_q);
  if (max_kv < 1) return set_error(MA_ERR_INVALID, "max_kv must be >= 1");
  if ((int64_t)max_pages * page_size < max_kv)
    return set_error(MA_ERR_INVALID, "page table shorter than max_kv");
  if (in_dtype != MA_BF16) return set_error(MA_ERR_UNSUPPORTED, "small-q attention needs bf16 inputs");
  if (d != 64 && d != 128 && d != 256) return set_error(MA_ERR_UNSUPPORTED, "head_dim %d", d);
  if (out_dtype != MA_BF16 && out_dtype != MA_F32) return set_error(MA_ERR_UNSUPPORTED, "out dtype %d", out_dtype);
  if (kv_strides[2] < d) return set_error(MA_ERR_INVALID, "head stride < head_dim");
  if (total_q < 0 || total_q > (int64_t)batch * max_q) return set_error(MA_ERR_INVALID, "total_q out of range");
  return MA_OK;
}

// A dense or packed mask needs at least one element per query row (every
// row that exists has kv_len >= q_len >= 1 keys).  The exact size depends on
// the device-resident lengths and is not known here; the kernels read
// elements at or past mask_numel as 0 (masked), never past the buffer.
static ma_status check_mask_rows(const void *mask, int64_t mask_numel, int64_t total_q) {
  if (!mask || mask_numel < 1) return set_error(MA_ERR_INVALID, "mask is required");
  if (mask_numel < total_q)
    return set_error(MA_ERR_SIZE, "mask has %lld elements, fewer than its %lld query rows need",
                     (long long)mask_numel, (long long)total_q);
  return MA_OK;
}

static ma_status run_small_q(const void *q, int32_t hq, const void *k_cache, const void *v_cache, int32_t hkv,
                             int32_t d, int32_t page_size, const int64_t kv_strides[3], const int32_t *page_table,
                             int32_t max_pages, const int32_t *cu_seqlens_q, const int32_t *kv_lens,
                             int32_t batch, int32_t max_q, int32_t max_kv, int32_t mask_kind, int32_t window,
                             const int32_t *prefix_len, const void *mask, int64_t mask_numel, int32_t out_dtype,
                             float scale, void *workspace, size_t ws_bytes, void *out, float *lse,
                             void *stream, int32_t kv8 = 0, float k_descale = 1.f, float v_descale = 1.f) {
  const size_t need = verify_workspace(batch, max_q, max_kv, hq, hkv, d);
  if (need > 0 && (!workspace || ws_bytes < need))
    return set_error(MA_ERR_SIZE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  VerifyArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.hq = hq;
  a.hkv = hkv;
  a.d = d;
  a.page_shift = log2i(page_size);
  a.s_page = kv_strides[0];
  a.s_slot = kv_strides[1];
  a.s_head = kv_strides[2];
  a.page_table = page_table;
  a.max_pages = max_pages;
  a.cu_seqlens_q = cu_seqlens_q;
  a.kv_lens = kv_lens;
  a.batch = batch;
  a.max_q = max_q;
  a.max_kv = max_kv;
  a.mask_kind = mask_kind;
  a.mask = mask;
  a.mask_numel = mask_numel;
  a.window = window;
  a.prefix_len = prefix_len;
  a.out_dtype = out_dtype;
  a.scale = scale;
  a.workspace = workspace;
  a.ws_bytes = ws_bytes;
  a.out = out;
  a.lse = lse;
  a.stream = stream;
  a.kv8 = kv8;
  a.k_descale = k_descale;
  a.v_descale = v_descale;
  return launch_verify(a);
}

size_t attn_decode_workspace(int32_t batch, int32_t max_q, int32_t max_kv, int32_t hq, int32_t hkv, int32_t d) {
  if (batch < 1 || max_q < 1 || max_q > 64 || max_kv < 1 || hq < 1 || hkv < 1 || d < 1 || hq % hkv != 0) return 0;
  return verify_workspace(batch, max_q, max_kv, hq, hkv, d);
}

ma_status attn_decode(const void *q, int64_t total_q, int32_t hq, const void *k_cache, const void *v_cache,
                      int32_t hkv, int32_t d, int32_t page_size, const int64_t kv_strides[3],
                      const int32_t *page_table, int32_t max_pages, const int32_t *cu_seqlens_q,
                      const int32_t *kv_lens, int32_t batch, int32_t max_q, int32_t max_kv, int32_t mask_kind,
                      int32_t window, const int32_t *prefix_len, const void *mask, int64_t mask_numel,
                      int32_t in_dtype, int32_t out_dtype, float scale, void *workspace, size_t ws_bytes,
                      void *out, float *lse, void *stream) {
  clear_error();
  ma_status st = check_small_q(q, k_cache, v_cache, out, page_table, hq, hkv, page_size, kv_strides, max_pages,
                               scale, cu_seqlens_q, kv_lens, batch, max_q, max_kv, in_dtype, out_dtype, d, total_q);
  if (st != MA_OK) return st;
  switch (mask_kind) {
    case MA_KIND_CAUSAL:
      break;
    case MA_KIND_SLIDING_WINDOW:
      if (window < 1) return set_error(MA_ERR_INVALID, "window must be >= 1 (got %d)", window);
      break;
    case MA_KIND_PREFIX_LM:
      if (!prefix_len) return set_error(MA_ERR_INVALID, "prefix_len is required for PREFIX_LM");
      break;
    case MA_KIND_DENSE_BOOL:
    case MA_KIND_PACKED_U64:
      if ((st = check_mask_rows(mask, mask_numel, total_q)) != MA_OK) return st;
      break;
    case MA_KIND_RANGES:
      return set_error(MA_ERR_UNSUPPORTED, "decode takes RANGES masks as dense or packed rows");
    default:
      return set_error(MA_ERR_INVALID, "mask kind %d", mask_kind);
  }
  return run_small_q(q, hq, k_cache, v_cache, hkv, d, page_size, kv_strides, page_table, max_pages, cu_seqlens_q,
                     kv_lens, batch, max_q, max_kv, mask_kind, window, prefix_len, mask, mask_numel, out_dtype,
                     scale, workspace, ws_bytes, out, lse, stream);
}

ma_status attn_decode_kv8(const void *q, int64_t total_q, int32_t hq, const void *k_cache, const void *v_cache,
                          int32_t hkv, int32_t d, int32_t page_size, const int64_t kv_strides[3],
                          const int32_t *page_table, int32_t max_pages, const int32_t *cu_seqlens_q,
                          const int32_t *kv_lens, int32_t batch, int32_t max_q, int32_t max_kv, int32_t mask_kind,
                          int32_t window, const int32_t *prefix_len, const void *mask, int64_t mask_numel,
                          int32_t out_dtype, float scale, float k_descale, float v_descale, void *workspace,
                          size_t ws_bytes, void *out, float *lse, void *stream) {
  clear_error();
  ma_status st = check_small_q(q, k_cache, v_cache, out, page_table, hq, hkv, page_size, kv_strides, max_pages,
                               scale, cu_seqlens_q, kv_lens, batch, max_q, max_kv, MA_BF16, out_dtype, d, total_q);
  if (st != MA_OK) return st;
  if (!(k_descale > 0.f) || !(v_descale > 0.f) || !std::isfinite(k_descale) || !std::isfinite(v_descale))
    return set_error(MA_ERR_INVALID, "descale factors must be positive and finite");
  if (page_size < 1024 / d)
    return set_error(MA_ERR_UNSUPPORTED, "fp8 caches need pages of at least %d keys at head_dim %d", 1024 / d, d);
  if ((int64_t)page_size * kv_strides[1] >= ((int64_t)1 << 31) || kv_strides[0] >= ((int64_t)1 << 32))
    return set_error(MA_ERR_UNSUPPORTED, "a page's bytes exceed a 32-bit offset");
  switch (mask_kind) {
    case MA_KIND_CAUSAL:
      break;
    case MA_KIND_SLIDING_WINDOW:
      if (window < 1) return set_error(MA_ERR_INVALID, "window must be >= 1 (got %d)", window);
      break;
    case MA_KIND_PREFIX_LM:
      if (!prefix_len) return set_error(MA_ERR_INVALID, "prefix_len is required for PREFIX_LM");
      break;
    case MA_KIND_DENSE_BOOL:
    case MA_KIND_PACKED_U64:
      if ((st = check_mask_rows(mask, mask_numel, total_q)) != MA_OK) return st;
      break;
    case MA_KIND_RANGES:
      return set_error(MA_ERR_UNSUPPORTED, "decode takes RANGES masks as dense or packed rows");
    default:
      return set_error(MA_ERR_INVALID, "mask kind %d", mask_kind);
  }
  return run_small_q(q, hq, k_cache, v_cache, hkv, d, page_size, kv_strides, page_table, max_pages, cu_seqlens_q,
                     kv_lens, batch, max_q, max_kv, mask_kind, window, prefix_len, mask, mask_numel, out_dtype,
                     scale, workspace, ws_bytes, out, lse, stream, 1, k_descale, v_descale);
}

ma_status attn_verify_tree(const void *q, int64_t total_q, int32_t hq, const void *k_cache,
                           const void *v_cache, int32_t hkv, int32_t d, int32_t page_size,
                           const int64_t kv_strides[3], const int32_t *page_table,
                           int32_t max_pages, const int32_t *cu_seqlens_q, const int32_t *kv_lens,
                           int32_t batch, int32_t max_q, int32_t max_kv, int32_t mask_kind,
                           const void *mask, int64_t mask_numel, int32_t in_dtype,
                           int32_t out_dtype, float scale, void *workspace, size_t ws_bytes,
                           void *out, float *lse, void *stream) {
  clear_error();
  ma_status st = check_small_q(q, k_cache, v_cache, out, page_table, hq, hkv, page_size, kv_strides, max_pages,
                               scale, cu_seqlens_q, kv_lens, batch, max_q, max_kv, in_dtype, out_dtype, d, total_q);
  if (st != MA_OK) return st;
  if (mask_kind != MA_KIND_DENSE_BOOL && mask_kind != MA_KIND_PACKED_U64)
    return set_error(MA_ERR_CONFLICT, "tree verify takes a custom mask (dense or packed), got kind %d", mask_kind);
  if ((st = check_mask_rows(mask, mask_numel, total_q)) != MA_OK) return st;
  return run_small_q(q, hq, k_cache, v_cache, hkv, d, page_size, kv_strides, page_table, max_pages, cu_seqlens_q,
                     kv_lens, batch, max_q, max_kv, mask_kind, 0, nullptr, mask, mask_numel, out_dtype, scale,
                     workspace, ws_bytes, out, lse, stream);
}

ma_status attn_verify_tree_noalloc(const void *q, int64_t total_q, int32_t hq, const void *k_cache,
                                   const void *v_cache, int32_t hkv, int32_t d, int32_t page_size,
                                   const int64_t kv_strides[3], const int32_t *page_table, int32_t max_pages,
                                   const int32_t *cu_seqlens_q, const int32_t *kv_lens, int32_t batch,
                                   int32_t max_q, int32_t max_kv, int32_t mask_kind, const void *mask,
                                   int64_t mask_numel, int32_t in_dtype, int32_t out_dtype, float scale, void *out,
                                   float *lse, void *stream) {
  clear_error();
  ma_status st = check_small_q(q, k_cache, v_cache, out, page_table, hq, hkv, page_size, kv_strides, max_pages,
                               scale, cu_seqlens_q, kv_lens, batch, max_q, max_kv, in_dtype, out_dtype, d, total_q);
  if (st != MA_OK) return st;
  if (mask_kind != MA_KIND_DENSE_BOOL && mask_kind != MA_KIND_PACKED_U64)
    return set_error(MA_ERR_CONFLICT, "tree verify takes a custom mask (dense or packed), got kind %d", mask_kind);
  if ((st = check_mask_rows(mask, mask_numel, total_q)) != MA_OK) return st;
  const size_t need = verify_workspace(batch, max_q, max_kv, hq, hkv, d);
  if (need > kVerifyScratchBytes)
    return set_error(MA_ERR_SIZE, "these bounds need %zu bytes of scratch, the library holds %zu per GPU", need,
                     kVerifyScratchBytes);
  void *ws = nullptr;
  if (need > 0 && (st = verify_scratch(&ws)) != MA_OK) return st;
  return run_small_q(q, hq, k_cache, v_cache, hkv, d, page_size, kv_strides, page_table, max_pages, cu_seqlens_q,
                     kv_lens, batch, max_q, max_kv, mask_kind, 0, nullptr, mask, mask_numel, out_dtype, scale, ws,
                     need, out, lse, stream);
}

}  // extern "C"
