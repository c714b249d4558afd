// Internal declarations shared by the host side of libmaskattn (plan
// compiler, C ABI) and the kernel launchers.  Not installed.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "maskattn.h"

namespace maskattn {

// Device-side plan records.  A plan buffer holds, in this order:
//   SeqInfo  seqs[batch]
//   SeqAux   aux[batch]
//   Item     items[num_rows]         execution order (most work first)
//   Entry    entries[cap_entries]    non-SKIP tiles of each q-tile, k ascending
//   uint64   words[cap_wblk][tile_q] one word per row of each PARTIAL tile
struct SeqInfo {
  int32_t q_start, q_len, kv_len, nkt;
};
struct Item {
  int32_t seq, qt, ent_begin, ent_end;
};
// Per-sequence offsets used by the device classifier.
struct SeqAux {
  int64_t tile_base;  // first global tile index
  int64_t moff;       // first mask element of the sequence
  int32_t row_base;   // first global q-tile row
  int32_t nqt;
};
struct Entry {
  int32_t kt_cls;  // k-tile index | class << 30
  int32_t wblk;    // word block of a PARTIAL tile, -1 otherwise
};
constexpr int kClsShift = 30;
constexpr int32_t kKtMask = (1 << kClsShift) - 1;
#if defined(__HIPCC__)
#define MA_HD __host__ __device__
#else
#define MA_HD
#endif
MA_HD inline int32_t entry_kt(int32_t kt_cls) { return kt_cls & kKtMask; }
MA_HD inline int32_t entry_cls(int32_t kt_cls) { return (int32_t)((uint32_t)kt_cls >> kClsShift); }

}  // namespace maskattn

struct ma_plan {
  int32_t batch = 0, tile_q = 0, tile_k = 0;
  std::vector<int32_t> q_start, q_len, kv_len, nqt, nkt;
  std::vector<int64_t> tile_base;  // first global tile index of each sequence
  std::vector<int32_t> row_base;   // first global q-tile row of each sequence
  int32_t num_rows = 0;
  int64_t num_tiles = 0;
  int64_t total_q = 0;

  // host copy (host-compiled plans)
  bool host_valid = false;
  std::vector<maskattn::Item> items;
  std::vector<maskattn::Entry> entries;
  std::vector<uint64_t> words;
  int64_t num_wblk = 0;

  // device copy
  bool on_device = false;
  bool device_built = false;  // entries / word blocks laid out by the device classifier
  int device_id = -1;
  void *dbuf = nullptr;
  size_t dbytes = 0;       // bytes the plan's layout uses
  size_t dbuf_bytes = 0;   // bytes of the buffer (a reused buffer may be larger)
  size_t off_seqs = 0, off_aux = 0, off_items = 0, off_entries = 0, off_words = 0;
  size_t off_extra = 0;          // scratch after the words (device classification: class bytes)
  // pinned host staging of the last upload, kept until the plan is destroyed
  // so that uploads are stream-ordered without waiting for them
  void *staging = nullptr;
  size_t staging_bytes = 0;
  int64_t cap_entries = 0, cap_wblk = 0;

  // k-major transpose for the backward (built on first use): one item per
  // (sequence, k-tile), every k-tile included, entries (q-tile | class,
  // word block) in descending q-tile order, items most work first.
  void *kbuf = nullptr;
  size_t off_kitems = 0, off_kentries = 0;
  int32_t num_kitems = 0;
};

namespace maskattn {

ma_status set_error(ma_status st, const char *fmt, ...);
void clear_error();

// plan.cpp
ma_status validate_desc(const ma_mask_desc *d);
ma_status plan_shape(const ma_mask_desc *d, ma_plan *p);
ma_status compile_host(const ma_mask_desc *d, ma_plan *p);
ma_status plan_alloc_device(ma_plan *p, int64_t cap_entries, int64_t cap_wblk, size_t extra = 0);
// A pinned host buffer of at least `bytes` owned by the plan (p->staging).
ma_status plan_staging(ma_plan *p, size_t bytes);
ma_status plan_upload(ma_plan *p, void *stream);
void fill_seqinfo(const ma_plan *p, int32_t kind, std::vector<SeqInfo> &s, std::vector<SeqAux> &aux);
ma_status plan_fetch_host_view(const ma_plan *p, std::vector<Item> &items,
                               std::vector<Entry> &entries, std::vector<uint64_t> &words);
// Builds and uploads the k-major transpose (KItem.qt holds the k-tile; the
// entries' first field holds q-tile | class << 30).  Synchronises `stream`.
ma_status plan_build_kmajor(ma_plan *p, void *stream);
void plan_free_device(ma_plan *p);

// mask_classify.hip
ma_status launch_classify(ma_plan *p, const void *mask, int32_t kind, int64_t mask_numel, int32_t window,
                          void *stream);

// attn_fwd.hip
struct PrefillArgs {
  const ma_plan *plan;
  const void *q, *k, *v;
  int32_t hq, hkv, d, page_shift;
  int64_t s_page, s_slot, s_head;
  const int32_t *page_table;
  int32_t max_pages;
  int32_t in_dtype, out_dtype;
  float scale;
  void *out;
  float *lse;
  void *stream;
};
ma_status launch_prefill(const PrefillArgs &a);

// attn_fp8.hip
struct Fp8Args {
  const ma_plan *plan;
  const void *q, *k, *v;
  int32_t hq, hkv, d, page_shift;
  int64_t s_page, s_slot, s_head;
  const int32_t *page_table;
  int32_t max_pages;
  int32_t out_dtype;
  float scale, q_descale, k_descale, v_descale;
  void *out;
  float *lse;
  void *stream;
};
int32_t fp8_rows_per_gather(int32_t d);
ma_status launch_prefill_fp8(const Fp8Args &a);

// attn_bwd.hip
struct BackwardArgs {
  ma_plan *plan;
  const void *q, *k, *v, *o, *dout;
  const float *lse;
  int32_t hq, hkv, d, page_shift;
  int64_t total_q;
  int64_t s_page, s_slot, s_head;
  const int32_t *page_table;
  int32_t max_pages;
  int32_t o_dtype;
  float scale;
  float *dq, *dk, *dv;
  void *workspace;
  void *stream;
};
size_t backward_workspace(int64_t total_q, int32_t hq);
ma_status launch_backward(const BackwardArgs &a);

// verify.hip
struct VerifyArgs {
  const void *q, *k, *v;
  int32_t hq, hkv, d, page_shift;
  int64_t s_page, s_slot, s_head;
  const int32_t *page_table;
  int32_t max_pages;
  const int32_t *cu_seqlens_q, *kv_lens;
  int32_t batch, max_q, max_kv;
  int32_t mask_kind;
  const void *mask;
  int64_t mask_numel;
  int32_t window;              // SLIDING_WINDOW
  const int32_t *prefix_len;   // PREFIX_LM, device [batch]
  int32_t out_dtype;
  float scale;
  void *workspace;
  size_t ws_bytes;
  void *out;
  float *lse;
  void *stream;
  int32_t kv8;                 // 1: k / v hold e4m3 bytes, scaled by k_descale / v_descale
  float k_descale, v_descale;
};
size_t verify_workspace(int32_t batch, int32_t max_q, int32_t max_kv, int32_t hq, int32_t hkv,
                        int32_t d);
// The library's own scratch for attn_verify_tree_noalloc: kVerifyScratchBytes
// of device memory per GPU (a static device array), its address on the
// current device in *out.
constexpr size_t kVerifyScratchBytes = (size_t)64 << 20;
ma_status verify_scratch(void **out);
ma_status launch_verify(const VerifyArgs &a);

}  // namespace maskattn
