// Masked flash-attention prefill over a compiled plan (gfx950).
//
// One workgroup per (q-tile, query head).  The plan lists, per q-tile, the
// k-tiles that are not SKIP in ascending key order, each FULL or PARTIAL;
// SKIP tiles cost nothing (the block-sparse form flashinfer issue 724
// recommends).  A PARTIAL tile carries one 64-bit word per query row; each
// lane fetches its own row's word with one coalesced 8-byte load, prefetched
// one tile ahead, and masks its scores with shifts of that word.  The mask
// is thus never read per element from memory (the non-coalesced pattern
// that issue holds responsible for a custom mask taking roughly double the
// causal kernel's time).
//
// Per tile (64 keys), every wave owns 32 query rows:
//   paged K/V gather -> registers (one tile ahead) -> LDS (K row-major, V
//   transposed), S^T = K Q^T on bf16 matrix cores, mask, online softmax in
//   fp32 with exp2, O^T += V^T P^T on bf16 matrix cores.
// Two LDS stages, one barrier per tile.  The fp32 variant (fp32 inputs, fp32
// matrix cores, no bf16 rounding anywhere) keeps the same walk with a single
// stage.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "internal.h"
#include "kernels_common.h"
#include "tile_bf16.h"
#include "tile_dma_bf16.h"

namespace maskattn {
using namespace dev;
using namespace dev::staged;

namespace {

struct PrefillParams {
  const SeqInfo *seqs;
  const Item *items;
  const Entry *entries;
  const uint64_t *words;
  const void *q;
  const void *k;
  const void *v;
  const int32_t *page_table;
  void *out;
  float *lse;
  int64_t s_page, s_slot, s_head;
  int32_t max_pages, page_shift;
  int32_t hq, group;
  int32_t num_items;
  float scale;
  float scale_log2;
};

// Workgroup -> (work item, query head).  Workgroups are dispatched to the 8
// XCDs round-robin; when Hq is a multiple of 8, each XCD gets a contiguous
// block of Hq/8 query heads (so its L2 serves the K/V of few K/V heads) and
// walks the work items in plan order (most work first).  When an XCD would
// hold fewer query heads than a GQA group (Hq/8 < group), the r = group /
// (Hq/8) XCDs of one K/V head instead take all of that group's query heads,
// each XCD every r-th work item: the heads that read the same K/V tiles
// then run side by side behind one L2.  The grid is then padded to a
// multiple of r work items; padding workgroups get item >= num_items.
__device__ __forceinline__ void map_block(int b, int num_items, int hq, int group, int &item, int &h) {
  if ((hq & 7) == 0) {
    const int m = hq >> 3, x = b & 7, slot = b >> 3;
    if (m < group && group % m == 0) {
      const int r = group / m;
      item = (slot / group) * r + x % r;
      h = (x / r) * group + slot % group;
    } else {
      item = slot / m;
      h = x * m + slot % m;
    }
  } else {
    item = b / hq;
    h = b - item * hq;
  }
}

// m_ref is the softmax reference in log2 units (scale * log2 e applied); lt
// is the row's sum of probabilities relative to it.
template <int D, typename OutT>
__device__ __forceinline__ void epilogue(const PrefillParams &p, const f32x16 (&o)[D / 32], float m_ref,
                                         float lt, int64_t tok, int h, bool row_ok, int hi) {
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (!row_ok) return;
  store_row<D, OutT>((OutT *)p.out + (tok * p.hq + h) * D, o, inv, hi);
  if (p.lse && hi == 0) p.lse[tok * p.hq + h] = lt > 0.f ? (m_ref + __log2f(lt)) * kLn2 : neg_inf();
}

// ---------------------------------------------------------------------------
// bf16 inputs, bf16 matrix cores
// ---------------------------------------------------------------------------
// Two ways to move a tile's K/V from the paged cache into LDS:
//  * DMA (pages of at least 512 / d keys): global_load_lds writes the
//    swizzled, unpadded stage directly; page ids are scalar loads, one per
//    gather instruction.  No staging registers, no LDS stores.
//  * staged (any page size): per-thread loads into registers one tile ahead,
//    stored to the padded stage at the end of the tile.
// Both keep two stages and one barrier per tile and compute the same
// products in the same order, so their results are identical.
template <int D, int BQ, bool DMA>
struct Bf16Cfg {
  static constexpr int NW = BQ / 32;
  static constexpr int NT = NW * 64;
  static constexpr size_t STAGE_ELEMS = DMA ? (size_t)dma::Stage<D>::ELEMS : (size_t)Stage<D>::ELEMS;
  static constexpr size_t LDS_BYTES = 2 * STAGE_ELEMS * sizeof(uint16_t);
  static constexpr bool PIPE = DMA && D <= 128 && BQ == 128;
};

// Plan entries are read through the constant address space: uniform reads
// there are scalar loads, which neither wait for nor delay the gathers.
__device__ __forceinline__ Entry load_entry(const Entry *e, int i) {
  const __attribute__((address_space(4))) Entry *c = (const __attribute__((address_space(4))) Entry *)e;
  return Entry{c[i].kt_cls, c[i].wblk};
}

// Waves per SIMD: 2, or 3 for the pipelined d = 64 kernel (168 registers;
// its two spilled values are reloaded only after the loop), 1 for d = 256
// and 64-row tiles.
template <int D, int BQ, bool DMA>
constexpr int prefill_occupancy() {
  return D == 256 || BQ == 64 ? 1 : (D == 64 && DMA ? 3 : 2);
}

template <int D, int BQ, typename OutT, bool DMA>
__global__ __launch_bounds__(BQ * 2, (prefill_occupancy<D, BQ, DMA>())) void prefill_bf16_kernel(PrefillParams p) {
  using C = Bf16Cfg<D, BQ, DMA>;
  extern __shared__ __align__(16) uint16_t lds[];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  int item_idx, h;
  map_block(blockIdx.x, p.num_items, p.hq, p.group, item_idx, h);
  if (item_idx >= p.num_items) return;
  const Item it = p.items[item_idx];
  const SeqInfo sq = p.seqs[it.seq];
  const int g = h / p.group;
  const int wrow = wave * 32 + l32;  // row inside the q-tile
  const int row_local = it.qt * BQ + wrow;
  const bool row_ok = row_local < sq.q_len;
  const int64_t tok = (int64_t)sq.q_start + row_local;
  const int kv_len = sq.kv_len;

  bf16x8 qf[D / 16];
  load_q<D>(qf, (const uint16_t *)p.q + (tok * p.hq + h) * D, row_ok, hi);

  const uint16_t *kbase = (const uint16_t *)p.k + (int64_t)g * p.s_head;
  const uint16_t *vbase = (const uint16_t *)p.v + (int64_t)g * p.s_head;
  const int32_t *pt = p.page_table + (int64_t)it.seq * p.max_pages;

  auto load_word = [&](Entry e) -> uint64_t {
    if (entry_cls(e.kt_cls) != MA_TILE_PARTIAL) return 0ull;
    return p.words[(int64_t)e.wblk * BQ + wrow];
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n) oacc[n] = f32x16{};
  float m_ref = neg_inf();
  float lsum = 0.f;   // this lane's half of its row sum
  const float c = p.scale_log2;

  const int eb = it.ent_begin, ee = it.ent_end;
  uint64_t word_nxt = 0;
  if constexpr (C::PIPE) {
    // Software-pipelined over tiles: step j issues the products S^T of tile
    // j + 1 and, beside them, the masking and softmax of tile j, then
    // O^T += V^T P^T of tile j, so the vector work of one tile runs while the
    // matrix cores take the next tile's scores.  K of tile t is gathered at
    // step t - 2 and V at step t - 1: step j reads K(j + 1) from stage
    // (j + 1) % 2 and V(j) from stage j % 2 while the gathers write K(j + 2)
    // into stage j % 2 and V(j + 1) into stage (j + 1) % 2.  Each step ends
    // with a wait for this wave's gathers and a workgroup barrier.
    using KV = dma::KvDma<D, C::NW>;
    constexpr uint32_t SB = (uint32_t)dma::Stage<D>::BYTES, VB = 2u * dma::Stage<D>::V_OFF;
    constexpr int SE = dma::Stage<D>::ELEMS;
    const dma::LaneOffsets<D> lo(lane);
    const uint32_t lds0 = dma::lds_addr(lds);
    const int n = ee - eb;
    auto pages_of = [&](int j) { return KV::pages_uniform(pt, p.page_shift, entry_kt(load_entry(p.entries, eb + j).kt_cls), kv_len, wave); };
    using IsK = std::integral_constant<bool, false>;
    using IsV = std::integral_constant<bool, true>;
    const dma::LaneGather<D, C::NW, dma::SwzK<D>> lgk(wave, lane, p.s_slot);
    const dma::LaneGather<D, C::NW, dma::SwzV<D>> lgv(wave, lane, p.s_slot);
    const uint32_t page_bytes = (uint32_t)(p.s_page * 2), slot_bytes = (uint32_t)(p.s_slot * 2);
    // log2 of the keys one wave gathers per matrix and tile (RPI * IPW)
    constexpr int kPageRunShift = __builtin_ctz(KV::RPI * KV::IPW);
    auto gather = [&](auto is_v, const typename KV::Pages &pg, int j, uint32_t dst) {
      constexpr bool V = decltype(is_v)::value;
      const int kt = entry_kt(load_entry(p.entries, eb + j).kt_cls);
      auto go = [&](auto clamp) {
        constexpr bool CL = decltype(clamp)::value;
        if constexpr (V)
          dma::issue_mat_fast<D, C::NW, dma::SwzV<D>, CL>(vbase, pg, lgv, p.page_shift, page_bytes, slot_bytes, kt, kv_len,
                                                  dst, wave, lane);
        else
          dma::issue_mat_fast<D, C::NW, dma::SwzK<D>, CL>(kbase, pg, lgk, p.page_shift, page_bytes, slot_bytes, kt, kv_len,
                                                   dst, wave, lane);
      };
      if (kt * 64 + 64 <= kv_len) {
        if (p.page_shift >= kPageRunShift) {
          if constexpr (V)
            dma::issue_mat_page<D, C::NW, dma::SwzV<D>>(vbase, pg.id[0], lgv, p.page_shift, page_bytes, slot_bytes, kt, dst,
                                                wave);
          else
            dma::issue_mat_page<D, C::NW, dma::SwzK<D>>(kbase, pg.id[0], lgk, p.page_shift, page_bytes, slot_bytes, kt, dst,
                                                 wave);
        } else {
          go(std::integral_constant<bool, false>{});
        }
      } else {
        go(std::integral_constant<bool, true>{});
      }
    };
    typename KV::Pages pg_a, pg_b;   // pages of tiles j + 2 and j + 1 at the start of step j
    uint64_t word_cur = 0;
    f32x16 sa[2], sb[2];
    if (n > 0) {
      const typename KV::Pages pg0 = pages_of(0);
      gather(IsK{}, pg0, 0, lds0);
      gather(IsV{}, pg0, 0, lds0 + VB);
      word_cur = load_word(load_entry(p.entries, eb));
      if (n > 1) {
        pg_b = pages_of(1);
        gather(IsK{}, pg_b, 1, lds0 + SB);
        word_nxt = load_word(load_entry(p.entries, eb + 1));
        if (n > 2) pg_a = pages_of(2);
      }
      dma::wait_vmem();
      __syncthreads();
      dma::qk_tile<D, (D > 64 ? 4 : D / 16)>(lds, lo, qf, sa);
      if (n > 2) __syncthreads();   // every wave has read K(0) before K(2) replaces it
    }
    auto step = [&](f32x16 (&scur)[2], f32x16 (&snxt)[2], int j) {
      const int cur = j & 1;
      const Entry ec = load_entry(p.entries, eb + j);
      const uint64_t wcur = word_cur;
      if (j + 2 < n) gather(IsK{}, pg_a, j + 2, lds0 + (uint32_t)cur * SB);
      if (j + 1 < n) gather(IsV{}, pg_b, j + 1, lds0 + (uint32_t)(cur ^ 1) * SB + VB);
      word_cur = word_nxt;
      if (j + 2 < n) {
        word_nxt = load_word(load_entry(p.entries, eb + j + 2));
        pg_b = pg_a;
        if (j + 3 < n) pg_a = pages_of(j + 3);
      }
      const int kt = entry_kt(ec.kt_cls);
      const int cls = entry_cls(ec.kt_cls);
      const int kin = kv_len - kt * 64;
      if (cls == MA_TILE_PARTIAL || kin < 64)
        apply_word(scur, (cls == MA_TILE_PARTIAL ? wcur : ~0ull) & low_bits(kin), hi);
      // unconditional (at the last step the result is unused): a branch here
      // would split the products from the softmax they are to overlap
      dma::qk_tile_free<D>(lds + (cur ^ 1) * SE, lo, qf, snxt);
      float alpha, ps;
      const bool any = softmax_tile(scur, m_ref, c, alpha);
      bf16x8 pb[4];
      dma::pack_p(scur, pb, ps);
      // P is complete here, in the same block as the products above: without
      // this the exponentials sink past the rescale branch below and run
      // after the products instead of beside them
      asm volatile("" : "+v"(pb[0]), "+v"(pb[1]), "+v"(pb[2]), "+v"(pb[3]), "+v"(ps));
      if (any) {
#pragma unroll
        for (int x = 0; x < D / 32; ++x) oacc[x] *= alpha;
        lsum *= alpha;
      }
      lsum += ps;
      dma::pv_tile_packed<D>(lds + cur * SE, lo, pb, oacc);
      dma::wait_vmem();
      __syncthreads();
    };
    for (int j = 0; j < n; j += 2) {
      step(sa, sb, j);
      if (j + 1 < n) step(sb, sa, j + 1);
    }
  } else if constexpr (DMA) {
    using KV = dma::KvDma<D, C::NW>;
    const dma::LaneOffsets<D> lo(lane);
    const uint32_t lds0 = dma::lds_addr(lds);
    typename KV::Pages pg_nxt;
    [[maybe_unused]] const dma::LaneGather<D, C::NW, dma::SwzK<D>> lgk(wave, lane, p.s_slot);
    [[maybe_unused]] const dma::LaneGather<D, C::NW, dma::SwzV<D>> lgv(wave, lane, p.s_slot);
    [[maybe_unused]] const uint32_t page_bytes = (uint32_t)(p.s_page * 2), slot_bytes = (uint32_t)(p.s_slot * 2);
    constexpr int kPageRunShift = __builtin_ctz(KV::RPI * KV::IPW);
    auto issue_tile = [&](const typename KV::Pages &pg, int kt, uint32_t st) {
      const uint32_t sv = st + 2u * dma::Stage<D>::V_OFF;
      if constexpr (D > 128) {
        // d = 256 keeps the per-lane form: the constant offsets' registers
        // cost it more than the vector arithmetic they save (measured +3%)
        KV::issue(kbase, vbase, pg, p.page_shift, p.s_page, p.s_slot, kt, kv_len, st, wave, lane);
        return;
      }
      if (kt * 64 + 64 <= kv_len) {
        if (p.page_shift >= kPageRunShift) {
          dma::issue_mat_page<D, C::NW, dma::SwzK<D>>(kbase, pg.id[0], lgk, p.page_shift, page_bytes, slot_bytes, kt, st, wave);
          dma::issue_mat_page<D, C::NW, dma::SwzV<D>>(vbase, pg.id[0], lgv, p.page_shift, page_bytes, slot_bytes, kt, sv, wave);
        } else {
          dma::issue_mat_fast<D, C::NW, dma::SwzK<D>, false>(kbase, pg, lgk, p.page_shift, page_bytes, slot_bytes, kt, kv_len, st, wave, lane);
          dma::issue_mat_fast<D, C::NW, dma::SwzV<D>, false>(vbase, pg, lgv, p.page_shift, page_bytes, slot_bytes, kt, kv_len, sv, wave, lane);
        }
      } else {
        dma::issue_mat_fast<D, C::NW, dma::SwzK<D>, true>(kbase, pg, lgk, p.page_shift, page_bytes, slot_bytes, kt, kv_len, st, wave, lane);
        dma::issue_mat_fast<D, C::NW, dma::SwzV<D>, true>(vbase, pg, lgv, p.page_shift, page_bytes, slot_bytes, kt, kv_len, sv, wave, lane);
      }
    };
    if (eb < ee) {
      const Entry e0 = load_entry(p.entries, eb);
      const int kt0 = entry_kt(e0.kt_cls);
      const typename KV::Pages pg0 = KV::pages_uniform(pt, p.page_shift, kt0, kv_len, wave);
      issue_tile(pg0, kt0, lds0);
      word_nxt = load_word(e0);
      if (eb + 1 < ee)
        pg_nxt = KV::pages_uniform(pt, p.page_shift, entry_kt(load_entry(p.entries, eb + 1).kt_cls), kv_len, wave);
      dma::wait_vmem();
      __syncthreads();
    }
    for (int e = eb; e < ee; ++e) {
      const int cur = (e - eb) & 1;
      const Entry ec = load_entry(p.entries, e);
      const uint64_t wcur = word_nxt;
      if (e + 1 < ee) {
        const Entry en = load_entry(p.entries, e + 1);
        issue_tile(pg_nxt, entry_kt(en.kt_cls), lds0 + (uint32_t)((cur ^ 1) * dma::Stage<D>::BYTES));
        word_nxt = load_word(en);
        if (e + 2 < ee)
          pg_nxt = KV::pages_uniform(pt, p.page_shift, entry_kt(load_entry(p.entries, e + 2).kt_cls), kv_len, wave);
      }
      const uint16_t *stage = lds + cur * dma::Stage<D>::ELEMS;
      f32x16 sacc[2];
      dma::qk_tile<D>(stage, lo, qf, sacc);
      {
        const int kt = entry_kt(ec.kt_cls);
        const int cls = entry_cls(ec.kt_cls);
        const int kin = kv_len - kt * 64;
        if (cls == MA_TILE_PARTIAL || kin < 64)
          apply_word(sacc, (cls == MA_TILE_PARTIAL ? wcur : ~0ull) & low_bits(kin), hi);
        float alpha;
        if (softmax_tile(sacc, m_ref, c, alpha)) {
#pragma unroll
          for (int n = 0; n < D / 32; ++n) oacc[n] *= alpha;
          lsum *= alpha;
        }
      }
      dma::pv_tile<D>(stage, lo, sacc, oacc, lsum);
      dma::wait_vmem();
      __syncthreads();
    }
  } else {
    using KV = KvTile<D, C::NT>;
    KV kv;
    typename KV::Pages pg_nxt;
    if (eb < ee) {
      const Entry e0 = load_entry(p.entries, eb);
      const int kt0 = entry_kt(e0.kt_cls);
      const typename KV::Pages pg0 = kv.pages(pt, p.page_shift, kt0, kv_len, tid);
      kv.load(kbase, vbase, pg0, p.page_shift, p.s_page, p.s_slot, kt0, kv_len, tid);
      word_nxt = load_word(e0);
      if (eb + 1 < ee) pg_nxt = kv.pages(pt, p.page_shift, entry_kt(load_entry(p.entries, eb + 1).kt_cls), kv_len, tid);
      kv.store(lds, tid);
      __syncthreads();
    }
    // d = 256 stages K and V of the next tile one after the other (K during
    // Q K^T and the softmax, V during P V) to halve the staging registers.
    constexpr bool kSplit = D == 256;
    for (int e = eb; e < ee; ++e) {
      const int cur = (e - eb) & 1;
      const Entry ec = load_entry(p.entries, e);
      const uint64_t wcur = word_nxt;
      const bool has_next = e + 1 < ee;
      int kt_next = 0;
      typename KV::Pages pg_use = pg_nxt;
      if (has_next) {
        const Entry en = load_entry(p.entries, e + 1);
        kt_next = entry_kt(en.kt_cls);
        if (kSplit)
          kv.load_one(kbase, pg_use, p.page_shift, p.s_page, p.s_slot, kt_next, kv_len, tid);
        else
          kv.load(kbase, vbase, pg_use, p.page_shift, p.s_page, p.s_slot, kt_next, kv_len, tid);
        word_nxt = load_word(en);
        if (e + 2 < ee) pg_nxt = kv.pages(pt, p.page_shift, entry_kt(load_entry(p.entries, e + 2).kt_cls), kv_len, tid);
      }
      const uint16_t *stage = lds + cur * Stage<D>::ELEMS;
      uint16_t *next = lds + (cur ^ 1) * Stage<D>::ELEMS;
      f32x16 sacc[2];
      qk_tile<D>(stage, qf, sacc, l32, hi);
      {
        const int kt = entry_kt(ec.kt_cls);
        const int cls = entry_cls(ec.kt_cls);
        const int kin = kv_len - kt * 64;
        if (cls == MA_TILE_PARTIAL || kin < 64)
          apply_word(sacc, (cls == MA_TILE_PARTIAL ? wcur : ~0ull) & low_bits(kin), hi);
        float alpha;
        if (softmax_tile(sacc, m_ref, c, alpha)) {
#pragma unroll
          for (int n = 0; n < D / 32; ++n) oacc[n] *= alpha;
          lsum *= alpha;
        }
      }
      if (kSplit && has_next) {
        kv.store_one(next, Stage<D>::KS, tid);
        kv.load_one(vbase, pg_use, p.page_shift, p.s_page, p.s_slot, kt_next, kv_len, tid);
      }
      pv_tile<D>(stage, sacc, oacc, lsum, l32, hi);
      if (has_next) {
        if (kSplit)
          kv.store_one(next + Stage<D>::V_OFF, Stage<D>::VS, tid);
        else
          kv.store(next, tid);
      }
      __syncthreads();
    }
  }
  epilogue<D, OutT>(p, oacc, m_ref, sum_halves(lsum), tok, h, row_ok, hi);
}

// ---------------------------------------------------------------------------
// fp32 inputs, fp32 matrix cores (v_mfma_f32_32x32x2_f32)
// ---------------------------------------------------------------------------
template <int D, int BQ>
struct F32Cfg {
  static constexpr int NW = BQ / 32;
  static constexpr int NT = NW * 64;
  static constexpr int KS = D + 1;   // odd stride: column reads are conflict-free
  static constexpr int VS = D + 4;
  static constexpr int CH = D / 4;   // 16-byte chunks per key row
  static constexpr int CHUNKS = 64 * CH;
  static constexpr size_t LDS_BYTES = (64 * KS + 64 * VS) * sizeof(float);
};

template <int D, int BQ>
__global__ __launch_bounds__(BQ * 2, 1) void prefill_f32_kernel(PrefillParams p) {
  using C = F32Cfg<D, BQ>;
  extern __shared__ __align__(16) float ldsf[];
  float *Ks = ldsf;
  float *Vs = ldsf + 64 * C::KS;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  int item_idx, h;
  map_block(blockIdx.x, p.num_items, p.hq, p.group, item_idx, h);
  if (item_idx >= p.num_items) return;
  const Item it = p.items[item_idx];
  const SeqInfo sq = p.seqs[it.seq];
  const int g = h / p.group;
  const int row_local = it.qt * BQ + wave * 32 + l32;
  const bool row_ok = row_local < sq.q_len;
  const int64_t tok = (int64_t)sq.q_start + row_local;
  const int kv_len = sq.kv_len;

  float qf[D / 2];
  {
    const float *qb = (const float *)p.q + (tok * p.hq + h) * D + hi;
#pragma unroll
    for (int s = 0; s < D / 2; ++s) qf[s] = row_ok ? qb[2 * s] : 0.f;
  }
  const float *kbase = (const float *)p.k + (int64_t)g * p.s_head;
  const float *vbase = (const float *)p.v + (int64_t)g * p.s_head;
  const int32_t *pt = p.page_table + (int64_t)it.seq * p.max_pages;
  const int pmask = (1 << p.page_shift) - 1;
  const int wrow = wave * 32 + l32;

  f32x16 oacc[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n) oacc[n] = f32x16{};
  float m_ref = neg_inf(), l_run = 0.f;
  const float c = p.scale_log2;

  for (int e = it.ent_begin; e < it.ent_end; ++e) {
    const Entry ec = load_entry(p.entries, e);
    const int kt = entry_kt(ec.kt_cls);
    const int cls = entry_cls(ec.kt_cls);
    __syncthreads();  // previous tile fully consumed
    for (int idx = tid; idx < C::CHUNKS; idx += C::NT) {
      const int key = idx / C::CH, ch = idx % C::CH;
      const int kk = kt * 64 + key;
      f32x4 kv4 = {0.f, 0.f, 0.f, 0.f}, vv4 = {0.f, 0.f, 0.f, 0.f};
      if (kk < kv_len) {
        const int32_t page = pt[kk >> p.page_shift];
        const int64_t off = (int64_t)page * p.s_page + (int64_t)(kk & pmask) * p.s_slot + 4 * ch;
        kv4 = *(const f32x4 *)(kbase + off);
        vv4 = *(const f32x4 *)(vbase + off);
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) Ks[key * C::KS + 4 * ch + x] = kv4[x];
      *(f32x4 *)(Vs + key * C::VS + 4 * ch) = vv4;
    }
    const uint64_t word = cls == MA_TILE_PARTIAL ? p.words[(int64_t)ec.wblk * BQ + wrow] : ~0ull;
    __syncthreads();

    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s = 0; s < D / 2; ++s)
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[(32 * kb + l32) * C::KS + 2 * s + hi], qf[s],
                                                       sacc[kb], 0, 0, 0);
    const int kin = kv_len - kt * 64;
    if (cls == MA_TILE_PARTIAL || kin < 64) apply_word(sacc, word & low_bits(kin), hi);
    float alpha;
    const bool any = softmax_tile(sacc, m_ref, c, alpha);
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) ps += sacc[0][r] + sacc[1][r];
    l_run = l_run * alpha + ps;
    if (any) {
#pragma unroll
      for (int n = 0; n < D / 32; ++n) oacc[n] *= alpha;
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
#pragma unroll
        for (int n = 0; n < D / 32; ++n)
          oacc[n] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * C::VS + 32 * n + l32], sacc[kb][r], oacc[n],
                                                         0, 0, 0);
      }
  }
  epilogue<D, float>(p, oacc, m_ref, sum_halves(l_run), tok, h, row_ok, hi);
}

template <typename K>
ma_status launch_kernel(K kernel, int grid, int block, size_t lds, const PrefillParams &prm, void *stream) {
  hipError_t e = hipSuccess;
  if (lds > 64 * 1024) e = hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return set_error(MA_ERR_HIP, "hipFuncSetAttribute: %s", hipGetErrorString(e));
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(block), lds, (hipStream_t)stream, prm);
  e = hipGetLastError();
  if (e != hipSuccess) return set_error(MA_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return MA_OK;
}

template <int D, int BQ, bool DMA>
ma_status dispatch_bf16_mode(const PrefillArgs &a, const PrefillParams &prm, int grid) {
  using C = Bf16Cfg<D, BQ, DMA>;
  if (a.out_dtype == MA_F32)
    return launch_kernel(prefill_bf16_kernel<D, BQ, float, DMA>, grid, C::NT, C::LDS_BYTES, prm, a.stream);
  return launch_kernel(prefill_bf16_kernel<D, BQ, uint16_t, DMA>, grid, C::NT, C::LDS_BYTES, prm, a.stream);
}

// The direct gather needs the key rows of one gather instruction (512 / d of
// them) inside one page, and a page's bytes addressable by a 32-bit offset.
template <int D, int BQ>
ma_status dispatch_bf16(const PrefillArgs &a, const PrefillParams &prm, int grid) {
  const bool fits = ((int64_t)1 << a.page_shift) * a.s_slot * 2 < ((int64_t)1 << 31) &&
                    a.s_page * 2 < ((int64_t)1 << 32);
  if ((1 << a.page_shift) >= dma::KvDma<D, BQ / 32>::RPI && fits) return dispatch_bf16_mode<D, BQ, true>(a, prm, grid);
  return dispatch_bf16_mode<D, BQ, false>(a, prm, grid);
}

template <int D, int BQ>
ma_status dispatch_f32(const PrefillArgs &a, const PrefillParams &prm, int grid) {
  using C = F32Cfg<D, BQ>;
  return launch_kernel(prefill_f32_kernel<D, BQ>, grid, C::NT, C::LDS_BYTES, prm, a.stream);
}

}  // namespace

ma_status launch_prefill(const PrefillArgs &a) {
  const ma_plan *pl = a.plan;
  PrefillParams prm{};
  const char *base = (const char *)pl->dbuf;
  prm.seqs = (const SeqInfo *)(base + pl->off_seqs);
  prm.items = (const Item *)(base + pl->off_items);
  prm.entries = (const Entry *)(base + pl->off_entries);
  prm.words = (const uint64_t *)(base + pl->off_words);
  prm.q = a.q;
  prm.k = a.k;
  prm.v = a.v;
  prm.page_table = a.page_table;
  prm.out = a.out;
  prm.lse = a.lse;
  prm.s_page = a.s_page;
  prm.s_slot = a.s_slot;
  prm.s_head = a.s_head;
  prm.max_pages = a.max_pages;
  prm.page_shift = a.page_shift;
  prm.hq = a.hq;
  prm.group = a.hq / a.hkv;
  prm.num_items = pl->num_rows;
  prm.scale = a.scale;
  prm.scale_log2 = a.scale * kLog2e;
  // work items padded for map_block's K/V-group mapping
  int64_t items = pl->num_rows;
  if (a.hq % 8 == 0 && a.hq / 8 < prm.group && prm.group % (a.hq / 8) == 0) {
    const int64_t r = prm.group / (a.hq / 8);
    items = (items + r - 1) / r * r;
  }
  const int64_t grid64 = items * a.hq;
  if (grid64 > INT32_MAX) return set_error(MA_ERR_UNSUPPORTED, "grid too large");
  const int grid = (int)grid64;
  const bool bq128 = pl->tile_q == 128;
  if (a.in_dtype == MA_BF16) {
    switch (a.d) {
      case 64: return bq128 ? dispatch_bf16<64, 128>(a, prm, grid) : dispatch_bf16<64, 64>(a, prm, grid);
      case 128: return bq128 ? dispatch_bf16<128, 128>(a, prm, grid) : dispatch_bf16<128, 64>(a, prm, grid);
      case 256: return bq128 ? dispatch_bf16<256, 128>(a, prm, grid) : dispatch_bf16<256, 64>(a, prm, grid);
    }
  } else {
    switch (a.d) {
      case 64: return bq128 ? dispatch_f32<64, 128>(a, prm, grid) : dispatch_f32<64, 64>(a, prm, grid);
      case 128: return bq128 ? dispatch_f32<128, 128>(a, prm, grid) : dispatch_f32<128, 64>(a, prm, grid);
    }
  }
  return set_error(MA_ERR_UNSUPPORTED, "no kernel for dtype %d, head_dim %d", a.in_dtype, a.d);
}

}  // namespace maskattn
