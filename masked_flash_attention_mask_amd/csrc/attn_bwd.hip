// Backward of masked flash-attention over a compiled plan (gfx950): dQ, dK
// and dV of O = softmax(scale Q K^T + mask) V over ragged sequences and paged
// K/V, reusing the forward's LSE.  With P = exp(S - LSE) on visible entries,
//   D = rowsum(dO * O),  dP = dO V^T,  dS = P (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO
// (a K/V head sums its query heads).  Deterministic, without atomics:
//  * bwd_prep:  D and LSE in log2 units per (query, head).
//  * bwd_dq:    one workgroup per (q-tile, query head) walks the plan's row
//               of k-tiles, like the forward: S^T = K Q^T, dP^T = V dO^T,
//               dQ^T += K^T dS^T (lane = query row).
//  * bwd_dkdv:  one workgroup per (k-tile, K/V head) walks the plan's k-major
//               transpose (every q-tile that sees the tile, every query head
//               of the group, 32-query blocks): S = Q K^T, dP = dO V^T,
//               dV^T += dO^T P, dK^T += Q^T dS (lane = key); every key below
//               kv_len is written once (0 when no query sees it).
// Masking is the forward's: a PARTIAL tile's row words, keys past kv_len.
// Matrix products are bf16 with fp32 accumulation (P and dS rounded to bf16
// for their products); gradients are written in fp32.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "kernels_common.h"
#include "tile_bf16.h"
#include "tile_dma_bf16.h"

namespace maskattn {
using namespace dev;

namespace {

__device__ __forceinline__ bf16x8 to_bf16x8(const f32x16 &s, int half) {
  f32x8 v;
#pragma unroll
  for (int x = 0; x < 8; ++x) v[x] = s[8 * half + x];
  return __builtin_convertvector(v, bf16x8);
}

struct BwdParams {
  const SeqInfo *seqs;
  const Item *items;     // forward rows (dQ)
  const Entry *entries;
  const Item *kitems;    // k-major items: seq, k-tile, entries (dK / dV)
  const Entry *kentries; // q-tile | class << 30, word block
  const uint64_t *words;
  const uint16_t *q, *k, *v, *dout;
  const void *o;
  const float *lse;
  float *dq, *dk, *dv;
  float *dd, *l2;        // workspace: D and LSE * log2 e per (token, head)
  const int32_t *page_table;
  int64_t s_page, s_slot, s_head;
  int64_t total_q;
  int32_t max_pages, page_shift;
  int32_t hq, group, num_items, num_kitems, tile_q, o_f32;
  float scale, scale_log2;
};

// One 64-row block of Q or dO in LDS: dense rows of D bf16, 16-byte chunks
// XOR swizzled by the row so that both the row reads (ds_read_b128 over 16
// rows, one chunk each) and the transposed reads (ds_read_b64_tr_b16 over 4
// rows x 4 chunks per half wave) hit distinct banks.  f is a bijection of the
// row's low bits that keeps 16 consecutive rows on distinct chunks and puts
// the 4 rows of a transposed read into distinct 4-chunk groups.
template <int D>
struct QBlk {
  static constexpr int CH = D / 8;
  static constexpr int ELEMS = 64 * D;
  __host__ __device__ static constexpr int f(int r) {
    return CH >= 16 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }
  static constexpr int META = 2 * ELEMS;          // element offset of the row metadata
  static constexpr int STAGE = META + 4 * 64 * 2;  // Q, dO, then l2, dd, word low, word high (64 x 4 bytes each)
  static constexpr size_t BYTES = 2 * STAGE * sizeof(uint16_t);   // two stages
};

__device__ __forceinline__ void lds_load4(const void *src, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}

__device__ __forceinline__ Entry load_entry(const Entry *e, int i) {
  const __attribute__((address_space(4))) Entry *c = (const __attribute__((address_space(4))) Entry *)e;
  return Entry{c[i].kt_cls, c[i].wblk};
}

using dma::gptr_t;

// Direct global -> LDS load of 4 bytes per lane with a scalar base and a
// 32-bit per-lane byte offset: lane l writes LDS address m0 + 4 l.  See
// dma::lds_load16 for how the kernels order them.
using dma::lds_load16_s;
__device__ __forceinline__ void lds_load4_s(gptr_t base, uint32_t voff, uint32_t m0) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "{m0}"(m0) : "memory");
}

// ---------------------------------------------------------------------------
// D[t, h] = <dO[t, h], O[t, h]>, L2[t, h] = LSE[t, h] log2 e (+inf for a row
// with no visible key, so that its probabilities come out exactly 0).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_prep(BwdParams p) {
  // D / 8 lanes per (token, head) row, 8 elements (16 bytes of dO) per lane;
  // 256 / (D / 8) rows per workgroup
  constexpr int LPR = D / 8, RPB = 256 / LPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int c = (threadIdx.x % LPR) * 8;
  float acc = 0.f;
  if (row < p.total_q * p.hq) {
    const u32x4 g = *(const u32x4 *)(p.dout + row * D + c);
    float o[8];
    if (p.o_f32) {
      const f32x4 a = *(const f32x4 *)((const float *)p.o + row * D + c);
      const f32x4 b = *(const f32x4 *)((const float *)p.o + row * D + c + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[i] = a[i];
        o[4 + i] = b[i];
      }
    } else {
      const u32x4 ob = *(const u32x4 *)((const uint16_t *)p.o + row * D + c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[2 * i] = __uint_as_float(ob[i] << 16);
        o[2 * i + 1] = __uint_as_float(ob[i] & 0xFFFF0000u);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc += o[2 * i] * __uint_as_float(g[i] << 16);
      acc += o[2 * i + 1] * __uint_as_float(g[i] & 0xFFFF0000u);
    }
  }
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, LPR);
  if (row < p.total_q * p.hq && threadIdx.x % LPR == 0) {
    p.dd[row] = acc;
    const float lse = p.lse[row];
    p.l2[row] = lse == neg_inf() ? __builtin_inff() : lse * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (q-tile, query head), BQ / 32 waves x 32 query rows
// (Q and dO rows held as B operands).  The K / V tiles of the plan's row are
// gathered straight into LDS (global_load_lds) one tile ahead into two
// alternating stages, both swizzled like a query block, so the row reads of
// K and V (the A operands of S^T and dP^T) and the transposed reads of K (the
// A operand of dQ^T) are free of bank conflicts.
// ---------------------------------------------------------------------------
// FAST (pages of at least 512 / D keys, a page's bytes below 2^32 and
// page_size * slot stride below 2^31): page ids by scalar loads and, for
// tiles inside kv_len, a scalar page-and-slot base with per-lane constant
// offsets (the forward's gather); otherwise a 64-bit address per lane.
template <int D>
struct SwzQ {
  __device__ static constexpr int f(int r) { return QBlk<D>::f(r); }
};

// Waves per SIMD of the dQ kernel: two for 128-row tiles at d <= 128; one
// for 64-row tiles and at d = 256 (Q, dO and the dQ accumulators of a 32-row
// block take 256 registers per lane there).
template <int D, int BQ>
constexpr int dq_occupancy() {
  return BQ == 128 && D <= 128 ? 2 : 1;
}

template <int D, int BQ, bool FAST>
__global__ __launch_bounds__(BQ * 2, (dq_occupancy<D, BQ>())) void bwd_dq(BwdParams p) {
  using QB = QBlk<D>;
  constexpr int NW = BQ / 32, CH = D / 8, NI = CH / NW;   // gather instructions per wave per matrix
  constexpr int TILE = 64 * D;                             // elements of one 64-key matrix
  extern __shared__ __align__(16) uint16_t lds[];          // [2 stages][K tile, V tile]
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int item_idx = blockIdx.x / p.hq, h = blockIdx.x - item_idx * p.hq;
  const Item it = p.items[item_idx];
  const SeqInfo sq = p.seqs[it.seq];
  const int g = h / p.group;
  const int wrow = wave * 32 + l32;
  const int row_local = it.qt * BQ + wrow;
  const bool row_ok = row_local < sq.q_len;
  const int64_t tok = (int64_t)sq.q_start + row_local;
  const int kv_len = sq.kv_len;

  bf16x8 qf[D / 16], dof[D / 16];
  load_q<D>(qf, p.q + (tok * p.hq + h) * D, row_ok, hi);
  load_q<D>(dof, p.dout + (tok * p.hq + h) * D, row_ok, hi);
  const float l2 = row_ok ? p.l2[tok * p.hq + h] : __builtin_inff();
  const float dd = row_ok ? p.dd[tok * p.hq + h] : 0.f;
  const float c = p.scale_log2;

  const uint16_t *kbase = p.k + (int64_t)g * p.s_head;
  const uint16_t *vbase = p.v + (int64_t)g * p.s_head;
  const int32_t *pt = p.page_table + (int64_t)it.seq * p.max_pages;
  const int pmask = (1 << p.page_shift) - 1;
  // Gather: instruction t of a matrix fills LDS chunks [64 t, 64 t + 64);
  // lane l of it loads key row (64 t + l) / CH, logical chunk ((64 t + l) %
  // CH) ^ f(row).  Keys past kv_len repeat the last key (masked to 0).
  using KV = dma::KvDma<D, NW>;
  static_assert(KV::IPW == NI, "gather geometry");
  typename KV::Pages pg;
  [[maybe_unused]] const dma::LaneGather<D, NW, SwzQ<D>> lg(wave, lane, p.s_slot);
  [[maybe_unused]] const uint32_t page_bytes = (uint32_t)(p.s_page * 2), slot_bytes = (uint32_t)(p.s_slot * 2);
  [[maybe_unused]] const uint32_t lds_b = dma::lds_addr(lds);
  auto pages = [&](int kt) {
    if constexpr (FAST) {
      pg = KV::pages_uniform(pt, p.page_shift, kt, kv_len, wave);
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int r = (64 * (wave * NI + i) + lane) / CH;
        pg.id[i] = pt[min(kt * 64 + r, kv_len - 1) >> p.page_shift];
      }
    }
  };
  auto issue = [&](int kt, int sl) {
    uint16_t *st = lds + sl * 2 * TILE;
    if constexpr (FAST) {
      const uint32_t sk = lds_b + (uint32_t)(sl * 2 * TILE * 2), sv = sk + (uint32_t)(TILE * 2);
      if (kt * 64 + 64 <= kv_len) {
        if (p.page_shift >= __builtin_ctz(KV::RPI * KV::IPW)) {
          dma::issue_mat_page<D, NW, SwzQ<D>>(kbase, pg.id[0], lg, p.page_shift, page_bytes, slot_bytes, kt, sk, wave);
          dma::issue_mat_page<D, NW, SwzQ<D>>(vbase, pg.id[0], lg, p.page_shift, page_bytes, slot_bytes, kt, sv, wave);
        } else {
          dma::issue_mat_fast<D, NW, SwzQ<D>, false>(kbase, pg, lg, p.page_shift, page_bytes, slot_bytes, kt, kv_len,
                                                     sk, wave, lane);
          dma::issue_mat_fast<D, NW, SwzQ<D>, false>(vbase, pg, lg, p.page_shift, page_bytes, slot_bytes, kt, kv_len,
                                                     sv, wave, lane);
        }
      } else {
        dma::issue_mat_fast<D, NW, SwzQ<D>, true>(kbase, pg, lg, p.page_shift, page_bytes, slot_bytes, kt, kv_len, sk,
                                                  wave, lane);
        dma::issue_mat_fast<D, NW, SwzQ<D>, true>(vbase, pg, lg, p.page_shift, page_bytes, slot_bytes, kt, kv_len, sv,
                                                  wave, lane);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int t = wave * NI + i;
        const int pos = 64 * t + lane, r = pos / CH, pc = pos % CH;
        const int key = min(kt * 64 + r, kv_len - 1);
        const int64_t off = (int64_t)pg.id[i] * p.s_page + (int64_t)(key & pmask) * p.s_slot + 8 * (pc ^ QB::f(r));
        dma::lds_load16(kbase + off, dma::lds_addr(st + 512 * t));
        dma::lds_load16(vbase + off, dma::lds_addr(st + TILE + 512 * t));
      }
    }
  };
  // Row reads (K, V rows 32 kb + l32, chunk 2 k + hi) and transposed reads
  // (K rows 16 u + j (+ 8), columns 32 n + ...) in the swizzled layout.
  const int rx = 8 * (hi ^ QB::f(l32));
  const int j = 4 * hi + ((lane & 15) >> 2);
  const int cb = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tax = 8 * (cb ^ QB::f(j)) + 4 * (lane & 1);
  const int tbx = 8 * (cb ^ QB::f(j + 8)) + 4 * (lane & 1);
  auto tr_read = [&](const uint16_t *m, int u, int n) -> bf16x8 {
    const uint16_t *b = m + (j + 16 * u) * D;
    const i16x4 r0 =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(b + ((32 * n) ^ tax)));
    const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4 *)(b + 8 * D + ((32 * n) ^ tbx)));
    const i16x8 v = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
    return __builtin_bit_cast(bf16x8, v);
  };

  f32x16 dqacc[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n) dqacc[n] = f32x16{};

  const int eb = it.ent_begin, ee = it.ent_end;
  auto load_word = [&](Entry e) -> uint64_t {
    return entry_cls(e.kt_cls) == MA_TILE_PARTIAL ? p.words[(int64_t)e.wblk * BQ + wrow] : 0ull;
  };
  if (eb < ee) {
    const Entry e0 = load_entry(p.entries, eb);
    pages(entry_kt(e0.kt_cls));
    issue(entry_kt(e0.kt_cls), 0);
    uint64_t word_nxt = load_word(e0);
    if (eb + 1 < ee) pages(entry_kt(load_entry(p.entries, eb + 1).kt_cls));
    for (int e = eb; e < ee; ++e) {
      const int cur = (e - eb) & 1;
      dma::wait_vmem();
      __syncthreads();   // tile e is in stage cur; every wave is done with stage cur ^ 1
      const Entry ec = load_entry(p.entries, e);
      const uint64_t wcur = word_nxt;
      if (e + 1 < ee) {
        const Entry en = load_entry(p.entries, e + 1);
        issue(entry_kt(en.kt_cls), cur ^ 1);
        word_nxt = load_word(en);
        if (e + 2 < ee) pages(entry_kt(load_entry(p.entries, e + 2).kt_cls));
      }
      const uint16_t *ks = lds + cur * 2 * TILE;
      const uint16_t *vs = ks + TILE;
      // S^T = K Q^T (64 keys x this wave's 32 query rows), then dP^T = V dO^T
      // with P = exp2(S c - L2) computed beside it; operands of step k + 1
      // are read while step k's products run.
      const int kt = entry_kt(ec.kt_cls), cls = entry_cls(ec.kt_cls);
      const int kin = kv_len - kt * 64;
      f32x16 sacc[2], dpacc[2];
      {
        bf16x8 ka[2][2];
        auto read_k = [&](int k, int sl) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            ka[sl][kb] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(ks + (32 * kb + l32) * D + ((16 * k) ^ rx)));
        };
        read_k(0, 0);
#pragma unroll
        for (int k = 0; k < D / 16; ++k) {
          if (k + 1 < D / 16) read_k(k + 1, (k + 1) & 1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            sacc[kb] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[k & 1][kb], qf[k], k == 0 ? f32x16{} : sacc[kb], 0, 0, 0);
        }
      }
      if (cls == MA_TILE_PARTIAL || kin < 64)
        apply_word(sacc, (cls == MA_TILE_PARTIAL ? wcur : ~0ull) & low_bits(kin), hi);
      {
        constexpr int KS = D / 16, RPS = 32 / KS;   // P elements finished per dP step
        bf16x8 va[2][2];
        auto read_v = [&](int k, int sl) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            va[sl][kb] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(vs + (32 * kb + l32) * D + ((16 * k) ^ rx)));
        };
        read_v(0, 0);
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          if (k + 1 < KS) read_v(k + 1, (k + 1) & 1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            dpacc[kb] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[k & 1][kb], dof[k], k == 0 ? f32x16{} : dpacc[kb], 0, 0, 0);
#pragma unroll
          for (int x = 0; x < RPS; ++x) {
            const int el = RPS * k + x, kb = el >> 4, r = el & 15;
            sacc[kb][r] = fast_exp2(__builtin_fmaf(sacc[kb][r], c, -l2));
          }
        }
      }
      // dS = P (dP - D), rounded to bf16
      bf16x8 dsb[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) dpacc[kb][r] = sacc[kb][r] * (dpacc[kb][r] - dd);
        dsb[2 * kb] = to_bf16x8(dpacc[kb], 0);
        dsb[2 * kb + 1] = to_bf16x8(dpacc[kb], 1);
      }
      // dQ^T += K^T dS^T (keys 16 u .. of the tile); transposed operands read one step ahead
      {
        constexpr int NS = 4 * (D / 32);
        bf16x8 ta[2];
        auto read_t = [&](int x, int sl) { ta[sl] = tr_read(ks, x / (D / 32), x % (D / 32)); };
        read_t(0, 0);
#pragma unroll
        for (int x = 0; x < NS; ++x) {
          if (x + 1 < NS) read_t(x + 1, (x + 1) & 1);
          __builtin_amdgcn_sched_barrier(0);
          const int u = x / (D / 32), n = x % (D / 32);
          dqacc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[x & 1], dsb[u], dqacc[n], 0, 0, 0);
        }
      }
    }
  }
  if (row_ok) store_row<D, float>(p.dq + (tok * p.hq + h) * D, dqacc, p.scale, hi);
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (k-tile, K/V head), 4 waves.  Wave w owns keys
// 32 (w % 2) .. + 31 of the tile (K and V rows held as B operands) and query
// rows 32 (w / 2) .. + 31 of every 64-row block; the two waves of a key half
// add their partial sums at the end.  Query blocks (Q, dO, and per row L2, D
// and the tile word) are gathered straight into LDS (global_load_lds) one
// block ahead, into two alternating stages.
// ---------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(256, (D == 256 ? 1 : 2)) void bwd_dkdv(BwdParams p) {
  using QB = QBlk<D>;
  constexpr int CH = D / 8, NI = CH / 4;   // gather instructions per wave per matrix
  extern __shared__ __align__(16) uint16_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int kh = wave & 1, qh = wave >> 1;
  const int hkv = p.hq / p.group;
  const int item_idx = blockIdx.x / hkv, g = blockIdx.x - item_idx * hkv;
  const Item it = p.kitems[item_idx];   // it.qt holds the k-tile
  const SeqInfo sq = p.seqs[it.seq];
  const int kt = it.qt, kv_len = sq.kv_len;
  const int kk = 32 * kh + l32;         // the lane's key inside the tile
  const bool key_ok = kk < kv_len - kt * 64;
  const int32_t *pt = p.page_table + (int64_t)it.seq * p.max_pages;
  const int pmask = (1 << p.page_shift) - 1;
  const int tq = p.tile_q;

  // K and V rows of the lane's key (clamped to the last key) as B operands.
  bf16x8 kf[D / 16], vf[D / 16];
  {
    const int key = min(kt * 64 + kk, kv_len - 1);
    const int64_t off =
        (int64_t)pt[key >> p.page_shift] * p.s_page + (int64_t)(key & pmask) * p.s_slot + (int64_t)g * p.s_head;
    load_q<D>(kf, p.k + off, true, hi);
    load_q<D>(vf, p.v + off, true, hi);
  }

  // Per-lane LDS offsets (elements) inside a block.  Row reads: row 32 qh +
  // l32, chunk 2 k + hi, stored at chunk (2 k + hi) ^ f = 2 k ^ (hi ^ f).
  // Transposed reads: rows 32 qh + 16 u + j (+ 8), j = 4 hi + (lane % 16) / 4,
  // columns 32 n + 16 ((lane / 16) % 2) + 4 (lane % 4), i.e. chunk 4 n + cb
  // at 4 n ^ (cb ^ f).  The swizzle depends on the row modulo 16 only.
  const int rrow = (32 * qh + l32) * D;
  const int rx = 8 * (hi ^ QB::f(l32));
  const int j = 4 * hi + ((lane & 15) >> 2);
  const int trow = (32 * qh + j) * D;
  const int cb = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tax = 8 * (cb ^ QB::f(j)) + 4 * (lane & 1);
  const int tbx = 8 * (cb ^ QB::f(j + 8)) + 4 * (lane & 1);
  auto tr_read = [&](const uint16_t *m, int u, int n) -> bf16x8 {
    const uint16_t *b = m + trow + 16 * u * D;
    const i16x4 r0 =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(b + ((32 * n) ^ tax)));
    const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4 *)(b + 8 * D + ((32 * n) ^ tbx)));
    const i16x8 v = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
    return __builtin_bit_cast(bf16x8, v);
  };

  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n) {
    dkacc[n] = f32x16{};
    dvacc[n] = f32x16{};
  }

  // Work list: entries (q-tiles, descending) x query heads of the group x the
  // q-tile's 64-row blocks that hold rows of the sequence.
  const int eb = it.ent_begin, ee = it.ent_end;
  auto nblk = [&](int e) {
    const int qt = entry_kt(load_entry(p.kentries, e).kt_cls);
    return min(tq / 64, (sq.q_len - qt * tq + 63) / 64);
  };
  auto issue = [&](int e, int hh, int qb, uint16_t *st) {
    const Entry en = load_entry(p.kentries, e);
    const int qt = entry_kt(en.kt_cls), cls = entry_cls(en.kt_cls);
    const int h = g * p.group + hh;
    const int t0 = qt * tq + qb * 64, last = sq.q_len - 1;
    int ln = lane;
    asm volatile("" : "+v"(ln));   // recompute the per-lane addressing here rather than hold it in registers
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int t = wave * NI + i;
      const int pos = 64 * t + ln, r = pos / CH, pc = pos % CH;
      const int row = min(t0 + r, last);
      const int64_t src = (((int64_t)sq.q_start + row) * p.hq + h) * D + 8 * (pc ^ QB::f(r));
      dma::lds_load16(p.q + src, dma::lds_addr(st + 512 * t));
      dma::lds_load16(p.dout + src, dma::lds_addr(st + QB::ELEMS + 512 * t));
    }
    const int row = min(t0 + lane, last);
    const int64_t ridx = ((int64_t)sq.q_start + row) * p.hq + h;
    uint16_t *meta = st + QB::META + 128 * wave;   // 64 x 4 bytes per wave
    if (wave == 0) {
      lds_load4(p.l2 + ridx, dma::lds_addr(meta));
    } else if (wave == 1) {
      lds_load4(p.dd + ridx, dma::lds_addr(meta));
    } else if (cls == MA_TILE_PARTIAL) {
      const uint32_t *wp = (const uint32_t *)(p.words + (int64_t)en.wblk * tq + qb * 64 + lane) + (wave - 2);
      lds_load4(wp, dma::lds_addr(meta));
    }
  };

  if (eb < ee) {
    int e = eb, hh = 0, qb = 0, nb = nblk(eb);
    issue(e, hh, qb, lds);
    for (int i = 0;; ++i) {
      dma::wait_vmem();
      __syncthreads();   // stage i % 2 is filled; every wave is done with stage (i + 1) % 2
      // next block
      int e2 = e, hh2 = hh, qb2 = qb + 1, nb2 = nb;
      if (qb2 >= nb) {
        qb2 = 0;
        if (++hh2 >= p.group) {
          hh2 = 0;
          ++e2;
          if (e2 < ee) nb2 = nblk(e2);
        }
      }
      const bool more = e2 < ee;
      if (more) issue(e2, hh2, qb2, lds + ((i + 1) & 1) * QB::STAGE);

      const uint16_t *st = lds + (i & 1) * QB::STAGE;
      const uint16_t *qs = st, *ds = st + QB::ELEMS;
      const Entry en = load_entry(p.kentries, e);
      const int cls = entry_cls(en.kt_cls);
      const int nrows = sq.q_len - (entry_kt(en.kt_cls) * tq + qb * 64);
      // S = Q K^T, dP = dO V^T: this wave's 32 query rows x 32 keys (lane = key)
      f32x16 sb = f32x16{}, dpb = f32x16{};
#pragma unroll
      for (int k = 0; k < D / 16; ++k) {
        const bf16x8 qa = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qs + rrow + ((16 * k) ^ rx)));
        const bf16x8 da = __builtin_bit_cast(bf16x8, *(const u32x4 *)(ds + rrow + ((16 * k) ^ rx)));
        sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[k], sb, 0, 0, 0);
        dpb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vf[k], dpb, 0, 0, 0);
      }
      // P and dS: register r holds query row 32 qh + 8 (r / 4) + 4 hi + r % 4
      const float *meta = (const float *)(st + QB::META);
      const uint32_t *wd = (const uint32_t *)(st + QB::META + 128 * (2 + kh));
      const float c = p.scale_log2;
      // Branch-free: every probability is computed, then selected; a FULL
      // tile's words are read (stale) and overridden by `full`.
      const uint32_t full = cls == MA_TILE_PARTIAL ? 0u : ~0u;
      const uint32_t kbit = key_ok ? (1u << l32) : 0u;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int r0 = 32 * qh + 8 * a + 4 * hi;
        const f32x4 l2v = *(const f32x4 *)(meta + r0);
        const f32x4 ddv = *(const f32x4 *)(meta + 64 + r0);
        const u32x4 wv = *(const u32x4 *)(wd + r0);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int r = 4 * a + b;
          const uint32_t bits = (wv[b] | full) & (r0 + b < nrows ? kbit : 0u);
          const float ex = fast_exp2(__builtin_fmaf(sb[r], c, -l2v[b]));
          const float pr = bits ? ex : 0.f;
          sb[r] = pr;
          dpb[r] = pr * (dpb[r] - ddv[b]);
        }
      }
      const bf16x8 pb0 = to_bf16x8(sb, 0), pb1 = to_bf16x8(sb, 1);
      const bf16x8 sb0 = to_bf16x8(dpb, 0), sb1 = to_bf16x8(dpb, 1);
      // dV^T += dO^T P, dK^T += Q^T dS (query rows 16 u .. of this wave's 32)
#pragma unroll
      for (int n = 0; n < D / 32; ++n) {
        dvacc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_read(ds, 0, n), pb0, dvacc[n], 0, 0, 0);
        dvacc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_read(ds, 1, n), pb1, dvacc[n], 0, 0, 0);
        dkacc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_read(qs, 0, n), sb0, dkacc[n], 0, 0, 0);
        dkacc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_read(qs, 1, n), sb1, dkacc[n], 0, 0, 0);
      }
      if (!more) break;
      e = e2;
      hh = hh2;
      qb = qb2;
      nb = nb2;
    }
  }

  // The two waves of a key half add their partial sums: wave (kh, 0) keeps
  // dK and receives the other's dK, wave (kh, 1) keeps dV and receives dV.
  __syncthreads();   // every wave is done with the stages (no gather is outstanding)
  float *red = (float *)lds;
  constexpr int RSZ = (D / 32) * 16 * 64;   // floats per wave region
  {
    float *mine = red + (2 * kh + qh) * RSZ;
#pragma unroll
    for (int n = 0; n < D / 32; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) mine[(16 * n + r) * 64 + lane] = qh == 0 ? dvacc[n][r] : dkacc[n][r];
  }
  __syncthreads();
  {
    const float *other = red + (2 * kh + (qh ^ 1)) * RSZ;
#pragma unroll
    for (int n = 0; n < D / 32; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = other[(16 * n + r) * 64 + lane];
        if (qh == 0)
          dkacc[n][r] += x;
        else
          dvacc[n][r] += x;
      }
  }
  if (!key_ok) return;
  const int key = kt * 64 + kk;
  const int64_t off =
      (int64_t)pt[key >> p.page_shift] * p.s_page + (int64_t)(key & pmask) * p.s_slot + (int64_t)g * p.s_head;
  if (qh == 0)
    store_row<D, float>(p.dk + off, dkacc, p.scale, hi);
  else
    store_row<D, float>(p.dv + off, dvacc, 1.f, hi);
}

// ---------------------------------------------------------------------------
// dK, dV for plans with 128-row q-tiles: one workgroup per (k-tile, K/V
// head), 4 waves, each wave all 64 keys and query rows 32 w .. + 31 of every
// 128-row block, so every Q / dO operand read from LDS feeds two products.
// K rows of the first 32 keys are held as B operands; the other K rows and
// the V rows (the B operands of dP) are read from LDS copies of the tile,
// for the register budget.  Each wave gathers its own 32 query rows (Q, dO, L2, D) straight
// into its own pair of LDS stages one block ahead, so the waves run without
// barriers until the four partial sums are added at the end.
// ---------------------------------------------------------------------------
template <int D>
struct QBlkW {
  static constexpr int ROWS = 32;                    // rows per wave
  static constexpr int ELEMS = ROWS * D;
  static constexpr int META = 2 * ELEMS;             // l2 [64], dd [64] floats (lanes 32..63 repeat 0..31),
                                                     // then the 32 rows' tile words (u64)
  static constexpr int WSTAGE = META + 3 * 64 * 2;   // elements of one wave stage
  static constexpr int V_OFF = 4 * 2 * WSTAGE;       // V tile, 64 x D, swizzled like a block
  static constexpr int K1_OFF = V_OFF + 64 * D;      // K rows of keys 32..63, 32 x D, swizzled likewise
  static constexpr size_t LDS = (size_t)(K1_OFF + 32 * D) * sizeof(uint16_t);
};

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_wide(BwdParams p) {
  using QB = QBlk<D>;
  using QW = QBlkW<D>;
  constexpr int CH = D / 8, NI = CH / 2;   // gather instructions per wave per matrix (32 rows)
  extern __shared__ __align__(16) uint16_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int hkv = p.hq / p.group;
  const int item_idx = blockIdx.x / hkv, g = blockIdx.x - item_idx * hkv;
  const Item it = p.kitems[item_idx];
  const SeqInfo sq = p.seqs[it.seq];
  const int kt = it.qt, kv_len = sq.kv_len;
  const int kin = kv_len - kt * 64;
  const int32_t *pt = p.page_table + (int64_t)it.seq * p.max_pages;
  const int pmask = (1 << p.page_shift) - 1;

  // K rows of keys 0..31 as B operands in registers; K rows of keys 32..63
  // and all V rows in LDS (the register file holds the dK / dV sums).
  bf16x8 kf[D / 16];
  {
    const int key = min(kt * 64 + l32, kv_len - 1);
    const int64_t off =
        (int64_t)pt[key >> p.page_shift] * p.s_page + (int64_t)(key & pmask) * p.s_slot + (int64_t)g * p.s_head;
    load_q<D>(kf, p.k + off, true, hi);
  }
  uint16_t *vt = lds + QW::V_OFF;
  uint16_t *k1t = lds + QW::K1_OFF;
  {
    // thread -> key tid / 4, chunks (tid % 4) + 4 x
    const int r = tid >> 2;
    const int key = min(kt * 64 + r, kv_len - 1);
    const int64_t off =
        (int64_t)pt[key >> p.page_shift] * p.s_page + (int64_t)(key & pmask) * p.s_slot + (int64_t)g * p.s_head;
#pragma unroll
    for (int x = 0; x < CH / 4; ++x) {
      const int c = (tid & 3) + 4 * x;
      *(u32x4 *)(vt + r * D + 8 * (c ^ QB::f(r))) = *(const u32x4 *)(p.v + off + 8 * c);
      if (r >= 32) *(u32x4 *)(k1t + (r - 32) * D + 8 * (c ^ QB::f(r))) = *(const u32x4 *)(p.k + off + 8 * c);
    }
  }

  // Row reads: row l32 of the wave's block, chunk 2 k + hi, stored at chunk
  // 2 k ^ (hi ^ f).  Transposed reads: rows 16 u + j (+ 8), j = 4 hi +
  // (lane % 16) / 4, columns 32 n + 16 ((lane / 16) % 2) + 4 (lane % 4), i.e.
  // chunk 4 n + cb at 4 n ^ (cb ^ f).  f depends on the row modulo 16.
  const int rrow = l32 * D;
  const int rx = 8 * (hi ^ QB::f(l32));
  const int j = 4 * hi + ((lane & 15) >> 2);
  const int trow = j * D;
  const int cb = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tax = 8 * (cb ^ QB::f(j)) + 4 * (lane & 1);
  const int tbx = 8 * (cb ^ QB::f(j + 8)) + 4 * (lane & 1);
  auto tr_read = [&](const uint16_t *m, int u, int n) -> bf16x8 {
    const uint16_t *b = m + trow + 16 * u * D;
    const i16x4 r0 =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(b + ((32 * n) ^ tax)));
    const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4 *)(b + 8 * D + ((32 * n) ^ tbx)));
    const i16x8 v = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
    return __builtin_bit_cast(bf16x8, v);
  };

  // Gather addressing: instruction i, lane l loads row (64 / CH) i + l / CH of
  // the wave's 32, logical chunk (l % CH) ^ f(row) into LDS position 64 i + l.
  const uint32_t lds_base = dma::lds_addr(lds);
  const uint32_t row_bytes = (uint32_t)p.hq * D * 2;

  f32x16 dkacc[2][D / 32], dvacc[2][D / 32];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int n = 0; n < D / 32; ++n) {
      dkacc[kb][n] = f32x16{};
      dvacc[kb][n] = f32x16{};
    }

  const int eb = it.ent_begin, ee = it.ent_end;
  // Gathers the wave's rows of block (e, hh) into its stage sl; rows past the
  // sequence repeat its last row (their probabilities are masked to 0).
  auto issue = [&](int e, int hh, int sl) {
    const Entry en = load_entry(p.kentries, e);
    const int qt = entry_kt(en.kt_cls);
    const int h = g * p.group + hh;
    const int t0 = qt * 128 + 32 * wave;
    const int rb = min(t0, sq.q_len - 1);
    const int rmax = max(0, min(31, sq.q_len - 1 - t0));
    const int64_t row0 = ((int64_t)sq.q_start + rb) * p.hq + h;
    const gptr_t qb = (gptr_t)(p.q + row0 * D);
    const gptr_t db = (gptr_t)(p.dout + row0 * D);
    const uint32_t st = lds_base + (uint32_t)((2 * wave + sl) * QW::WSTAGE) * 2;
    int ln = lane;
    asm volatile("" : "+v"(ln));   // keep the per-lane addressing local to the gather
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = (64 / CH) * i + ln / CH, pc = ln % CH;
      const uint32_t voff = (uint32_t)min(r, rmax) * row_bytes + 16 * (pc ^ QB::f(r));
      lds_load16_s(qb, voff, st + 1024 * i);
      lds_load16_s(db, voff, st + QW::ELEMS * 2 + 1024 * i);
    }
    const uint32_t moff = (uint32_t)min(ln & 31, rmax) * (uint32_t)p.hq * 4;
    lds_load4_s((gptr_t)(p.l2 + row0), moff, st + QW::META * 2);
    lds_load4_s((gptr_t)(p.dd + row0), moff, st + QW::META * 2 + 256);
    if (entry_cls(en.kt_cls) == MA_TILE_PARTIAL)   // lane l: dword l of the wave's 32 words
      lds_load4_s((gptr_t)(p.words + (int64_t)en.wblk * 128 + 32 * wave), 4 * ln, st + QW::META * 2 + 512);
  };

  __syncthreads();   // the V tile
  if (eb < ee) {
    int e = eb, hh = 0;
    issue(e, hh, 0);
    for (int i = 0;; ++i) {
      dma::wait_vmem();   // this wave's gathers of block i have landed
      int e2 = e, hh2 = hh + 1;
      if (hh2 >= p.group) {
        hh2 = 0;
        ++e2;
      }
      const bool more = e2 < ee;
      if (more) issue(e2, hh2, (i + 1) & 1);

      const Entry en = load_entry(p.kentries, e);
      const int cls = entry_cls(en.kt_cls);
      const int nv = sq.q_len - (entry_kt(en.kt_cls) * 128 + 32 * wave);   // valid rows of this wave
      {
        const uint16_t *qs = lds + (2 * wave + (i & 1)) * QW::WSTAGE;
        const uint16_t *ds = qs + QW::ELEMS;
        float *meta = (float *)(lds + (2 * wave + (i & 1)) * QW::WSTAGE + QW::META);
        // Rows past the sequence (gathered as copies of its last row) get
        // L2 = +inf, so their probabilities are exactly 0.
        if (nv < 32 && l32 >= nv) meta[lane] = __builtin_inff();
        // The block in four phases, each VALU phase placed beside the
        // products of the next so that one wave keeps the matrix cores busy:
        //   S = Q K^T | dP = dO V^T beside P | dV^T += dO^T P beside dS |
        //   dK^T += Q^T dS.
        // Register r of a lane holds query row 8 (r / 4) + 4 hi + r % 4 and
        // key 32 kb + l32; its visibility is bit l32 of half kb of the row's
        // tile word.  Operands of step k + 1 are read while step k's products
        // run.
        constexpr int KS = D / 16;              // k-steps of S and dP
        constexpr int RPS = 16 / KS;            // rows of P finished per dP step
        const uint32_t *wd = (const uint32_t *)(qs + QW::META + 256);
        const uint32_t full = cls == MA_TILE_PARTIAL ? 0u : ~0u;
        const uint32_t kbit0 = l32 < kin ? (1u << l32) : 0u;
        const uint32_t kbit1 = 32 + l32 < kin ? (1u << l32) : 0u;
        const float c = p.scale_log2;

        f32x16 sb[2];
        {
          bf16x8 qa[2], kb1[2];
          auto read_s = [&](int k, int sl) {
            qa[sl] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qs + rrow + ((16 * k) ^ rx)));
            kb1[sl] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(k1t + rrow + ((16 * k) ^ rx)));
          };
          read_s(0, 0);
#pragma unroll
          for (int k = 0; k < KS; ++k) {
            if (k + 1 < KS) read_s(k + 1, (k + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
            const int sl = k & 1;
            sb[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[sl], kf[k], k == 0 ? f32x16{} : sb[0], 0, 0, 0);
            sb[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[sl], kb1[sl], k == 0 ? f32x16{} : sb[1], 0, 0, 0);
          }
        }
        // Masked entries (PARTIAL tiles, keys past kv_len) get S = -inf, so
        // exp2 gives them exactly 0; FULL interior tiles skip this.
        if (cls == MA_TILE_PARTIAL || kin < 64) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = 8 * (r >> 2) + 4 * hi + (r & 3);
            const uint32_t wlo = wd[2 * row], whi = wd[2 * row + 1];
            if (!((wlo | full) & kbit0)) sb[0][r] = neg_inf();
            if (!((whi | full) & kbit1)) sb[1][r] = neg_inf();
          }
        }
        // dP, and beside it P = exp2(S c - L2)
        f32x16 dpb[2];
        f32x8 pv[2][2];   // P as fp32 (for dS), [kb][u]
        bf16x8 pb[2][2];
        {
          bf16x8 da[2], vb[2][2];
          auto read_p = [&](int k, int sl) {
            da[sl] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(ds + rrow + ((16 * k) ^ rx)));
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
              vb[sl][kb] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(vt + (32 * kb + l32) * D + ((16 * k) ^ rx)));
          };
          read_p(0, 0);
#pragma unroll
          for (int k = 0; k < KS; ++k) {
            if (k + 1 < KS) read_p(k + 1, (k + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
            const int sl = k & 1;
            dpb[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[sl], vb[sl][0], k == 0 ? f32x16{} : dpb[0], 0, 0, 0);
            dpb[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[sl], vb[sl][1], k == 0 ? f32x16{} : dpb[1], 0, 0, 0);
#pragma unroll
            for (int rr = 0; rr < RPS; ++rr) {
              const int r = RPS * k + rr, a4 = r >> 2, b = r & 3;
              const float l2 = meta[8 * a4 + 4 * hi + b];
              pv[0][r >> 3][r & 7] = fast_exp2(__builtin_fmaf(sb[0][r], c, -l2));
              pv[1][r >> 3][r & 7] = fast_exp2(__builtin_fmaf(sb[1][r], c, -l2));
            }
          }
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int u = 0; u < 2; ++u) pb[kb][u] = __builtin_convertvector(pv[kb][u], bf16x8);
        }
        // dV^T += dO^T P, and beside it dS = P (dP - D)
        bf16x8 sbf[2][2];
        {
          constexpr int NS = 2 * (D / 32);   // steps (n, u)
          constexpr int EPS = 32 / NS;       // dS elements finished per step
          f32x8 dv[2][2];
          bf16x8 ta[2];
          auto read_v = [&](int x, int sl) { ta[sl] = tr_read(ds, x & 1, x >> 1); };
          read_v(0, 0);
#pragma unroll
          for (int x = 0; x < NS; ++x) {
            if (x + 1 < NS) read_v(x + 1, (x + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
            const int n = x >> 1, u = x & 1;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
              dvacc[kb][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[x & 1], pb[kb][u], dvacc[kb][n], 0, 0, 0);
#pragma unroll
            for (int ee2 = 0; ee2 < EPS; ++ee2) {
              const int el = EPS * x + ee2, kb = el >> 4, r = el & 15;
              const int row = 8 * (r >> 2) + 4 * hi + (r & 3);
              dv[kb][r >> 3][r & 7] = pv[kb][r >> 3][r & 7] * (dpb[kb][r] - meta[64 + row]);
            }
          }
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int u = 0; u < 2; ++u) sbf[kb][u] = __builtin_convertvector(dv[kb][u], bf16x8);
        }
        // dK^T += Q^T dS
        {
          constexpr int NS = 2 * (D / 32);
          bf16x8 tb[2];
          auto read_k = [&](int x, int sl) { tb[sl] = tr_read(qs, x & 1, x >> 1); };
          read_k(0, 0);
#pragma unroll
          for (int x = 0; x < NS; ++x) {
            if (x + 1 < NS) read_k(x + 1, (x + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
            const int n = x >> 1, u = x & 1;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
              dkacc[kb][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tb[x & 1], sbf[kb][u], dkacc[kb][n], 0, 0, 0);
          }
        }
      }
      if (!more) break;
      e = e2;
      hh = hh2;
    }
  }

  // Four partial sums per key are added in OWN rounds: in round q, wave w
  // owns accumulator w * OWN + q (accumulators indexed (matrix, kb, n)); the
  // other waves park their copies of it in LDS and the owner adds them, in
  // wave order, and stores the result.
  constexpr int NACC = 2 * 2 * (D / 32);
  constexpr int OWN = NACC / 4;
  constexpr int RSZ = 16 * 64;            // floats of one accumulator over a wave
  static_assert(16 * RSZ * 4 <= QW::V_OFF * 2, "reduction does not fit the stages");
  float *red = (float *)lds;              // [owner][writer][RSZ]
  auto acc_ref = [&](int a) -> f32x16 & {
    const int m = a / (2 * (D / 32)), kb = (a / (D / 32)) % 2, n = a % (D / 32);
    return m == 0 ? dkacc[kb][n] : dvacc[kb][n];
  };
  int64_t off[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = min(kt * 64 + 32 * kb + l32, kv_len - 1);
    off[kb] = (int64_t)pt[key >> p.page_shift] * p.s_page + (int64_t)(key & pmask) * p.s_slot +
              (int64_t)g * p.s_head;
  }
#pragma unroll
  for (int q = 0; q < OWN; ++q) {
    __syncthreads();   // the stages (or the previous round's slots) are free
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (w == wave) continue;
      float *dst = red + (4 * w + wave) * RSZ;
      const f32x16 &v = acc_ref(w * OWN + q);
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[r * 64 + lane] = v[r];
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (w != wave) continue;
      const int a = w * OWN + q;
      f32x16 &v = acc_ref(a);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        if (x == w) continue;
        const float *src = red + (4 * w + x) * RSZ;
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] += src[r * 64 + lane];
      }
      const int m = a / (2 * (D / 32)), kb = (a / (D / 32)) % 2, n = a % (D / 32);
      if (32 * kb + l32 < kin) {
        float *dst = (m == 0 ? p.dk : p.dv) + off[kb];
        const float sc = m == 0 ? p.scale : 1.f;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d0 = 32 * n + 8 * r4 + 4 * hi;
          store4<float>(dst + d0, v[4 * r4] * sc, v[4 * r4 + 1] * sc, v[4 * r4 + 2] * sc, v[4 * r4 + 3] * sc);
        }
      }
    }
  }
}

template <typename K>
ma_status launch(K kern, int grid, int block, size_t lds, const BwdParams &prm, void *stream, const char *what) {
  if (grid == 0) return MA_OK;
  hipError_t e = hipSuccess;
  if (lds > 64 * 1024) e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return set_error(MA_ERR_HIP, "hipFuncSetAttribute: %s", hipGetErrorString(e));
  hipLaunchKernelGGL(kern, dim3(grid), dim3(block), lds, (hipStream_t)stream, prm);
  e = hipGetLastError();
  if (e != hipSuccess) return set_error(MA_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
  return MA_OK;
}

template <int D>
ma_status run(const BackwardArgs &a, const BwdParams &prm) {
  const int64_t rows = a.total_q * a.hq;
  constexpr int prep_rows = 256 / (D / 8);
  ma_status st = launch(bwd_prep<D>, (int)((rows + prep_rows - 1) / prep_rows), 256, 0, prm, a.stream,
                        "backward prep");
  if (st != MA_OK) return st;
  const size_t dq_lds = 2 * 2 * 64 * D * sizeof(uint16_t);
  const bool fast = (1 << prm.page_shift) >= dma::KvDma<D, 2>::RPI && prm.s_page * 2 < ((int64_t)1 << 32) &&
                    ((int64_t)1 << prm.page_shift) * prm.s_slot * 2 < ((int64_t)1 << 31);
  if (prm.tile_q == 128)
    st = fast ? launch(bwd_dq<D, 128, true>, prm.num_items * a.hq, 256, dq_lds, prm, a.stream, "backward dQ")
              : launch(bwd_dq<D, 128, false>, prm.num_items * a.hq, 256, dq_lds, prm, a.stream, "backward dQ");
  else
    st = fast ? launch(bwd_dq<D, 64, true>, prm.num_items * a.hq, 128, dq_lds, prm, a.stream, "backward dQ")
              : launch(bwd_dq<D, 64, false>, prm.num_items * a.hq, 128, dq_lds, prm, a.stream, "backward dQ");
  if (st != MA_OK) return st;
  // d 256: the 32-keys-per-wave form (the wide form's dK / dV sums of 64
  // keys would need 512 registers per lane); it walks 128-row q-tiles as two
  // 64-row blocks
  if constexpr (D <= 128) {
    if (prm.tile_q == 128)
      return launch(bwd_dkdv_wide<D>, prm.num_kitems * a.hkv, 256, QBlkW<D>::LDS, prm, a.stream, "backward dK dV");
  }
  return launch(bwd_dkdv<D>, prm.num_kitems * a.hkv, 256, QBlk<D>::BYTES, prm, a.stream, "backward dK dV");
}

}  // namespace

size_t backward_workspace(int64_t total_q, int32_t hq) { return (size_t)2 * total_q * hq * sizeof(float); }

ma_status launch_backward(const BackwardArgs &a) {
  ma_plan *pl = a.plan;
  ma_status st = plan_build_kmajor(pl, a.stream);
  if (st != MA_OK) return st;
  if ((int64_t)pl->num_rows * a.hq > INT32_MAX || (int64_t)pl->num_kitems * a.hkv > INT32_MAX ||
      (a.total_q * a.hq + 3) / 4 > INT32_MAX)
    return set_error(MA_ERR_UNSUPPORTED, "grid too large");
  const char *base = (const char *)pl->dbuf;
  const char *kb = (const char *)pl->kbuf;
  BwdParams prm{};
  prm.seqs = (const SeqInfo *)(base + pl->off_seqs);
  prm.items = (const Item *)(base + pl->off_items);
  prm.entries = (const Entry *)(base + pl->off_entries);
  prm.words = (const uint64_t *)(base + pl->off_words);
  prm.kitems = (const Item *)(kb + pl->off_kitems);
  prm.kentries = (const Entry *)(kb + pl->off_kentries);
  prm.q = (const uint16_t *)a.q;
  prm.k = (const uint16_t *)a.k;
  prm.v = (const uint16_t *)a.v;
  prm.dout = (const uint16_t *)a.dout;
  prm.o = a.o;
  prm.o_f32 = a.o_dtype == MA_F32 ? 1 : 0;
  prm.lse = a.lse;
  prm.dq = a.dq;
  prm.dk = a.dk;
  prm.dv = a.dv;
  prm.dd = (float *)a.workspace;
  prm.l2 = prm.dd + a.total_q * a.hq;
  prm.page_table = a.page_table;
  prm.s_page = a.s_page;
  prm.s_slot = a.s_slot;
  prm.s_head = a.s_head;
  prm.total_q = a.total_q;
  prm.max_pages = a.max_pages;
  prm.page_shift = a.page_shift;
  prm.hq = a.hq;
  prm.group = a.hq / a.hkv;
  prm.num_items = pl->num_rows;
  prm.num_kitems = pl->num_kitems;
  prm.tile_q = pl->tile_q;
  prm.scale = a.scale;
  prm.scale_log2 = a.scale * kLog2e;
  switch (a.d) {
    case 64: return run<64>(a, prm);
    case 128: return run<128>(a, prm);
    case 256: return run<256>(a, prm);
  }
  return set_error(MA_ERR_UNSUPPORTED, "backward head_dim %d", a.d);
}

}  // namespace maskattn
