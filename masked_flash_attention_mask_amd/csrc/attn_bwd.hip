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

namespace maskattn {
using namespace dev;

namespace {

// LDS rows of K, V, Q and dO in the backward: stride d + 8 (4 banks modulo
// 64), conflict-free for the row reads of the A operands; the transposed
// reads (ds_read_b64_tr_b16) of the dQ / dK / dV products accept some
// conflicts on this stride.
template <int D>
struct BwdStage {
  static constexpr int S = D + 8;
  static constexpr int TILE = 64 * S;   // elements of one 64-row matrix
};

// The lane's 8-element operand of rows [r0, r0 + 32) of a row-major matrix
// (rows = the MFMA's 32 rows, K-slots d 16 k + 8 hi .. + 7).
template <int D>
__device__ __forceinline__ bf16x8 row_op(const uint16_t *m, int l32, int hi, int k) {
  return __builtin_bit_cast(bf16x8, *(const u32x4 *)(m + l32 * BwdStage<D>::S + 8 * hi + 16 * k));
}

// Transposed operand of d-block n and 16-row step u of a row-major matrix
// (A = M^T: lane = d, K-slots = rows base + 8 (e / 4) + 4 (l / 32) + e % 4,
// base = 16 u), read with ds_read_b64_tr_b16 as in the forward's V^T.
template <int D>
__device__ __forceinline__ bf16x8 tr_op(const uint16_t *m, int lane, int u, int n) {
  constexpr int S = BwdStage<D>::S;
  const uint16_t *p = m + (4 * (lane >> 5) + ((lane & 15) >> 2)) * S + 16 * ((lane >> 4) & 1) + 4 * (lane & 3) +
                      16 * u * S + 32 * n;
  const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)p);
  const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(p + 8 * S));
  const i16x8 v = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
  return __builtin_bit_cast(bf16x8, v);
}

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

// ---------------------------------------------------------------------------
// D[t, h] = <dO[t, h], O[t, h]>, L2[t, h] = LSE[t, h] log2 e (+inf for a row
// with no visible key, so that its probabilities come out exactly 0).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_prep(BwdParams p) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (token, head)
  const int lane = threadIdx.x & 63;
  if (row >= p.total_q * p.hq) return;
  float acc = 0.f;
  for (int c = lane; c < D; c += 64) {
    const float o = p.o_f32 ? ((const float *)p.o)[row * D + c]
                            : __uint_as_float((uint32_t)((const uint16_t *)p.o)[row * D + c] << 16);
    const float g = __uint_as_float((uint32_t)p.dout[row * D + c] << 16);
    acc += o * g;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) {
    p.dd[row] = acc;
    const float lse = p.lse[row];
    p.l2[row] = lse == neg_inf() ? __builtin_inff() : lse * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (q-tile, query head), BQ / 32 waves x 32 query rows.
// ---------------------------------------------------------------------------
template <int D, int BQ>
__global__ __launch_bounds__(BQ * 2, BQ == 128 ? 2 : 1) void bwd_dq(BwdParams p) {
  constexpr int NT = BQ * 2, S = BwdStage<D>::S;
  extern __shared__ __align__(16) uint16_t lds[];   // [2 stages][K tile, V tile]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  using KV = staged::KvTile<D, NT>;
  KV kv;
  typename KV::Pages pg_nxt;
  auto store_kv = [&](uint16_t *stage) {
#pragma unroll
    for (int i = 0; i < KV::PPT; ++i) {
      const int pair = tid + i * NT;
      if (KV::PAIRS % NT == 0 || pair < KV::PAIRS) {
        const int kg = pair / KV::CH, cc = pair % KV::CH;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          *(u32x4 *)(stage + (4 * kg + j) * S + 8 * cc) = kv.kreg[i][j];
          *(u32x4 *)(stage + 64 * S + (4 * kg + j) * S + 8 * cc) = kv.vreg[i][j];
        }
      }
    }
  };

  f32x16 dqacc[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n) dqacc[n] = f32x16{};

  const int eb = it.ent_begin, ee = it.ent_end;
  uint64_t word_nxt = 0;
  auto load_word = [&](Entry e) -> uint64_t {
    return entry_cls(e.kt_cls) == MA_TILE_PARTIAL ? p.words[(int64_t)e.wblk * BQ + wrow] : 0ull;
  };
  if (eb < ee) {
    const Entry e0 = p.entries[eb];
    const int kt0 = entry_kt(e0.kt_cls);
    const typename KV::Pages pg0 = kv.pages(pt, p.page_shift, kt0, kv_len, tid);
    kv.load(kbase, vbase, pg0, p.page_shift, p.s_page, p.s_slot, kt0, kv_len, tid);
    word_nxt = load_word(e0);
    if (eb + 1 < ee) pg_nxt = kv.pages(pt, p.page_shift, entry_kt(p.entries[eb + 1].kt_cls), kv_len, tid);
    store_kv(lds);
    __syncthreads();
  }
  for (int e = eb; e < ee; ++e) {
    const int cur = (e - eb) & 1;
    const Entry ec = p.entries[e];
    const uint64_t wcur = word_nxt;
    const bool has_next = e + 1 < ee;
    if (has_next) {
      const Entry en = p.entries[e + 1];
      kv.load(kbase, vbase, pg_nxt, p.page_shift, p.s_page, p.s_slot, entry_kt(en.kt_cls), kv_len, tid);
      word_nxt = load_word(en);
      if (e + 2 < ee) pg_nxt = kv.pages(pt, p.page_shift, entry_kt(p.entries[e + 2].kt_cls), kv_len, tid);
    }
    const uint16_t *ks = lds + cur * 2 * 64 * S;
    const uint16_t *vs = ks + 64 * S;
    // S^T = K Q^T and dP^T = V dO^T (keys x this wave's 32 query rows)
    f32x16 sacc[2], dpacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16{};
      dpacc[kb] = f32x16{};
#pragma unroll
      for (int k = 0; k < D / 16; ++k) {
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_op<D>(ks + 32 * kb * S, l32, hi, k), qf[k], sacc[kb], 0, 0, 0);
        dpacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_op<D>(vs + 32 * kb * S, l32, hi, k), dof[k], dpacc[kb], 0, 0, 0);
      }
    }
    const int kt = entry_kt(ec.kt_cls), cls = entry_cls(ec.kt_cls);
    const int kin = kv_len - kt * 64;
    if (cls == MA_TILE_PARTIAL || kin < 64)
      apply_word(sacc, (cls == MA_TILE_PARTIAL ? wcur : ~0ull) & low_bits(kin), hi);
    // P = exp2(S c - L2); dS = P (dP - D)
    bf16x8 dsb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = fast_exp2(__builtin_fmaf(sacc[kb][r], c, -l2));
        dpacc[kb][r] = pr * (dpacc[kb][r] - dd);
      }
      dsb[2 * kb] = to_bf16x8(dpacc[kb], 0);
      dsb[2 * kb + 1] = to_bf16x8(dpacc[kb], 1);
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int n = 0; n < D / 32; ++n)
        dqacc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_op<D>(ks + 32 * (u >> 1) * S, lane, u & 1, n), dsb[u],
                                                           dqacc[n], 0, 0, 0);
    if (has_next) store_kv(lds + (cur ^ 1) * 2 * 64 * S);
    __syncthreads();
  }
  if (row_ok) store_row<D, float>(p.dq + (tok * p.hq + h) * D, dqacc, p.scale, hi);
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (k-tile, K/V head), 2 waves x 32 keys.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(128, 1) void bwd_dkdv(BwdParams p) {
  constexpr int NT = 128, S = BwdStage<D>::S, CH = D / 8;
  extern __shared__ __align__(16) uint16_t lds[];   // K tile, V tile, Q block, dO block
  __shared__ float l2s[32], dds[32];
  __shared__ uint64_t wds[32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int item_idx = blockIdx.x / (p.hq / p.group), g = blockIdx.x - item_idx * (p.hq / p.group);
  const Item it = p.kitems[item_idx];   // it.qt holds the k-tile
  const SeqInfo sq = p.seqs[it.seq];
  const int kt = it.qt;
  const int kv_len = sq.kv_len;
  const int kin = kv_len - kt * 64;
  const int kk = wave * 32 + l32;       // this lane's key inside the tile
  uint16_t *ks = lds, *vs = lds + 64 * S, *qs = lds + 2 * 64 * S, *ds = qs + 32 * S;

  // K and V of the tile -> LDS (clamped keys), then the lane's key rows -> registers
  {
    using KV = staged::KvTile<D, NT>;
    KV kv;
    const int32_t *pt = p.page_table + (int64_t)it.seq * p.max_pages;
    const typename KV::Pages pg = kv.pages(pt, p.page_shift, kt, kv_len, tid);
    kv.load(p.k + (int64_t)g * p.s_head, p.v + (int64_t)g * p.s_head, pg, p.page_shift, p.s_page, p.s_slot, kt,
            kv_len, tid);
#pragma unroll
    for (int i = 0; i < KV::PPT; ++i) {
      const int pair = tid + i * NT;
      if (KV::PAIRS % NT == 0 || pair < KV::PAIRS) {
        const int kg = pair / KV::CH, cc = pair % KV::CH;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          *(u32x4 *)(ks + (4 * kg + j) * S + 8 * cc) = kv.kreg[i][j];
          *(u32x4 *)(vs + (4 * kg + j) * S + 8 * cc) = kv.vreg[i][j];
        }
      }
    }
  }
  __syncthreads();
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int k = 0; k < D / 16; ++k) {
    kf[k] = row_op<D>(ks + wave * 32 * S, l32, hi, k);
    vf[k] = row_op<D>(vs + wave * 32 * S, l32, hi, k);
  }
  const bool key_ok = kk < kin;
  const float c = p.scale_log2;

  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n) {
    dkacc[n] = f32x16{};
    dvacc[n] = f32x16{};
  }

  const int tq = p.tile_q;
  for (int e = it.ent_begin; e < it.ent_end; ++e) {
    const Entry en = p.kentries[e];
    const int qt = entry_kt(en.kt_cls), cls = entry_cls(en.kt_cls);
    for (int hh = 0; hh < p.group; ++hh) {
      const int h = g * p.group + hh;
      for (int qb = 0; qb < tq / 32; ++qb) {
        const int t0 = qt * tq + qb * 32;             // first query row of the block
        if (t0 >= sq.q_len) break;
        // Q and dO blocks (32 rows), L2, D and the block's row words -> LDS
        __syncthreads();
        for (int x = tid; x < 32 * CH; x += NT) {
          const int r = x / CH, cc = x % CH;
          const int t = t0 + r;
          u32x4 qv = {0, 0, 0, 0}, gv = {0, 0, 0, 0};
          if (t < sq.q_len) {
            const int64_t off = (((int64_t)sq.q_start + t) * p.hq + h) * D + 8 * cc;
            qv = *(const u32x4 *)(p.q + off);
            gv = *(const u32x4 *)(p.dout + off);
          }
          *(u32x4 *)(qs + r * S + 8 * cc) = qv;
          *(u32x4 *)(ds + r * S + 8 * cc) = gv;
        }
        if (tid < 32) {
          const int t = t0 + tid;
          const bool ok = t < sq.q_len;
          const int64_t row = ((int64_t)sq.q_start + t) * p.hq + h;
          l2s[tid] = ok ? p.l2[row] : __builtin_inff();
          dds[tid] = ok ? p.dd[row] : 0.f;
          wds[tid] = (ok && cls == MA_TILE_PARTIAL) ? p.words[(int64_t)en.wblk * tq + qb * 32 + tid] : ~0ull;
        }
        __syncthreads();
        // S = Q K^T, dP = dO V^T (32 queries x this wave's 32 keys)
        f32x16 sb = f32x16{}, dpb = f32x16{};
#pragma unroll
        for (int k = 0; k < D / 16; ++k) {
          sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_op<D>(qs, l32, hi, k), kf[k], sb, 0, 0, 0);
          dpb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_op<D>(ds, l32, hi, k), vf[k], dpb, 0, 0, 0);
        }
        // P and dS for the lane's key and the queries of its registers
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qr = 8 * (r >> 2) + 4 * hi + (r & 3);
          const bool vis = key_ok && ((wds[qr] >> kk) & 1ull);
          const float pr = vis ? fast_exp2(__builtin_fmaf(sb[r], c, -l2s[qr])) : 0.f;
          sb[r] = pr;
          dpb[r] = pr * (dpb[r] - dds[qr]);
        }
        const bf16x8 pb0 = to_bf16x8(sb, 0), pb1 = to_bf16x8(sb, 1);
        const bf16x8 sb0 = to_bf16x8(dpb, 0), sb1 = to_bf16x8(dpb, 1);
        // dV^T += dO^T P, dK^T += Q^T dS
#pragma unroll
        for (int n = 0; n < D / 32; ++n) {
          dvacc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_op<D>(ds, lane, 0, n), pb0, dvacc[n], 0, 0, 0);
          dvacc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_op<D>(ds, lane, 1, n), pb1, dvacc[n], 0, 0, 0);
          dkacc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_op<D>(qs, lane, 0, n), sb0, dkacc[n], 0, 0, 0);
          dkacc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_op<D>(qs, lane, 1, n), sb1, dkacc[n], 0, 0, 0);
        }
      }
    }
  }
  if (!key_ok) return;
  const int key = kt * 64 + kk;
  const int pmask = (1 << p.page_shift) - 1;
  const int64_t off = (int64_t)p.page_table[(int64_t)it.seq * p.max_pages + (key >> p.page_shift)] * p.s_page +
                      (int64_t)(key & pmask) * p.s_slot + (int64_t)g * p.s_head;
  store_row<D, float>(p.dk + off, dkacc, p.scale, hi);
  store_row<D, float>(p.dv + off, dvacc, 1.f, hi);
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
  ma_status st = launch(bwd_prep<D>, (int)((rows + 3) / 4), 256, 0, prm, a.stream, "backward prep");
  if (st != MA_OK) return st;
  const size_t dq_lds = 2 * 2 * 64 * BwdStage<D>::S * sizeof(uint16_t);
  if (prm.tile_q == 128)
    st = launch(bwd_dq<D, 128>, prm.num_items * a.hq, 256, dq_lds, prm, a.stream, "backward dQ");
  else
    st = launch(bwd_dq<D, 64>, prm.num_items * a.hq, 128, dq_lds, prm, a.stream, "backward dQ");
  if (st != MA_OK) return st;
  return launch(bwd_dkdv<D>, prm.num_kitems * a.hkv, 128, (2 * 64 + 2 * 32) * BwdStage<D>::S * sizeof(uint16_t), prm,
                a.stream, "backward dK dV");
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
  }
  return set_error(MA_ERR_UNSUPPORTED, "backward head_dim %d", a.d);
}

}  // namespace maskattn
