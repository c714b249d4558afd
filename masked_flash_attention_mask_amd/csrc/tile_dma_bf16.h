// bf16 tile machinery of the kernels that gather paged K/V straight from the
// cache into LDS (global_load_lds_dwordx4): the swizzled LDS stage layout,
// the gather, and the two matrix-core products of a wave's 32 query rows.
#pragma once

#include "internal.h"
#include "kernels_common.h"

namespace maskattn {
namespace dev {
namespace dma {

// LDS stage of one 64-key tile: K and V, each [64 keys][D] bf16 without
// padding, stored as 16-byte chunks whose position inside a row is XOR
// swizzled by the row (key) index.  The gather writes whole 1 KB runs per
// wave instruction (global_load_lds_dwordx4), so the swizzle is applied on
// the source side.  K's swizzle makes the 16 rows x 1 chunk of an operand
// read (ds_read_b128) hit distinct banks; V's makes the 4 rows x 4 chunks a
// 16-lane group reads with ds_read_b64_tr_b16 hit distinct banks.
template <int D>
struct Stage {
  static constexpr int CH = D / 8;          // 16-byte chunks per row
  static constexpr int V_OFF = 64 * D;      // elements
  static constexpr int ELEMS = 2 * 64 * D;
  static constexpr size_t BYTES = ELEMS * sizeof(uint16_t);
  __host__ __device__ static constexpr int fk(int r) { return CH >= 16 ? (r & 15) : ((r >> 1) & 7); }
  __host__ __device__ static constexpr int fv(int r) { return CH >= 16 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

// Direct global -> LDS load of 16 bytes per lane to LDS address lds + 16 lane
// (M0 holds lds).  Inline asm keeps the compiler from tracking it: it would
// otherwise wait for every outstanding LDS gather before each later LDS read,
// including reads of the other stage.  The kernels order the gathers
// themselves (wait_vmem() before the barrier that publishes a stage).  The
// load writes no registers; its address registers are read at issue.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p);
}
__device__ __forceinline__ void lds_load16(const void *src, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}
// The same with a scalar (SGPR) base and a 32-bit per-lane byte offset.
typedef const __attribute__((address_space(1))) void *gptr_t;
__device__ __forceinline__ void lds_load16_s(gptr_t base, uint32_t voff, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
}

// Direct global -> LDS gather of one tile by NW waves: wave instruction t
// fills LDS chunks [64 t, 64 t + 64) of K (and of V); lane l of it loads the
// chunk that belongs at position 64 t + l.  Keys at or past kv_len are
// clamped to the last key, so every load is in bounds: such keys are masked
// to probability exactly 0 and read finite V, so they add nothing.
template <int D, int NW>
struct KvDma {
  static constexpr int CH = D / 8;
  static constexpr int IPW = CH / NW;       // instructions per wave per matrix
  static_assert(CH % NW == 0, "tile gather needs CH to be a multiple of the wave count");
  struct Pages {
    int32_t id[IPW];
  };

  static constexpr int RPI = 64 / CH;       // key rows per instruction

  // Page of the key each lane loads in each of its instructions for tile kt
  // (any page size; one vector load per instruction).
  __device__ __forceinline__ static Pages pages(const int32_t *pt, int page_shift, int kt, int kv_len, int wave,
                                               int lane) {
    Pages pg;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int r = (64 * (wave * IPW + i) + lane) / CH;
      pg.id[i] = pt[min(kt * 64 + r, kv_len - 1) >> page_shift];
    }
    return pg;
  }

  // The same for pages of at least RPI keys: the RPI rows of an instruction
  // (an RPI-aligned key group, or keys clamped to the last key, which lies in
  // the same group or past it) share one page, read with a scalar load
  // through the constant address space.  Scalar loads leave the vector
  // memory counter to the gathers, so no wait for a page id drains them.
  __device__ __forceinline__ static Pages pages_uniform(const int32_t *pt, int page_shift, int kt, int kv_len,
                                                       int wave) {
    const __attribute__((address_space(4))) int32_t *cpt = (const __attribute__((address_space(4))) int32_t *)pt;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    Pages pg;
#pragma unroll
    for (int i = 0; i < IPW; ++i) pg.id[i] = cpt[min(kt * 64 + RPI * (wv * IPW + i), kv_len - 1) >> page_shift];
    return pg;
  }

  // Issues this wave's gathers of tile kt into the stage at LDS byte address
  // stage (scalar), with page ids from pages_uniform: each instruction's RPI
  // rows share one page,
  // so its source is a scalar page base plus a 32-bit per-lane offset (the
  // SGPR-base form of the instruction), and M0 is scalar arithmetic: no
  // 64-bit per-lane address math.  Needs page_size * s_slot * 2 < 2^31.
  // Per-lane page ids (any page size): a 64-bit address per lane.
  __device__ __forceinline__ static void issue_lanes(const uint16_t *kbase, const uint16_t *vbase, const Pages &pg,
                                               int page_shift, int64_t s_page, int64_t s_slot, int kt,
                                               int kv_len, uint16_t *stage, int wave, int lane) {
    const int pmask = (1 << page_shift) - 1;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int t = wave * IPW + i;
      const int pos = 64 * t + lane;
      const int r = pos / CH, pc = pos % CH;
      const int key = min(kt * 64 + r, kv_len - 1);
      const int64_t off = (int64_t)pg.id[i] * s_page + (int64_t)(key & pmask) * s_slot;
      lds_load16(kbase + off + 8 * (pc ^ Stage<D>::fk(r)), lds_addr(stage + 512 * t));
      lds_load16(vbase + off + 8 * (pc ^ Stage<D>::fv(r)), lds_addr(stage + Stage<D>::V_OFF + 512 * t));
    }
  }

  __device__ __forceinline__ static void issue(const uint16_t *kbase, const uint16_t *vbase, const Pages &pg,
                                               int page_shift, int64_t s_page, int64_t s_slot, int kt,
                                               int kv_len, uint32_t stage, int wave, int lane) {
    const int pmask = (1 << page_shift) - 1;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int t = wave * IPW + i;
      const int pos = 64 * t + lane;
      const int r = pos / CH, pc = pos % CH;
      const int key = min(kt * 64 + r, kv_len - 1);
      const int64_t pb = (int64_t)pg.id[i] * s_page;
      const uint32_t slot = (uint32_t)((key & pmask) * (int)s_slot) * 2;
      lds_load16_s((gptr_t)(kbase + pb), slot + 16 * (pc ^ Stage<D>::fk(r)), stage + 1024 * t);
      lds_load16_s((gptr_t)(vbase + pb), slot + 16 * (pc ^ Stage<D>::fv(r)), stage + 2 * Stage<D>::V_OFF + 1024 * t);
    }
  }
};

// One matrix (K when !IS_V, V when IS_V) of issue(), into the LDS byte address
// dst of that matrix's half of a stage: the software-pipelined kernel
// gathers a tile's K one step before its V.
template <int D, int NW, bool IS_V>
__device__ __forceinline__ void issue_mat(const uint16_t *base, const typename KvDma<D, NW>::Pages &pg,
                                          int page_shift, int64_t s_page, int64_t s_slot, int kt, int kv_len,
                                          uint32_t dst, int wave, int lane) {
  constexpr int CH = KvDma<D, NW>::CH, IPW = KvDma<D, NW>::IPW;
  const int pmask = (1 << page_shift) - 1;
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int t = wave * IPW + i;
    const int pos = 64 * t + lane;
    const int r = pos / CH, pc = pos % CH;
    const int key = min(kt * 64 + r, kv_len - 1);
    const int64_t pb = (int64_t)pg.id[i] * s_page;
    const uint32_t slot = (uint32_t)((key & pmask) * (int)s_slot) * 2;
    const int sw = IS_V ? Stage<D>::fv(r) : Stage<D>::fk(r);
    lds_load16_s((gptr_t)(base + pb), slot + 16 * (pc ^ sw), dst + 1024 * t);
  }
}

// issue_mat for a tile that lies wholly below kv_len (no key is clamped):
// an instruction's RPI rows are then consecutive slots of one page, so the
// lane's source offset splits into a scalar part (page base and the first
// row's slot, folded into the SGPR base) and a per-lane constant (the row
// inside the group and the swizzled chunk), computed once per kernel.  No
// vector instruction per gather.  Needs page bytes (2 s_page) < 2^32 and page
// ids >= 0.
// Swz::f(r): the chunk swizzle of key row r in the destination layout.
template <int D>
struct SwzK {
  __device__ static constexpr int f(int r) { return Stage<D>::fk(r); }
};
template <int D>
struct SwzV {
  __device__ static constexpr int f(int r) { return Stage<D>::fv(r); }
};

template <int D, int NW, typename Swz>
struct LaneGather {
  static constexpr int CH = KvDma<D, NW>::CH, IPW = KvDma<D, NW>::IPW, RPI = KvDma<D, NW>::RPI;
  uint32_t off[IPW];
  __device__ __forceinline__ LaneGather(int wave, int lane, int64_t s_slot) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int t = wave * IPW + i;
      const int r = RPI * t + lane / CH, pc = lane % CH;
      off[i] = (uint32_t)((lane / CH) * (int)s_slot) * 2 + 16 * (pc ^ Swz::f(r));
    }
  }
};

// CLAMP: the tile may reach past kv_len; keys past it are clamped to the last
// key, which lies in the page of the instruction's first row (pages hold a
// multiple of RPI keys, and a group is clamped only where it starts at or
// before the last key or lies wholly past it, when pages_uniform took the
// last key's page), so only the lane's slot moves: by (clamped key -
// unclamped key) slots, a few vector instructions on the last tile only.
template <int D, int NW, typename Swz, bool CLAMP>
__device__ __forceinline__ void issue_mat_fast(const uint16_t *base, const typename KvDma<D, NW>::Pages &pg,
                                               const LaneGather<D, NW, Swz> &lg, int page_shift,
                                               uint32_t page_bytes, uint32_t slot_bytes, int kt, int kv_len,
                                               uint32_t dst, int wave, int lane) {
  constexpr int IPW = KvDma<D, NW>::IPW, RPI = KvDma<D, NW>::RPI, CH = KvDma<D, NW>::CH;
  const int pmask = (1 << page_shift) - 1;
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int t = wave * IPW + i;
    const int key0 = kt * 64 + RPI * t;
    uint32_t voff = lg.off[i];
    int k0 = key0;
    if constexpr (CLAMP) {
      // rows of a group wholly past the last key all read the last key
      k0 = min(key0, kv_len - 1);
      const int key = min(key0 + lane / CH, kv_len - 1);
      voff += (uint32_t)((key - k0 - lane / CH) * (int)slot_bytes);
    }
    const uint32_t row0 = (uint32_t)(k0 & pmask);
    const uint64_t off = (uint64_t)(uint32_t)pg.id[i] * page_bytes + row0 * slot_bytes;
    lds_load16_s((gptr_t)((const char *)base + off), voff, dst + 1024 * t);
  }
}

// issue_mat_fast without clamping for pages of at least RPI * IPW keys: the
// rows of this wave's IPW instructions then lie in one page (an aligned run
// of RPI * IPW keys), so one page id and one scalar base serve all of them
// and each further instruction adds a constant: two scalar adds and the M0
// write per gather.
template <int D, int NW, typename Swz>
__device__ __forceinline__ void issue_mat_page(const uint16_t *base, int32_t page_id,
                                               const LaneGather<D, NW, Swz> &lg, int page_shift,
                                               uint32_t page_bytes, uint32_t slot_bytes, int kt, uint32_t dst,
                                               int wave) {
  constexpr int IPW = KvDma<D, NW>::IPW, RPI = KvDma<D, NW>::RPI;
  const int pmask = (1 << page_shift) - 1;
  const uint32_t row0 = (uint32_t)((kt * 64 + RPI * IPW * wave) & pmask);
  const char *b0 = (const char *)base + ((uint64_t)(uint32_t)page_id * page_bytes + row0 * slot_bytes);
#pragma unroll
  for (int i = 0; i < IPW; ++i)
    lds_load16_s((gptr_t)(b0 + (uint64_t)(i * RPI) * slot_bytes), lg.off[i], dst + 1024 * (wave * IPW + i));
}

// Waits for this wave's outstanding global loads (the LDS gathers among them).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Per-lane LDS offsets (elements) of the matrix-core operand reads; the
// swizzle makes them lane-dependent, so they are computed once per kernel.
template <int D>
struct LaneOffsets {
  static constexpr int NK = D / 16 < 8 ? D / 16 : 8;   // distinct K operand offsets
  static constexpr int NV = D / 32 < 4 ? D / 32 : 4;   // distinct V operand offsets
  int k[NK];     // K operand x: chunk (2 x + hi) of row l32 -> in-row element offset
  int krow;      // l32 * D
  int v[NV];     // V operand n: chunk 4 n + 2 (g % 2) + q / 2 of row r -> in-row element offset
  int vrow;      // r * D, r = 4 (lane / 32) + (lane % 16) / 4
  __device__ __forceinline__ explicit LaneOffsets(int lane) {
    const int l32 = lane & 31, hi = lane >> 5;
    const int f = Stage<D>::fk(l32);   // the same for rows l32 and l32 + 32
#pragma unroll
    for (int x = 0; x < NK; ++x) k[x] = 8 * ((2 * x + hi) ^ f);
    krow = l32 * D;
    const int g = lane >> 4, s = lane & 15, j = s >> 2, q = s & 3;
    const int r = 4 * (g >> 1) + j;    // row offset from the product's base row (a multiple of 4)
    const int fvr = Stage<D>::fv(r);   // the same for every base and for base + 8
#pragma unroll
    for (int n = 0; n < NV; ++n) v[n] = 8 * ((4 * n + 2 * (g & 1) + (q >> 1)) ^ fvr) + 4 * (q & 1);
    vrow = r * D;
  }
  // K operand element offset of product x (0 .. D/16-1) inside a row: the
  // swizzle only touches the low 4 chunk bits, so x >= 8 adds 16 chunks.
  __device__ __forceinline__ int kop(int x) const { return x < 8 ? k[x] : k[x - 8] + 128; }
  // V operand element offset of d-block n inside a row (n >= 4 adds 16 chunks
  // per 4 blocks for the same reason).
  __device__ __forceinline__ int vop(int n) const { return n < 4 ? v[n] : v[n - 4] + 128; }
};

// S^T = K Q^T for keys [0, 64) of the staged tile and the wave's 32 query
// rows.  Operands are read in register-budget-sized groups before their
// products (sched_barrier keeps the compiler from sinking each read onto its
// use): both 32-key blocks for d <= 128, half a block for d = 256.
template <int D, int GROUP = (D <= 128 ? 2 * (D / 16) : 8)>
__device__ __forceinline__ void qk_tile(const uint16_t *stage, const LaneOffsets<D> &lo, const bf16x8 (&qf)[D / 16],
                                        f32x16 (&s)[2]) {
  constexpr int NG = 2 * (D / 16) / GROUP;
  const uint16_t *kl = stage + lo.krow;
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    bf16x8 a[GROUP];
#pragma unroll
    for (int x = 0; x < GROUP; ++x) {
      const int idx = gi * GROUP + x, kb = idx / (D / 16), k = idx % (D / 16);
      a[x] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(kl + 32 * kb * D + lo.kop(k)));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int x = 0; x < GROUP; ++x) {
      const int idx = gi * GROUP + x, kb = idx / (D / 16), k = idx % (D / 16);
      if (k == 0) s[kb] = f32x16{};
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[x], qf[k], s[kb], 0, 0, 0);
    }
  }
}

// O^T += V^T P^T.  P leaves the S^T accumulator as the B operand: product u
// takes registers 8 (u % 2) .. + 7 of score block u / 2, i.e. keys
// base + 8 (e/4) + 4 (l/32) + e % 4 for element e, base = 32 (u/2) + 16 (u%2).
// The V^T operand is read straight from row-major V with ds_read_b64_tr_b16:
// inside each 16-lane group, lane i receives element i % 4 of the 8 bytes
// addressed by lane 4 j + i / 4, as its element j.  Lane 4 j + q addressing
// V[k0 + j][d0 + 4 q .. + 3] therefore hands lane i the keys k0 .. k0 + 3 of
// head-dim d0 + i; two such reads (k0 = base + 4 (l/32) and base + 8 +
// 4 (l/32), d0 = 32 n + 16 (l/16 % 2)) form the lane's 8 operand elements.
template <int D>
__device__ __forceinline__ void read_vt(const uint16_t *stage, const LaneOffsets<D> &lo, bf16x8 (&a)[D / 32],
                                        int u) {
  const uint16_t *p = stage + Stage<D>::V_OFF + lo.vrow + (32 * (u >> 1) + 16 * (u & 1)) * D;
#pragma unroll
  for (int n = 0; n < D / 32; ++n) {
    const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4 *)(p + lo.vop(n)));
    const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4 *)(p + 8 * D + lo.vop(n)));
    const i16x8 v = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
    a[n] = __builtin_bit_cast(bf16x8, v);
  }
}

// lsum accumulates the lane's share of its query-row sum (the 32 keys of the
// tile this lane's half holds), over exactly the bf16 probabilities that
// enter P V: v_dot2_f32_bf16 against (1, 1) adds two of them per vector
// instruction, which keeps the matrix cores for the products.  The two
// halves of a row are added once, at the end.  V^T operands of
// product u + 1 are read while product u runs (d <= 128); d = 256 reads each
// product's operands just before it (register budget).
template <int D>
__device__ __forceinline__ void pv_tile(const uint16_t *stage, const LaneOffsets<D> &lo, const f32x16 (&p)[2],
                                        f32x16 (&o)[D / 32], float &lsum) {
  constexpr int NB = D <= 128 ? 2 : 1;
  bf16x8 a[NB][D / 32];
  if (NB == 2) read_vt<D>(stage, lo, a[0], 0);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (NB == 2 && u + 1 < 4) read_vt<D>(stage, lo, a[(u + 1) % NB], u + 1);
    if (NB == 1) read_vt<D>(stage, lo, a[0], u);
    f32x8 pv;
#pragma unroll
    for (int x = 0; x < 8; ++x) pv[x] = p[u >> 1][8 * (u & 1) + x];
    const bf16x8 pb = __builtin_convertvector(pv, bf16x8);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int n = 0; n < D / 32; ++n) o[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u % NB][n], pb, o[n], 0, 0, 0);
    lsum = row_sum_bf16(pb, lsum);
  }
}

// S^T = K Q^T as qk_tile, without scheduling fences: the software-pipelined
// kernel lets the compiler interleave these products with the previous
// tile's softmax.
template <int D>
__device__ __forceinline__ void qk_tile_free(const uint16_t *stage, const LaneOffsets<D> &lo,
                                             const bf16x8 (&qf)[D / 16], f32x16 (&s)[2]) {
  const uint16_t *kl = stage + lo.krow;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    s[kb] = f32x16{};
#pragma unroll
    for (int k = 0; k < D / 16; ++k) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4 *)(kl + 32 * kb * D + lo.kop(k)));
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[k], s[kb], 0, 0, 0);
    }
  }
}

// P (the exponentiated S^T accumulators) as the four bf16 B operands of
// O^T += V^T P^T (operand u: registers 8 (u % 2) .. + 7 of block u / 2), and
// ps = the lane's sum of exactly those bf16 values (v_dot2_f32_bf16).
__device__ __forceinline__ void pack_p(const f32x16 (&p)[2], bf16x8 (&pb)[4], float &ps) {
  ps = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    f32x8 pv;
#pragma unroll
    for (int x = 0; x < 8; ++x) pv[x] = p[u >> 1][8 * (u & 1) + x];
    pb[u] = __builtin_convertvector(pv, bf16x8);
    ps = row_sum_bf16(pb[u], ps);
  }
}

// O^T += V^T P^T from packed operands (pack_p); the V^T operands of product
// u + 1 are read while product u runs.
template <int D>
__device__ __forceinline__ void pv_tile_packed(const uint16_t *stage, const LaneOffsets<D> &lo,
                                               const bf16x8 (&pb)[4], f32x16 (&o)[D / 32]) {
  static_assert(D <= 128, "packed P V reads two products' operands ahead");
  bf16x8 a[2][D / 32];
  read_vt<D>(stage, lo, a[0], 0);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (u + 1 < 4) read_vt<D>(stage, lo, a[(u + 1) & 1], u + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int n = 0; n < D / 32; ++n) o[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u & 1][n], pb[u], o[n], 0, 0, 0);
  }
}

}  // namespace dma
}  // namespace dev
}  // namespace maskattn
