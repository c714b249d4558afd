// bf16 tile machinery of the prefill kernel: paged K/V gathered through
// registers (one tile ahead) into the padded LDS stage layout, and the two
// matrix-core products of a wave's 32 query rows against a staged tile.
#pragma once

#include "internal.h"
#include "kernels_common.h"

namespace maskattn {
namespace dev {
namespace staged {

// LDS stage of one 64-key tile: K and V both row-major (bf16).  K rows are
// padded to D + 8 elements (a row stride of 4 banks modulo 64) so the 16 rows
// of one ds_read_b128 operand load hit distinct banks.  V rows are padded to
// D + 32 elements (16 banks modulo 64) so the 4 rows x 32 bytes a 16-lane
// group reads with ds_read_b64_tr_b16 hit distinct banks.  Row-wise gather
// writes (16 lanes fill one row) are conflict-free for both.
template <int D>
struct Stage {
  static constexpr int KS = D + 8;
  static constexpr int VS = D + 32;
  static constexpr int V_OFF = 64 * KS;  // elements
  static constexpr int ELEMS = 64 * KS + 64 * VS;
  static constexpr size_t BYTES = ELEMS * sizeof(uint16_t);
};

// Per-thread share of a tile gather: (4-key group, 16-byte chunk) pairs.
// Keys at or past kv_len are clamped to the last key, so every load is in
// bounds and branch-free: such keys are masked to probability exactly 0, and
// the V rows they read are finite, so they add nothing.  Page-table entries
// are looked up one tile ahead of the K/V loads that use them (pages()), so
// the dependent page-table -> cache load chain never stalls a tile.
template <int D, int NT>
struct KvTile {
  static constexpr int CH = D / 8;
  static constexpr int PAIRS = 16 * CH;
  static constexpr int PPT = (PAIRS + NT - 1) / NT;
  u32x4 kreg[PPT][4];
  u32x4 vreg[PPT][4];

  struct Pages {
    int32_t id[PPT][4];
  };

  // Page of each key this thread gathers for tile kt (one per 4-key group
  // when pages hold at least 4 keys).
  __device__ __forceinline__ Pages pages(const int32_t *pt, int page_shift, int kt, int kv_len, int tid) const {
    Pages pg;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int pair = tid + i * NT;
      const int kg = (PAIRS % NT == 0 || pair < PAIRS ? pair : 0) / CH;
      const int key0 = kt * 64 + 4 * kg;
      if (page_shift >= 2) {
        pg.id[i][0] = pt[min(key0, kv_len - 1) >> page_shift];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) pg.id[i][j] = pt[min(key0 + j, kv_len - 1) >> page_shift];
      }
    }
    return pg;
  }

  __device__ __forceinline__ void load(const uint16_t *kbase, const uint16_t *vbase, const Pages &pg,
                                       int page_shift, int64_t s_page, int64_t s_slot, int kt, int kv_len,
                                       int tid) {
    const int pmask = (1 << page_shift) - 1;
    if (page_shift >= 2 && (kt + 1) * 64 <= kv_len) {
      // Interior tile: the 4 keys of a group are consecutive slots of one page.
#pragma unroll
      for (int i = 0; i < PPT; ++i) {
        const int pair = tid + i * NT;
        if (PAIRS % NT == 0 || pair < PAIRS) {
          const int kg = pair / CH, c = pair % CH;
          const int key0 = kt * 64 + 4 * kg;
          const int64_t off0 = (int64_t)pg.id[i][0] * s_page + (int64_t)(key0 & pmask) * s_slot + 8 * c;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            kreg[i][j] = *(const u32x4 *)(kbase + off0 + j * s_slot);
            vreg[i][j] = *(const u32x4 *)(vbase + off0 + j * s_slot);
          }
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int pair = tid + i * NT;
      if (PAIRS % NT == 0 || pair < PAIRS) {
        const int kg = pair / CH, c = pair % CH;
        const int key0 = kt * 64 + 4 * kg;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = min(key0 + j, kv_len - 1);
          const int32_t page = page_shift >= 2 ? pg.id[i][0] : pg.id[i][j];
          const int64_t off = (int64_t)page * s_page + (int64_t)(key & pmask) * s_slot + 8 * c;
          kreg[i][j] = *(const u32x4 *)(kbase + off);
          vreg[i][j] = *(const u32x4 *)(vbase + off);
        }
      }
    }
  }
  // Split gather for tight register budgets: K and V staged one after the
  // other through the same registers (kreg).
  __device__ __forceinline__ void load_one(const uint16_t *base, const Pages &pg, int page_shift, int64_t s_page,
                                           int64_t s_slot, int kt, int kv_len, int tid) {
    const int pmask = (1 << page_shift) - 1;
    const bool interior = page_shift >= 2 && (kt + 1) * 64 <= kv_len;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int pair = tid + i * NT;
      if (PAIRS % NT == 0 || pair < PAIRS) {
        const int kg = pair / CH, c = pair % CH;
        const int key0 = kt * 64 + 4 * kg;
        if (interior) {
          const int64_t off0 = (int64_t)pg.id[i][0] * s_page + (int64_t)(key0 & pmask) * s_slot + 8 * c;
#pragma unroll
          for (int j = 0; j < 4; ++j) kreg[i][j] = *(const u32x4 *)(base + off0 + j * s_slot);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int key = min(key0 + j, kv_len - 1);
            const int32_t page = page_shift >= 2 ? pg.id[i][0] : pg.id[i][j];
            kreg[i][j] = *(const u32x4 *)(base + (int64_t)page * s_page + (int64_t)(key & pmask) * s_slot + 8 * c);
          }
        }
      }
    }
  }

  __device__ __forceinline__ void store_one(uint16_t *dst, int stride, int tid) const {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int pair = tid + i * NT;
      if (PAIRS % NT == 0 || pair < PAIRS) {
        const int kg = pair / CH, c = pair % CH;
#pragma unroll
        for (int j = 0; j < 4; ++j) *(u32x4 *)(dst + (4 * kg + j) * stride + 8 * c) = kreg[i][j];
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t *stage, int tid) const {
    uint16_t *Vs = stage + Stage<D>::V_OFF;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int pair = tid + i * NT;
      if (PAIRS % NT == 0 || pair < PAIRS) {
        const int kg = pair / CH, c = pair % CH;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          *(u32x4 *)(stage + (4 * kg + j) * Stage<D>::KS + 8 * c) = kreg[i][j];
          *(u32x4 *)(Vs + (4 * kg + j) * Stage<D>::VS + 8 * c) = vreg[i][j];
        }
      }
    }
  }
};

// S^T for keys [0, 64) of the staged tile and the wave's 32 query rows.
// The operand reads of both 32-key blocks are issued before the products
// (sched_barrier keeps the compiler from sinking each read onto its use), so
// LDS latency overlaps the matrix cores instead of preceding every product.
template <int D>
__device__ __forceinline__ void qk_tile(const uint16_t *stage, const bf16x8 (&qf)[D / 16], f32x16 (&s)[2],
                                        int l32, int hi) {
  // Operands read ahead per group of products: both 32-key blocks (64
  // registers) for d <= 128; half a block (32 registers) for d = 256, whose
  // accumulators already fill most of the register file.
  constexpr int GROUP = D <= 128 ? 2 * (D / 16) : 8;
  constexpr int NG = 2 * (D / 16) / GROUP;
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    bf16x8 a[GROUP];
#pragma unroll
    for (int x = 0; x < GROUP; ++x) {
      const int idx = gi * GROUP + x, kb = idx / (D / 16), k = idx % (D / 16);
      a[x] = __builtin_bit_cast(bf16x8,
                                *(const u32x4 *)(stage + (32 * kb + l32) * Stage<D>::KS + 8 * hi + 16 * k));
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
__device__ __forceinline__ void read_vt(const uint16_t *vlane, bf16x8 (&a)[D / 32], int u) {
  // vlane = V + (4 (lane / 32) + (lane % 16) / 4) * VS + 16 ((lane / 16) % 2) + 4 (lane % 4)
  const uint16_t *p = vlane + (32 * (u >> 1) + 16 * (u & 1)) * Stage<D>::VS;
  typedef short i16x8 __attribute__((ext_vector_type(8)));
#pragma unroll
  for (int n = 0; n < D / 32; ++n) {
    const i16x4 r0 =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(p + 32 * n));
    const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4 *)(p + 8 * Stage<D>::VS + 32 * n));
    const i16x8 v = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
    a[n] = __builtin_bit_cast(bf16x8, v);
  }
}

// lsum accumulates the lane's share of its query-row sum over exactly the
// bf16 probabilities that enter P V (see row_sum_bf16); the two halves of a
// row are added at the end.
template <int D>
__device__ __forceinline__ void pv_tile(const uint16_t *stage, const f32x16 (&p)[2], f32x16 (&o)[D / 32],
                                        float &lsum, int l32, int hi) {
  const int lane = 32 * hi + l32;
  const uint16_t *vlane = stage + Stage<D>::V_OFF + (4 * hi + ((lane & 15) >> 2)) * Stage<D>::VS +
                          16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  // V^T operands of product u + 1 are read while product u runs (d <= 128);
  // d = 256 reads each product's operands just before it (register budget).
  constexpr int NB = D <= 128 ? 2 : 1;
  bf16x8 a[NB][D / 32];
  if (NB == 2) read_vt<D>(vlane, a[0], 0);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (NB == 2 && u + 1 < 4) read_vt<D>(vlane, a[(u + 1) % NB], u + 1);
    if (NB == 1) read_vt<D>(vlane, a[0], u);
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

}  // namespace staged
}  // namespace dev
}  // namespace maskattn
