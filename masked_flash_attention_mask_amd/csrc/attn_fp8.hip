// Masked flash-attention prefill with fp8 (OCP e4m3) Q, K and V over a
// compiled plan (gfx950): the fp8 question of flashinfer issue 724 (its
// closing questions ask when fp8 comes to FA3).  Same plan walk, masking and
// online softmax as the bf16 kernel; the two products run on the fp8 matrix
// cores (v_mfma_scale_f32_32x32x64_f8f6f4, unit block scales):
//   S^T = K Q^T   A = K rows from LDS, B = Q rows in registers, 64 of d per
//                 instruction
//   O^T += V^T P^T   P is rounded to e4m3 (round to nearest even) in the
//                 S^T accumulator layout and used as B; V^T comes from
//                 row-major V in LDS through the transposing byte load
//                 ds_read_b64_tr_b8; 64 keys per instruction
// Per-tensor descale factors: S = scale * q_descale * k_descale * (Q8 . K8)
// and O = v_descale * (P V8) / rowsum(P).  The row sums run on the matrix
// cores too (an all-ones A operand), so they add exactly the e4m3
// probabilities that enter P V.
//
// Operand layout of the fp8 32x32x64 product (checked on the device): lane l
// holds row (A) / column (B) l % 32 and the 32 bytes of K-slots half l / 32;
// byte b of a lane pairs with byte b of the other operand's lane of the same
// half.  The K-slot labels are therefore free: for S^T a lane's 32 bytes are
// 32 consecutive d of its row (two 16-byte reads); for P V a lane half's
// bytes are the 32 keys that half holds in the S^T accumulator, byte
// 16 kb + r for register r of key block kb.
// ds_read_b64_tr_b8 (checked on the device): inside each 16-lane group, lane
// i receives byte i % 8 of the 8 bytes addressed by lane 2 j + i / 8 as its
// byte j (j = 0..7).
#include <hip/hip_runtime.h>

#include "internal.h"
#include "kernels_common.h"
#include "tile_dma_bf16.h"

namespace maskattn {
using namespace dev;

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

struct Fp8Params {
  const SeqInfo *seqs;
  const Item *items;
  const Entry *entries;
  const uint64_t *words;
  const uint8_t *q, *k, *v;
  const int32_t *page_table;
  void *out;
  float *lse;
  int64_t s_page, s_slot, s_head;
  int32_t max_pages, page_shift;
  int32_t hq, group, num_items;
  float c;          // scale * q_descale * k_descale * log2 e
  float v_descale;
};

// LDS stage of one 64-key tile: K and V, each [64 keys][D bytes] unpadded,
// 16-byte chunks XOR-swizzled by the key row.  K's swizzle puts the 16 rows
// of an operand read (ds_read_b128) on distinct banks; V's puts the 8 rows x
// 2 chunks of a half-wave's transposing reads on distinct banks.
template <int D>
struct Fp8Stage {
  static constexpr int CH = D / 16;        // 16-byte chunks per row
  static constexpr int V_OFF = 64 * D;     // bytes
  static constexpr int BYTES = 2 * 64 * D;
  static constexpr int RPI = 64 / CH;      // key rows per gather instruction
  __host__ __device__ static constexpr int fk(int r) { return CH >= 8 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
  __host__ __device__ static constexpr int fv(int r) {
    return CH >= 8 ? (2 * ((r >> 1) & 1) + 4 * ((r >> 3) & 1)) : 2 * ((r >> 3) & 1);
  }
};

__device__ __forceinline__ Entry load_entry(const Entry *e, int i) {
  const __attribute__((address_space(4))) Entry *c = (const __attribute__((address_space(4))) Entry *)e;
  return Entry{c[i].kt_cls, c[i].wblk};
}

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8 &a, const i32x8 &b, const f32x16 &c) {
  // format 0 (e4m3) for both operands, block scales 127 (2^0)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0x7F7F7F7F, 0, 0x7F7F7F7F);
}

// Gather of one 64-key tile's K or V by NW waves into an LDS slot: wave
// instruction t fills LDS chunks [64 t, 64 t + 64), lane l the chunk of row
// RPI t + l / CH, chunk l % CH (source side swizzled).  The RPI rows of an
// instruction lie in one page (a scalar page id), so the source is a scalar
// base plus a 32-bit lane offset; for tiles inside kv_len that offset is a
// per-lane constant (off[i], the row inside the group and the swizzled
// chunk) and the page and first row go into the scalar base.  Keys past
// kv_len (the last tile) repeat the last key: they lie in the page of the
// group's first row, so only the lane's slot moves.
template <int D, int NW, bool IS_V>
struct Fp8Gather {
  using St = Fp8Stage<D>;
  static constexpr int IPW = St::CH / NW;   // instructions per wave
  static constexpr int RUN = St::RPI * IPW; // keys one wave gathers
  static_assert(St::CH % NW == 0, "gather needs CH to be a multiple of the wave count");
  uint32_t off[IPW];
  __device__ __forceinline__ Fp8Gather(int wave, int lane, uint32_t slot_bytes) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int t = wave * IPW + i;
      const int r = St::RPI * t + lane / St::CH, pc = lane % St::CH;
      off[i] = (uint32_t)(lane / St::CH) * slot_bytes + 16 * (pc ^ (IS_V ? St::fv(r) : St::fk(r)));
    }
  }
  struct Pages {
    int32_t id[IPW];
  };
  __device__ __forceinline__ static Pages pages(const int32_t *pt, int page_shift, int kt, int kv_len, int wave) {
    const __attribute__((address_space(4))) int32_t *cpt = (const __attribute__((address_space(4))) int32_t *)pt;
    Pages pg;
#pragma unroll
    for (int i = 0; i < IPW; ++i) pg.id[i] = cpt[min(kt * 64 + St::RPI * (wave * IPW + i), kv_len - 1) >> page_shift];
    return pg;
  }
  __device__ __forceinline__ void issue(const uint8_t *base, const Pages &pg, int page_shift, uint32_t page_bytes,
                                        uint32_t slot_bytes, int kt, int kv_len, uint32_t dst, int wave,
                                        int lane) const {
    const int pmask = (1 << page_shift) - 1;
    if (kt * 64 + 64 <= kv_len && page_shift >= __builtin_ctz(RUN)) {
      // one page for the wave's whole run of keys
      const uint32_t row0 = (uint32_t)((kt * 64 + RUN * wave) & pmask);
      const uint8_t *b0 = base + ((uint64_t)(uint32_t)pg.id[0] * page_bytes + row0 * slot_bytes);
#pragma unroll
      for (int i = 0; i < IPW; ++i)
        dma::lds_load16_s((dma::gptr_t)(b0 + (uint64_t)(i * St::RPI) * slot_bytes), off[i],
                          dst + 1024 * (wave * IPW + i));
      return;
    }
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int t = wave * IPW + i;
      const int key0 = kt * 64 + St::RPI * t;
      const int k0 = min(key0, kv_len - 1);
      const int key = min(key0 + lane / St::CH, kv_len - 1);
      const uint32_t voff = off[i] + (uint32_t)((key - k0 - lane / St::CH) * (int)slot_bytes);
      const uint32_t row0 = (uint32_t)(k0 & pmask);
      const uint8_t *b = base + ((uint64_t)(uint32_t)pg.id[i] * page_bytes + row0 * slot_bytes);
      dma::lds_load16_s((dma::gptr_t)b, voff, dst + 1024 * t);
    }
  }
};

// LDS: K slots 0 and 1, then V slots 0 and 1, each [64 keys][D bytes].
template <int D>
struct Fp8Lds {
  static constexpr int SLOT = 64 * D;
  static constexpr int V0 = 2 * SLOT;
  static constexpr int BYTES = 4 * SLOT;
};

// Waves per SIMD: two; one at d = 256, whose O accumulators alone take 128
// registers per lane.
template <int D>
constexpr int fp8_occupancy() {
  return D == 256 ? 1 : 2;
}

template <int D, typename OutT>
__global__ __launch_bounds__(256, (fp8_occupancy<D>())) void prefill_fp8_kernel(Fp8Params p) {
  constexpr int BQ = 128, NW = 4;
  using St = Fp8Stage<D>;
  using L = Fp8Lds<D>;
  using GK = Fp8Gather<D, NW, false>;
  using GV = Fp8Gather<D, NW, true>;
  constexpr int KS = D / 64;                 // k-steps of S^T
  extern __shared__ __align__(16) uint8_t lds8[];
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

  // Q row as B operands: step s holds d 64 s + 32 hi .. + 31
  i32x8 qf[KS];
  {
    const uint8_t *qrow = p.q + (tok * p.hq + h) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4 a = row_ok ? *(const u32x4 *)(qrow + 64 * s + 32 * hi) : u32x4{0, 0, 0, 0};
      const u32x4 b = row_ok ? *(const u32x4 *)(qrow + 64 * s + 32 * hi + 16) : u32x4{0, 0, 0, 0};
      qf[s] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
    }
  }
  const uint8_t *kbase = p.k + (int64_t)g * p.s_head;
  const uint8_t *vbase = p.v + (int64_t)g * p.s_head;
  const int32_t *pt = p.page_table + (int64_t)it.seq * p.max_pages;
  const uint32_t page_bytes = (uint32_t)p.s_page, slot_bytes = (uint32_t)p.s_slot;
  const GK gk(wave, lane, slot_bytes);
  const GV gv(wave, lane, slot_bytes);

  // Per-lane LDS offsets.  K rows 32 kb + l32, chunks 4 s + 2 hi (+1).
  const int krow = l32 * D;
  const int kf = St::fk(l32);   // the same for rows l32 and l32 + 32
  // V^T: source lane s16 = lane % 16 of group G = lane / 16 loads row
  // 16 t + 8 (s16 / 8) + 4 hi + (s16 / 2) % 4 at byte 32 n + 16 (G % 2) +
  // 8 (s16 % 2); the swizzle depends on the row through bits 1 and 3 only.
  const int s16 = lane & 15, G = lane >> 4;
  const int vr = 8 * (s16 >> 3) + 4 * hi + ((s16 >> 1) & 3);
  const int vq = G & 1, vb = 8 * (s16 & 1);
  const int vfv = St::fv(vr);

  auto load_word = [&](Entry e) -> uint64_t {
    if (entry_cls(e.kt_cls) != MA_TILE_PARTIAL) return 0ull;
    return p.words[(int64_t)e.wblk * BQ + wrow];
  };
  // S^T = K Q^T of the K tile at LDS byte offset kslot
  auto qk = [&](int kslot, f32x16 (&sacc)[2]) {
    const uint8_t *ks = lds8 + kslot;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16{};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const uint8_t *row = ks + 32 * kb * D + krow;
        const u32x4 a = *(const u32x4 *)(row + 16 * ((4 * s + 2 * hi) ^ kf));
        const u32x4 b = *(const u32x4 *)(row + 16 * ((4 * s + 2 * hi + 1) ^ kf));
        const i32x8 ka = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
        sacc[kb] = mfma_fp8(ka, qf[s], sacc[kb]);
      }
    }
  };
  f32x16 oacc[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n) oacc[n] = f32x16{};
  f32x16 lacc = f32x16{};
  const i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                      0x38383838, 0x38383838, 0x38383838, 0x38383838};
  // O^T += V^T P^T and the row sums += ones P^T, V from LDS byte offset vslot
  auto pv = [&](int vslot, const i32x8 &pb) {
    const uint8_t *vs = lds8 + vslot;
#pragma unroll
    for (int n = 0; n < D / 32; ++n) {
      i32x8 va;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int row = 16 * t + vr;   // the swizzle of row 16 t + vr equals that of vr
        const uint8_t *src = vs + row * D + 16 * ((2 * n + vq) ^ vfv) + vb;
        const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2 *)src);
        va[2 * t] = x[0];
        va[2 * t + 1] = x[1];
      }
      oacc[n] = mfma_fp8(va, pb, oacc[n]);
    }
    lacc = mfma_fp8(ones, pb, lacc);
  };
  float m_ref = neg_inf();
  const float c = p.c;

  // Software pipeline over the item's tiles: step j runs the softmax of tile
  // j beside the products S^T of tile j + 1 and O^T += V^T P^T of tile j - 1
  // (all independent of it), so the vector work of a tile sits between
  // matrix instructions.  K(t) is gathered at step t - 2, V(t) at step t; step
  // j reads K(j + 1) from K slot (j + 1) % 2 and V(j - 1) from V slot
  // (j - 1) % 2 while K(j + 2) and V(j) are written to the other slots.  Each
  // step ends with a wait for the wave's gathers and a workgroup barrier.
  const uint32_t lds0 = dma::lds_addr(lds8);
  const int eb = it.ent_begin, n = it.ent_end - it.ent_begin;
  auto kt_of = [&](int j) { return entry_kt(load_entry(p.entries, eb + j).kt_cls); };
  typename GK::Pages pk_a;                   // pages of K(j + 2) at the start of step j
  typename GV::Pages pv_a;                   // pages of V(j)
  uint64_t word_cur = 0, word_nxt = 0;
  f32x16 sa[2], sb[2];
  i32x8 p_prev = i32x8{};
  if (n > 0) {
    // V slot 1 is read (with P = 0) at step 0: clear it so that stale bytes
    // (NaN codes) cannot reach the accumulators
    for (int x = tid; x < L::SLOT / 16; x += 256) *(u32x4 *)(lds8 + L::V0 + L::SLOT + 16 * x) = u32x4{0, 0, 0, 0};
    gk.issue(kbase, GK::pages(pt, p.page_shift, kt_of(0), kv_len, wave), p.page_shift, page_bytes, slot_bytes,
             kt_of(0), kv_len, lds0, wave, lane);
    if (n > 1)
      gk.issue(kbase, GK::pages(pt, p.page_shift, kt_of(1), kv_len, wave), p.page_shift, page_bytes, slot_bytes,
               kt_of(1), kv_len, lds0 + L::SLOT, wave, lane);
    if (n > 2) pk_a = GK::pages(pt, p.page_shift, kt_of(2), kv_len, wave);
    pv_a = GV::pages(pt, p.page_shift, kt_of(0), kv_len, wave);
    word_cur = load_word(load_entry(p.entries, eb));
    if (n > 1) word_nxt = load_word(load_entry(p.entries, eb + 1));
    dma::wait_vmem();
    __syncthreads();
    qk(0, sa);
    if (n > 2) __syncthreads();   // every wave has read K(0) before K(2) replaces it
  }
  auto step = [&](f32x16 (&scur)[2], f32x16 (&snxt)[2], int j) {
    const int cur = j & 1;
    const Entry ec = load_entry(p.entries, eb + j);
    const uint64_t wcur = word_cur;
    if (j + 2 < n)
      gk.issue(kbase, pk_a, p.page_shift, page_bytes, slot_bytes, kt_of(j + 2), kv_len,
               lds0 + (uint32_t)(cur * L::SLOT), wave, lane);
    gv.issue(vbase, pv_a, p.page_shift, page_bytes, slot_bytes, kt_of(j), kv_len,
             lds0 + (uint32_t)(L::V0 + cur * L::SLOT), wave, lane);
    word_cur = word_nxt;
    if (j + 2 < n) word_nxt = load_word(load_entry(p.entries, eb + j + 2));
    if (j + 1 < n) pv_a = GV::pages(pt, p.page_shift, kt_of(j + 1), kv_len, wave);
    if (j + 3 < n) pk_a = GK::pages(pt, p.page_shift, kt_of(j + 3), kv_len, wave);
    const int kt = entry_kt(ec.kt_cls);
    const int cls = entry_cls(ec.kt_cls);
    const int kin = kv_len - kt * 64;
    if (cls == MA_TILE_PARTIAL || kin < 64)
      apply_word(scur, (cls == MA_TILE_PARTIAL ? wcur : ~0ull) & low_bits(kin), hi);
    // unconditional: at the last step S^T of a tile past the end is unused
    qk((cur ^ 1) * L::SLOT, snxt);
    pv(L::V0 + (cur ^ 1) * L::SLOT, p_prev);
    float alpha;
    const bool any = softmax_tile(scur, m_ref, c, alpha);
    // P -> e4m3 B operand: byte 16 kb + r holds register r of key block kb
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int kb = w >> 2, r = 4 * (w & 3);
      int x = __builtin_amdgcn_cvt_pk_fp8_f32(scur[kb][r], scur[kb][r + 1], 0, false);
      x = __builtin_amdgcn_cvt_pk_fp8_f32(scur[kb][r + 2], scur[kb][r + 3], x, true);
      p_prev[w] = x;
    }
    // keep the softmax in the block of the products above (see the bf16 kernel)
    asm volatile("" : "+v"(p_prev));
    if (any) {
#pragma unroll
      for (int x = 0; x < D / 32; ++x) oacc[x] *= alpha;
      lacc *= alpha;
    }
    dma::wait_vmem();
    __syncthreads();
  };
  for (int j = 0; j < n; j += 2) {
    step(sa, sb, j);
    if (j + 1 < n) step(sb, sa, j + 1);
  }
  if (n > 0) pv(L::V0 + ((n - 1) & 1) * L::SLOT, p_prev);
  const float lt = lacc[0];
  if (!row_ok) return;
  const float inv = lt > 0.f ? p.v_descale / lt : 0.f;
  store_row<D, OutT>((OutT *)p.out + (tok * p.hq + h) * D, oacc, inv, hi);
  if (p.lse && hi == 0) p.lse[tok * p.hq + h] = lt > 0.f ? (m_ref + __log2f(lt)) * kLn2 : neg_inf();
}

template <int D, typename OutT>
ma_status launch_d(const Fp8Params &prm, int grid, void *stream) {
  auto kern = prefill_fp8_kernel<D, OutT>;
  constexpr size_t lds = Fp8Lds<D>::BYTES;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, (hipStream_t)stream, prm);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(MA_ERR_HIP, "fp8 prefill launch: %s", hipGetErrorString(e));
  return MA_OK;
}

}  // namespace

int32_t fp8_rows_per_gather(int32_t d) {
  return d == 64 ? Fp8Stage<64>::RPI : (d == 128 ? Fp8Stage<128>::RPI : Fp8Stage<256>::RPI);
}

ma_status launch_prefill_fp8(const Fp8Args &a) {
  const ma_plan *pl = a.plan;
  Fp8Params prm{};
  const char *base = (const char *)pl->dbuf;
  prm.seqs = (const SeqInfo *)(base + pl->off_seqs);
  prm.items = (const Item *)(base + pl->off_items);
  prm.entries = (const Entry *)(base + pl->off_entries);
  prm.words = (const uint64_t *)(base + pl->off_words);
  prm.q = (const uint8_t *)a.q;
  prm.k = (const uint8_t *)a.k;
  prm.v = (const uint8_t *)a.v;
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
  prm.c = a.scale * a.q_descale * a.k_descale * kLog2e;
  prm.v_descale = a.v_descale;
  const int64_t grid64 = (int64_t)pl->num_rows * a.hq;
  if (grid64 > INT32_MAX) return set_error(MA_ERR_UNSUPPORTED, "grid too large");
  const int grid = (int)grid64;
  const bool f32 = a.out_dtype == MA_F32;
  switch (a.d) {
    case 64: return f32 ? launch_d<64, float>(prm, grid, a.stream) : launch_d<64, uint16_t>(prm, grid, a.stream);
    case 128: return f32 ? launch_d<128, float>(prm, grid, a.stream) : launch_d<128, uint16_t>(prm, grid, a.stream);
    case 256: return f32 ? launch_d<256, float>(prm, grid, a.stream) : launch_d<256, uint16_t>(prm, grid, a.stream);
  }
  return set_error(MA_ERR_UNSUPPORTED, "fp8 head_dim %d (supported: 64, 128, 256)", a.d);
}

}  // namespace maskattn
