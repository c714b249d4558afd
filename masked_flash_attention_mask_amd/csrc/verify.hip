// Small-q attention over paged K/V (gfx950): speculative tree verify and
// masked decode.  Every sequence's few queries (q_len <= 64) attend to its
// cached keys under a per-row mask:
//  * a full-row custom mask that changes every decoding step (tree attention
//    through a custom mask, flashinfer issue 724), dense bytes or packed
//    words, or
//  * a closed form evaluated per row from its position pos = t + kv_len -
//    q_len: causal (keys <= pos), sliding window (pos - W < key <= pos),
//    prefixLM (keys <= pos or < P).
//
// Rows: the (query head, query) pairs of one GQA group are packed 32 to a
// wave, head-major, max_q row slots per head.  A workgroup takes GH heads of
// a group, so each K/V tile gathered from the paged cache serves all of
// their queries: a 64-node tree over 4 heads fills 8 waves; a single-token
// decode over a group of 8 heads fills 8 rows of one wave.
//
// The mask is turned into each row's 64-bit word per tile on the fly (a
// packed word is one load; a dense row's 64 bytes are one coalesced load
// and a wavefront ballot; a closed form is a bit interval), and a wave
// whose rows all see the whole tile skips masking.  A sliding window starts
// the walk at the first tile any row can see.  Long contexts are cut into
// contiguous k-tile ranges handled by separate workgroups; each writes a
// partial (O, LSE) and a second kernel merges the partials in fixed split
// order (deterministic, no atomics).
#include <hip/hip_runtime.h>

#include <climits>
#include <mutex>
#include <type_traits>

#include "internal.h"
#include "kernels_common.h"
#include "tile_dma_bf16.h"

namespace maskattn {
using namespace dev;
using namespace dev::dma;

namespace {

constexpr int kTargetWorkgroups = 512;
// Waves of a wave-split decode workgroup over e4m3 caches at d = 128.
constexpr int kDecodeWaves128 = 5;

enum MaskMode : int32_t { kDense = 0, kPacked = 1, kCausal = 2, kWindow = 3, kPrefix = 4 };

struct SplitShape {
  int tiles_per_split;
  int max_splits;
};

// Splits of a walk of at most max_tiles k-tiles so that about
// kTargetWorkgroups workgroups run.
SplitShape split_shape(int units, int max_tiles, int target = kTargetWorkgroups) {
  if (max_tiles < 1) return SplitShape{1, 1};
  int want = (target + units - 1) / units;
  want = want < 1 ? 1 : (want > max_tiles ? max_tiles : want);
  const int t = (max_tiles + want - 1) / want;
  return SplitShape{t, (max_tiles + t - 1) / t};
}

struct Shape {
  int gh;      // query heads per workgroup
  int nw;      // waves per workgroup (1, 2, 4 or 8; 5 for the e4m3 wave-split decode at d 128)
  SplitShape sp;
  bool waves_split = false;   // decode: the waves take the split's tiles in turn
};

// The largest GH dividing the GQA group whose GH x max_q rows fit the waves
// a workgroup may have (8; 4 at d = 256, whose accumulators need a whole
// SIMD's registers per wave).  Memory-bound decode loses nothing to the
// padding rows of a wave.
// waves_ok: the wave-split decode kernel may run (pages hold whole gather
// instructions).
Shape shape_for(int batch, int hq, int hkv, int d, int max_q, int max_tiles, bool positional = false,
                bool waves_ok = false, bool kv8 = false) {
  const int group = hq / hkv;
  const int max_rows = 32 * (d == 256 ? 4 : 8);
  int gh = 1;
  for (int c = group; c >= 1; --c)
    if (group % c == 0 && c * max_q <= max_rows) {
      gh = c;
      break;
    }
  const int need = (gh * max_q + 31) / 32;
  // At d = 256 a workgroup keeps 4 waves even for a few rows: each wave's
  // share of the tile gather (addresses in registers) then stays small.
  int nw = d == 256 ? 4 : 1;
  // Rows that fit one wave under a positional mask (decode): four waves.
  // Where pages hold whole gather instructions (waves_ok) they take the
  // split's tiles in turn (the wave-split kernel); otherwise they share each
  // tile's gather (the extra waves' rows are padding), which keeps more of it
  // in flight per CU (measured -6% on 16 x 4k-16k decode).
  const bool four = positional && d <= 128 && need <= 1;
  if (four) nw = 4;
  while (nw < need) nw <<= 1;
  const bool ws = four && waves_ok;
  // the wave-split kernel over e4m3 caches at d 128: five waves' 32 KB fill
  // the CU's 160 KB (measured -5%; over bf16 caches a fifth wave costs +9%)
  if (ws && kv8 && d == 128) nw = kDecodeWaves128;
  // One round of workgroups: eight-wave ones and the wave-split decode ones
  // at d 128 (128 KB of LDS, 160 KB over e4m3 caches) run one per CU.
  const int target = ws ? (d == 128 ? 256 : 512) : (nw >= 8 ? 256 : kTargetWorkgroups);
  Shape sh{gh, nw, split_shape(batch * (hq / gh), max_tiles, target)};
  sh.waves_split = ws;
  return sh;
}

// Tiles a sequence's walk can need: all of them, or for a sliding window the
// ones from the first visible key of row 0.
int max_walk_tiles(int mode, int window, int max_q, int max_kv) {
  const int all = (max_kv + 63) / 64;
  if (mode != kWindow) return all;
  const int span = (window + max_q - 1 + 63) / 64 + 1;
  return span < all ? span : all;
}

struct VerifyParams {
  const void *q, *k, *v;
  const int32_t *page_table;
  const int32_t *cu_seqlens_q, *kv_lens;
  const void *mask;
  int64_t mask_numel;
  const int32_t *prefix_len;
  void *out;
  float *lse;
  float *ws_o;    // [batch][max_splits][hq][qs][d]
  float *ws_lse;  // [batch][max_splits][hq][qs]
  int64_t s_page, s_slot, s_head;
  int32_t max_pages, page_shift;
  int32_t hq, group, gh, qs;
  int32_t mode, window;
  int32_t tiles_per_split, max_splits, max_kv;
  float scale, scale_log2;   // scale_log2 includes the K descale factor (fp8 caches)
  float v_scale;             // V descale factor (fp8 caches; 1 otherwise)
  // balanced tree verify (verify_pipe_kernel): head blocks per sequence,
  // workgroups, sequences
  int32_t nhb, grid, batch;
  // dense rows that verify_pipe_kernel turns into `mask` (the packed words)
  // itself, piece by piece; NULL when the mask is packed
  const void *dense;
  int64_t dense_numel;
};

__device__ __forceinline__ int64_t mask_offset(const VerifyParams &p, int b) {
  int64_t off = 0;
  if (p.mode != kDense && p.mode != kPacked) return 0;
  for (int i = 0; i < b; ++i) {
    const int64_t ql = p.cu_seqlens_q[i + 1] - p.cu_seqlens_q[i], kv = p.kv_lens[i];
    off += p.mode == kPacked ? ql * ((kv + 63) / 64) : ql * kv;
  }
  return off;
}

// A sequence's query count, clamped to the max_q row slots per head that the
// launch (and the workspace) provide: lengths live on the device, so the host
// cannot refuse a longer sequence; its rows past max_q are not computed.
__device__ __forceinline__ int seq_q_len(const VerifyParams &p, int b, int q0) {
  return max(0, min(p.cu_seqlens_q[b + 1] - q0, p.qs));
}

// Splits of a walk of ntiles k-tiles, never more than the launch has (a
// window walk is bounded by the host's max_walk_tiles only while q_len <=
// max_q, which seq_q_len ensures).
__device__ __forceinline__ int num_splits(const VerifyParams &p, int ntiles) {
  return min((ntiles + p.tiles_per_split - 1) / p.tiles_per_split, p.max_splits);
}

// First k-tile any row of the sequence can see.
__device__ __forceinline__ int first_tile(const VerifyParams &p, int q_len, int kv) {
  if (p.mode != kWindow) return 0;
  const int lo = kv - q_len + 1 - p.window;
  return lo > 0 ? lo / 64 : 0;
}

// Bits of keys [lo, hi] inside k-tile kt.
__device__ __forceinline__ uint64_t interval_word(int lo, int hi, int kt) {
  const int a = max(lo - 64 * kt, 0), b = min(hi - 64 * kt, 63);
  if (a > b) return 0ull;
  return (~0ull >> (63 - b)) & (~0ull << a);
}

// The word of query t of the sequence for k-tile kt (closed forms and packed
// masks: this lane's own row).
__device__ __forceinline__ uint64_t row_word(const VerifyParams &p, int64_t moff, int plen, int t, bool ok,
                                             int q_len, int kv, int kt) {
  if (!ok) return 0ull;
  const int pos = t + kv - q_len;
  switch (p.mode) {
    case kPacked: {
      const int64_t idx = moff + (int64_t)t * ((kv + 63) / 64) + kt;
      return idx < p.mask_numel ? ((const uint64_t *)p.mask)[idx] : 0ull;
    }
    case kCausal: return interval_word(0, pos, kt);
    case kWindow: return interval_word(pos - p.window + 1, pos, kt);
    default: return interval_word(0, max(pos, plen - 1), kt);  // kPrefix
  }
}

// Four dwords that need only dword alignment (a 16-byte load from any
// dword address).
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));

// Bits (LSB = lowest address) of the nonzero bytes of a dword: per byte the
// high bit is set iff the byte is nonzero (SWAR), then one multiply moves the
// four high bits to bits 21..24 (distinct partial products, no carries).
__device__ __forceinline__ uint32_t nonzero_bytes4(uint32_t x) {
  const uint32_t t = ((((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x) >> 7) & 0x01010101u;
  return ((t * 0x00204081u) >> 21) & 0xFu;
}

// The packed word of dense mask bytes [base, base + nb), 1 <= nb <= 64 (byte
// j -> bit j); bytes at or past numel read as 0.  Rows start at any byte
// (their stride is kv_len bytes): the 64 bytes are read as 17 dword-aligned
// dwords and shifted into place with v_alignbyte, so every load is aligned
// whatever the row's start.  A row's last word reads the same 64 bytes
// (those past the row belong to the next row, or the next sequence) and
// masks off the bits past nb; only at the end of the buffer, where the 17th
// dword would lie past it, are bytes read one by one.
__device__ __forceinline__ uint64_t dense_word(const uint8_t *m8, int64_t numel, int64_t base, int nb) {
  uint64_t bits = 0;
  const int64_t a4 = base & ~(int64_t)3;
  if (a4 + 68 <= numel) {
    const uint32_t sh = (uint32_t)(base & 3);
    const u32x4a4 *w4 = (const u32x4a4 *)(m8 + a4);
    uint32_t dw[17];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4a4 v = w4[q];
#pragma unroll
      for (int e = 0; e < 4; ++e) dw[4 * q + e] = v[e];
    }
    dw[16] = ((const uint32_t *)(m8 + a4))[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      bits |= (uint64_t)nonzero_bytes4(__builtin_amdgcn_alignbyte(dw[i + 1], dw[i], sh)) << (4 * i);
    if (nb < 64) bits &= (1ull << nb) - 1ull;
  } else {
    for (int j = 0; j < nb; ++j)
      if (base + j < numel && m8[base + j] != 0) bits |= 1ull << j;
  }
  return bits;
}

// The lane's row word for k-tile kt.  A dense mask is read by lane pairs:
// lanes 2i and 2i + 1 load the two 32-byte halves of wave row i's 64 bytes
// (two 16-byte loads each, one coalesced 2 KB read per wave), turn them into
// 32 bits, and the lanes holding row i (i and i + 32) take both halves with
// two shuffles (rows of the wave: r0 .. r0+31).
__device__ __forceinline__ uint64_t fetch_word(const VerifyParams &p, int64_t moff, int plen, int t, bool ok,
                                               int r0, int q_len, int kv, int kt, int lane) {
  if (p.mode != kDense) return row_word(p, moff, plen, t, ok, q_len, kv, kt);
  const int i = lane >> 1, half = lane & 1;
  const int r = r0 + i;
  const int ti = r % p.qs;
  uint32_t bits = 0;
  if (r / p.qs < p.gh && ti < q_len) {
    const uint8_t *m8 = (const uint8_t *)p.mask;
    const int64_t base = moff + (int64_t)ti * kv + 64 * kt + 32 * half;
    const int nb = min(32, kv - 64 * kt - 32 * half);   // this half's bytes inside the row
    if (nb <= 0) {
      // the half lies past the row's last key
    } else if (base + 32 <= p.mask_numel) {
      // a short half (the row's last) reads the same 32 bytes and masks off
      // those past the row
      u32x4 v0, v1;
      __builtin_memcpy(&v0, m8 + base, 16);
      __builtin_memcpy(&v1, m8 + base + 16, 16);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        bits |= nonzero_bytes4(v0[c]) << (4 * c);
        bits |= nonzero_bytes4(v1[c]) << (16 + 4 * c);
      }
      if (nb < 32) bits &= (1u << nb) - 1u;
    } else {
      // the end of the mask buffer only: byte by byte
      for (int j = 0; j < nb; ++j)
        if (base + j < p.mask_numel && m8[base + j] != 0) bits |= 1u << j;
    }
  }
  const int src = 2 * (lane & 31);
  const uint32_t lo = __shfl(bits, src, 64), hi_bits = __shfl(bits, src + 1, 64);
  return ((uint64_t)hi_bits << 32) | lo;
}

// UP: pages hold at least the key rows of one gather instruction, so page
// ids are scalar loads (uniform per instruction) instead of one vector load
// per lane and instruction.
// KV8: the caches hold e4m3 bytes (K = k_descale * decode(K8), likewise V).
// Each tile's bytes are gathered into an fp8 stage (two, one tile ahead),
// widened exactly to bf16 into the swizzled bf16 stage by all threads, and
// from there the bf16 products run unchanged; the descale factors fold into
// the softmax constant and the epilogue.
template <int D, int NW, typename OutT, bool UP, bool KV8 = false>
__global__ __launch_bounds__(NW * 64, 1) void verify_kernel(VerifyParams p) {
  extern __shared__ __align__(16) uint16_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int split = blockIdx.x, b = blockIdx.z;
  const int q0 = p.cu_seqlens_q[b], q_len = seq_q_len(p, b, q0);
  const int kv = min(p.kv_lens[b], p.max_kv);  // the page table covers max_kv keys
  const int nkt = (kv + 63) / 64;
  const int ktf = first_tile(p, q_len, kv);
  const int ntiles = nkt - ktf;
  const int nsplit = num_splits(p, ntiles);
  if (split >= nsplit && !(split == 0 && ntiles <= 0)) return;
  const int kt0 = ktf + split * p.tiles_per_split;
  const int kt1 = min(nkt, kt0 + p.tiles_per_split);
  // Row of this lane: (head hh of the workgroup's GH, query t).
  const int r0 = wave * 32;
  const int r = r0 + l32;
  const int hh = min(r / p.qs, p.gh - 1);
  const int t = r % p.qs;
  const bool row_ok = r / p.qs < p.gh && t < q_len;
  const int h = blockIdx.y * p.gh + hh;
  const int g = (blockIdx.y * p.gh) / p.group;
  const int64_t tok = (int64_t)q0 + t;
  const int64_t moff = mask_offset(p, b);
  const int plen = p.mode == kPrefix ? p.prefix_len[b] : 0;

  bf16x8 qf[D / 16];
  load_q<D>(qf, (const uint16_t *)p.q + (tok * p.hq + h) * D, row_ok, hi);
  const uint16_t *kbase = (const uint16_t *)p.k + (int64_t)g * p.s_head;
  const uint16_t *vbase = (const uint16_t *)p.v + (int64_t)g * p.s_head;
  const int32_t *pt = p.page_table + (int64_t)b * p.max_pages;
  using KV = KvDma<D, NW>;
  const LaneOffsets<D> lo(lane);
  const uint32_t lds0 = lds_addr(lds);
  typename KV::Pages pg_nxt;
  auto pages = [&](int kt) {
    if constexpr (UP)
      return KV::pages_uniform(pt, p.page_shift, kt, kv, wave);
    else
      return KV::pages(pt, p.page_shift, kt, kv, wave, lane);
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n) oacc[n] = f32x16{};
  float m_ref = neg_inf();
  float lsum = 0.f;   // this lane's half of its row sum
  const float c = p.scale_log2;

  if constexpr (KV8) {
    constexpr int CH8 = D / 16;        // 16-byte chunks of an fp8 row
    constexpr int T8 = D / 16;         // 1 KB gather instructions per matrix and tile
    constexpr int RPI8 = 1024 / D;     // key rows per gather instruction
    constexpr uint32_t F8 = 2u * 64 * D;   // bytes of one fp8 stage (K, then V)
    constexpr uint32_t BF = 2u * F8;       // byte offset of the bf16 stage
    uint8_t *l8 = (uint8_t *)lds;
    const int pmask = (1 << p.page_shift) - 1;
    const __attribute__((address_space(4))) int32_t *cpt = (const __attribute__((address_space(4))) int32_t *)pt;
    const uint8_t *k8 = (const uint8_t *)p.k + (int64_t)g * p.s_head;
    const uint8_t *v8 = (const uint8_t *)p.v + (int64_t)g * p.s_head;
    // Instruction t of a matrix fills LDS chunks [64 t, 64 t + 64) of the
    // plain row-major [64][D] byte tile; its RPI8 rows lie in one page (the
    // host requires pages of at least RPI8 keys), keys past kv_len repeat the
    // last key (same page as the group's first row, or the last key's page).
    auto gather8 = [&](int kt, int st) {
      for (int t8 = wave; t8 < T8; t8 += NW) {
        const int key0 = min(kt * 64 + RPI8 * t8, kv - 1);
        const int32_t pg = cpt[key0 >> p.page_shift];
        const int r = RPI8 * t8 + lane / CH8, pc = lane % CH8;
        const int key = min(kt * 64 + r, kv - 1);
        const uint32_t off = (uint32_t)((key & pmask) * (int)p.s_slot) + 16 * pc;
        const uint64_t pb = (uint64_t)(uint32_t)pg * (uint64_t)p.s_page;
        dma::lds_load16_s((dma::gptr_t)(k8 + pb), off, lds0 + (uint32_t)st * F8 + 1024 * t8);
        dma::lds_load16_s((dma::gptr_t)(v8 + pb), off, lds0 + (uint32_t)st * F8 + 64 * D + 1024 * t8);
      }
    };
    // fp8 stage st -> bf16 stage: 16 bytes in, two swizzled 8-element chunks out
    auto widen = [&](int st) {
      constexpr int NCH = 2 * 64 * CH8;
      for (int q = tid; q < NCH; q += NW * 64) {
        const int m = q / (64 * CH8), qq = q - m * (64 * CH8);
        const int r = qq / CH8, c16 = qq - r * CH8;
        const u32x4 x = *(const u32x4 *)(l8 + (uint32_t)st * F8 + m * 64 * D + 16 * qq);
        u32x4 y[2];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
          y[w >> 1][2 * (w & 1)] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[w], 1.0f, false));
          y[w >> 1][2 * (w & 1) + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[w], 1.0f, true));
        }
        const int f = m == 0 ? Stage<D>::fk(r) : Stage<D>::fv(r);
        uint16_t *dst = (uint16_t *)(l8 + BF) + m * Stage<D>::V_OFF + r * D;
        *(u32x4 *)(dst + 8 * ((2 * c16) ^ f)) = y[0];
        *(u32x4 *)(dst + 8 * ((2 * c16 + 1) ^ f)) = y[1];
      }
    };
    uint64_t word_nxt = 0;
    if (kt0 < kt1) {
      gather8(kt0, 0);
      word_nxt = fetch_word(p, moff, plen, t, row_ok, r0, q_len, kv, kt0, lane);
    }
    for (int kt = kt0; kt < kt1; ++kt) {
      const int cur = (kt - kt0) & 1;
      wait_vmem();
      __syncthreads();   // fp8 tile kt landed; every wave is done with the bf16 stage
      const uint64_t wcur = word_nxt;
      if (kt + 1 < kt1) {
        // the mask word first (a dense mask's ballots wait for its loads)
        word_nxt = fetch_word(p, moff, plen, t, row_ok, r0, q_len, kv, kt + 1, lane);
        gather8(kt + 1, cur ^ 1);
      }
      widen(cur);
      __syncthreads();
      const uint16_t *stage = (const uint16_t *)(l8 + BF);
      f32x16 sacc[2];
      qk_tile<D>(stage, lo, qf, sacc);
      const int kin = kv - 64 * kt;
      const uint64_t inb = low_bits(kin);
      const uint64_t w = wcur & inb;
      if (kin < 64 || __ballot(row_ok && w != inb) != 0ull) apply_word(sacc, w, hi);
      float alpha;
      if (softmax_tile(sacc, m_ref, c, alpha)) {
#pragma unroll
        for (int n = 0; n < D / 32; ++n) oacc[n] *= alpha;
        lsum *= alpha;
      }
      pv_tile<D>(stage, lo, sacc, oacc, lsum);
    }
  } else {
  uint64_t word_nxt = 0;
  if (kt0 < kt1) {
    const typename KV::Pages pg0 = pages(kt0);
    if constexpr (UP)
      KV::issue(kbase, vbase, pg0, p.page_shift, p.s_page, p.s_slot, kt0, kv, lds0, wave, lane);
    else
      KV::issue_lanes(kbase, vbase, pg0, p.page_shift, p.s_page, p.s_slot, kt0, kv, lds, wave, lane);
    word_nxt = fetch_word(p, moff, plen, t, row_ok, r0, q_len, kv, kt0, lane);
    if (kt0 + 1 < kt1) pg_nxt = pages(kt0 + 1);
    wait_vmem();
    __syncthreads();
  }
  for (int kt = kt0; kt < kt1; ++kt) {
    const int cur = (kt - kt0) & 1;
    const uint64_t wcur = word_nxt;
    if (kt + 1 < kt1) {
      // The mask word first: a dense mask's ballots wait for its loads, and
      // that wait would otherwise include the gather.
      word_nxt = fetch_word(p, moff, plen, t, row_ok, r0, q_len, kv, kt + 1, lane);
      if constexpr (UP)
        KV::issue(kbase, vbase, pg_nxt, p.page_shift, p.s_page, p.s_slot, kt + 1, kv,
                  lds0 + (uint32_t)((cur ^ 1) * Stage<D>::BYTES), wave, lane);
      else
        KV::issue_lanes(kbase, vbase, pg_nxt, p.page_shift, p.s_page, p.s_slot, kt + 1, kv,
                        lds + (cur ^ 1) * Stage<D>::ELEMS, wave, lane);
      if (kt + 2 < kt1) pg_nxt = pages(kt + 2);
    }
    const uint16_t *stage = lds + cur * Stage<D>::ELEMS;
    f32x16 sacc[2];
    qk_tile<D>(stage, lo, qf, sacc);
    const int kin = kv - 64 * kt;
    const uint64_t inb = low_bits(kin);
    const uint64_t w = wcur & inb;
    // Per-wave class: skip the bit tests when every valid row sees the whole
    // tile (keys past kv_len are always masked).
    if (kin < 64 || __ballot(row_ok && w != inb) != 0ull) apply_word(sacc, w, hi);
    float alpha;
    if (softmax_tile(sacc, m_ref, c, alpha)) {
#pragma unroll
      for (int n = 0; n < D / 32; ++n) oacc[n] *= alpha;
      lsum *= alpha;
    }
    pv_tile<D>(stage, lo, sacc, oacc, lsum);
    wait_vmem();
    __syncthreads();
  }
  }

  const float lt = sum_halves(lsum);
  const float inv = lt > 0.f ? p.v_scale / lt : 0.f;
  const float lse = lt > 0.f ? (m_ref + __log2f(lt)) * kLn2 : neg_inf();
  if (!row_ok) return;
  if (nsplit <= 1) {
    store_row<D, OutT>((OutT *)p.out + (tok * p.hq + h) * D, oacc, inv, hi);
    if (p.lse && hi == 0) p.lse[tok * p.hq + h] = lse;
  } else {
    const int64_t slot = (((int64_t)b * p.max_splits + split) * p.hq + h) * p.qs + t;
    store_row<D, float>(p.ws_o + slot * D, oacc, inv, hi);
    if (hi == 0) p.ws_lse[slot] = lse;
  }
}

// lgkmcnt(0): this wave's LDS reads (and scalar loads) have returned.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// vmcnt(n) for a compile-time n < 64 (the other counters left free).
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Decode with positional masks when the rows fit one wave (a GQA group's
// heads x a few queries): the NW waves of a workgroup take the split's tiles
// in turn (wave w: tiles kt0 + w, kt0 + w + NW, ...), each with its own LDS
// stage, online softmax and accumulators, so every tile is computed once
// (not once per wave); at the end the waves' partial results are merged
// through LDS in wave order.  Each wave gathers a whole tile itself: K and V
// separately, the next tile's K issued once this tile's K^T products are
// done and its V once P V is done, and waits only for its own gathers (no
// workgroup barrier in the loop).
// KV8 (e4m3 caches): each wave gathers its tile's bytes into its own fp8
// stage and widens them exactly to bf16 into its own one-matrix buffer, K
// before the K^T products and V after them (the buffer holds one at a
// time); the next tile's K bytes are gathered once K is widened, its V bytes
// once V is.
template <int D, int NW, typename OutT, bool KV8 = false>
__global__ __launch_bounds__(NW * 64, 1) void decode_waves_kernel(VerifyParams p) {
  extern __shared__ __align__(16) uint16_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int split = blockIdx.x, b = blockIdx.z;
  const int q0 = p.cu_seqlens_q[b], q_len = seq_q_len(p, b, q0);
  const int kv = min(p.kv_lens[b], p.max_kv);
  const int nkt = (kv + 63) / 64;
  const int ktf = first_tile(p, q_len, kv);
  const int ntiles = nkt - ktf;
  const int nsplit = num_splits(p, ntiles);
  if (split >= nsplit && !(split == 0 && ntiles <= 0)) return;
  const int kt0 = ktf + split * p.tiles_per_split;
  const int kt1 = min(nkt, kt0 + p.tiles_per_split);
  // every wave holds the same rows: (head hh of the group's GH, query t)
  const int r = l32;
  const int hh = min(r / p.qs, p.gh - 1);
  const int t = r % p.qs;
  const bool row_ok = r / p.qs < p.gh && t < q_len;
  const int h = blockIdx.y * p.gh + hh;
  const int g = (blockIdx.y * p.gh) / p.group;
  const int64_t tok = (int64_t)q0 + t;
  const int plen = p.mode == kPrefix ? p.prefix_len[b] : 0;

  bf16x8 qf[D / 16];
  load_q<D>(qf, (const uint16_t *)p.q + (tok * p.hq + h) * D, row_ok, hi);
  // Q has landed before the gathers start: otherwise the compiler's wait for
  // it sits at its first use inside the loop and drains every gather
  wait_vmem();
  const int32_t *pt = p.page_table + (int64_t)b * p.max_pages;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n) oacc[n] = f32x16{};
  float m_ref = neg_inf();
  float lsum = 0.f;
  const float c = p.scale_log2;
  const LaneOffsets<D> lo(lane);
  if constexpr (KV8) {
    constexpr int CH8 = D / 16;          // 16-byte chunks of an fp8 row
    constexpr int T8 = D / 16;           // 1 KB gather instructions per matrix and tile
    constexpr int RPI8 = 1024 / D;       // key rows per gather instruction
    constexpr uint32_t M8 = 64u * D;     // bytes of one fp8 matrix tile
    constexpr uint32_t WB = 4u * M8;     // bytes per wave: fp8 K, fp8 V, bf16 buffer
    uint8_t *l8 = (uint8_t *)lds + (uint32_t)wave * WB;
    uint16_t *buf = (uint16_t *)(l8 + 2 * M8);
    const uint32_t s8 = lds_addr(l8);
    const int pmask = (1 << p.page_shift) - 1;
    const __attribute__((address_space(4))) int32_t *cpt = (const __attribute__((address_space(4))) int32_t *)pt;
    const uint8_t *k8 = (const uint8_t *)p.k + (int64_t)g * p.s_head;
    const uint8_t *v8 = (const uint8_t *)p.v + (int64_t)g * p.s_head;
    // Instruction t fills chunks [64 t, 64 t + 64) of the plain row-major
    // [64][D] byte tile; its RPI8 rows share one page (pages hold at least
    // RPI8 keys), keys past kv repeat the last key.
    auto gather8 = [&](const uint8_t *base, int kt, uint32_t dst) {
#pragma unroll
      for (int t8 = 0; t8 < T8; ++t8) {
        const int key0 = min(kt * 64 + RPI8 * t8, kv - 1);
        const int32_t pg = cpt[key0 >> p.page_shift];
        const int r = RPI8 * t8 + lane / CH8, pc = lane % CH8;
        const int key = min(kt * 64 + r, kv - 1);
        const uint32_t off = (uint32_t)((key & pmask) * (int)p.s_slot) + 16 * pc;
        const uint64_t pb = (uint64_t)(uint32_t)pg * (uint64_t)p.s_page;
        dma::lds_load16_s((dma::gptr_t)(base + pb), off, dst + 1024 * t8);
      }
    };
    // fp8 matrix tile -> the bf16 buffer in that matrix's swizzled layout:
    // 16 bytes in, two 8-element chunks out, per lane and step.
    auto widen = [&](const uint8_t *src, bool is_v) {
#pragma unroll 4
      for (int q = lane; q < 64 * CH8; q += 64) {
        const int r = q / CH8, c16 = q - r * CH8;
        const u32x4 x = *(const u32x4 *)(src + 16 * q);
        u32x4 y[2];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          y[w >> 1][2 * (w & 1)] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[w], 1.0f, false));
          y[w >> 1][2 * (w & 1) + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[w], 1.0f, true));
        }
        const int f = is_v ? Stage<D>::fv(r) : Stage<D>::fk(r);
        uint16_t *dst = buf + r * D;
        *(u32x4 *)(dst + 8 * ((2 * c16) ^ f)) = y[0];
        *(u32x4 *)(dst + 8 * ((2 * c16 + 1) ^ f)) = y[1];
      }
      // every lane's chunks are in the buffer before any lane reads it
      wait_lds();
      __builtin_amdgcn_wave_barrier();
      asm volatile("" ::: "memory");
    };
    int kt = kt0 + wave;
    if (kt < kt1) {
      gather8(k8, kt, s8);
      gather8(v8, kt, s8 + M8);
    }
    for (; kt < kt1; kt += NW) {
      const int nk = kt + NW;
      uint64_t wcur = 0;
      if (row_ok) {
        const int pos = t + kv - q_len;
        wcur = p.mode == kCausal ? interval_word(0, pos, kt)
             : p.mode == kWindow ? interval_word(pos - p.window + 1, pos, kt)
                                 : interval_word(0, max(pos, plen - 1), kt);
      }
      wait_vmem_n<T8>();   // this tile's K bytes (its V bytes may still be in flight)
      widen(l8, false);
      if (nk < kt1) gather8(k8, nk, s8);   // the K bytes were read (wait_lds in widen)
      f32x16 sacc[2];
      qk_tile<D>(buf, lo, qf, sacc);
      const int kin = kv - 64 * kt;
      const uint64_t inb = low_bits(kin);
      const uint64_t w = wcur & inb;
      if (kin < 64 || __ballot(row_ok && w != inb) != 0ull) apply_word(sacc, w, hi);
      float alpha;
      if (softmax_tile(sacc, m_ref, c, alpha)) {
#pragma unroll
        for (int n = 0; n < D / 32; ++n) oacc[n] *= alpha;
        lsum *= alpha;
      }
      // the K^T products' buffer reads are done before V overwrites it
      wait_lds();
      asm volatile("" ::: "memory");
      if (nk < kt1)
        wait_vmem_n<T8>();   // this tile's V bytes (the next K bytes may be in flight)
      else
        wait_vmem();
      widen(l8 + M8, true);
      if (nk < kt1) gather8(v8, nk, s8 + M8);
      pv_tile<D>(buf - Stage<D>::V_OFF, lo, sacc, oacc, lsum);
      // the P V buffer reads are done before the next K is widened into it
      wait_lds();
      asm volatile("" ::: "memory");
    }
  } else {
  const uint16_t *kbase = (const uint16_t *)p.k + (int64_t)g * p.s_head;
  const uint16_t *vbase = (const uint16_t *)p.v + (int64_t)g * p.s_head;
  using KV = KvDma<D, 1>;
  constexpr int G = KV::IPW;   // gather instructions per matrix and tile (one wave)
  uint16_t *stage = lds + wave * Stage<D>::ELEMS;
  const uint32_t sk = lds_addr(stage), sv = sk + 2u * Stage<D>::V_OFF;


  int kt = kt0 + wave;
  typename KV::Pages pg;
  if (kt < kt1) {
    pg = KV::pages_uniform(pt, p.page_shift, kt, kv, 0);
    issue_mat<D, 1, false>(kbase, pg, p.page_shift, p.s_page, p.s_slot, kt, kv, sk, 0, lane);
    issue_mat<D, 1, true>(vbase, pg, p.page_shift, p.s_page, p.s_slot, kt, kv, sv, 0, lane);
  }
  for (; kt < kt1; kt += NW) {
    const int nk = kt + NW;
    uint64_t wcur = 0;
    if (row_ok) {
      const int pos = t + kv - q_len;
      wcur = p.mode == kCausal ? interval_word(0, pos, kt)
           : p.mode == kWindow ? interval_word(pos - p.window + 1, pos, kt)
                               : interval_word(0, max(pos, plen - 1), kt);
    }
    wait_vmem_n<G>();   // this tile's K (its V may still be in flight)
    f32x16 sacc[2];
    qk_tile<D>(stage, lo, qf, sacc);
    typename KV::Pages pgn;
    if (nk < kt1) {
      pgn = KV::pages_uniform(pt, p.page_shift, nk, kv, 0);
      wait_lds();   // this wave's K reads have returned before the K half is rewritten
      issue_mat<D, 1, false>(kbase, pgn, p.page_shift, p.s_page, p.s_slot, nk, kv, sk, 0, lane);
    }
    const int kin = kv - 64 * kt;
    const uint64_t inb = low_bits(kin);
    const uint64_t w = wcur & inb;
    if (kin < 64 || __ballot(row_ok && w != inb) != 0ull) apply_word(sacc, w, hi);
    float alpha;
    if (softmax_tile(sacc, m_ref, c, alpha)) {
#pragma unroll
      for (int n = 0; n < D / 32; ++n) oacc[n] *= alpha;
      lsum *= alpha;
    }
    // this tile's V (the next tile's K may still be in flight)
    if (nk < kt1)
      wait_vmem_n<G>();
    else
      wait_vmem();
    pv_tile<D>(stage, lo, sacc, oacc, lsum);
    if (nk < kt1) {
      wait_lds();   // likewise for the V reads
      issue_mat<D, 1, true>(vbase, pgn, p.page_shift, p.s_page, p.s_slot, nk, kv, sv, 0, lane);
    }
  }
  }
  wait_vmem();

  // Merge the waves' (m_ref, lsum, O) through LDS (the stages are free now):
  // wave w stores its lane-private values, wave 0 combines them in wave order.
  __syncthreads();
  float *mf = (float *)lds;
  constexpr int PER = D / 32 * 16 + 2;   // floats per lane: O, then m_ref and lsum
  {
    float *mine = mf + ((size_t)wave * 64 + lane) * PER;
#pragma unroll
    for (int n = 0; n < D / 32; ++n)
#pragma unroll
      for (int e = 0; e < 16; ++e) mine[16 * n + e] = oacc[n][e];
    mine[PER - 2] = m_ref;
    mine[PER - 1] = lsum;
  }
  __syncthreads();
  if (wave != 0) return;
  float mx = neg_inf();
#pragma unroll
  for (int w = 0; w < NW; ++w) mx = fmaxf(mx, mf[((size_t)w * 64 + lane) * PER + PER - 2]);
  float lt_lane = 0.f;
#pragma unroll
  for (int n = 0; n < D / 32; ++n) oacc[n] = f32x16{};
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float *src = mf + ((size_t)w * 64 + lane) * PER;
    const float mw = src[PER - 2];
    const float sc = mw == neg_inf() ? 0.f : fast_exp2(mw - mx);
    lt_lane += sc * src[PER - 1];
#pragma unroll
    for (int n = 0; n < D / 32; ++n)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[n][e] += sc * src[16 * n + e];
  }
  m_ref = mx;
  const float lt = sum_halves(lt_lane);
  const float inv = lt > 0.f ? p.v_scale / lt : 0.f;
  const float lse = lt > 0.f ? (m_ref + __log2f(lt)) * kLn2 : neg_inf();
  if (!row_ok) return;
  if (nsplit <= 1) {
    store_row<D, OutT>((OutT *)p.out + (tok * p.hq + h) * D, oacc, inv, hi);
    if (p.lse && hi == 0) p.lse[tok * p.hq + h] = lse;
  } else {
    const int64_t slot = (((int64_t)b * p.max_splits + split) * p.hq + h) * p.qs + t;
    store_row<D, float>(p.ws_o + slot * D, oacc, inv, hi);
    if (hi == 0) p.ws_lse[slot] = lse;
  }
}

// Merges the split partials of one (sequence, query head) in split order:
// O = sum_s exp(LSE_s - M) O_s / sum_s exp(LSE_s - M), LSE = M + ln(sum).
template <int D, typename OutT>
__global__ __launch_bounds__(256) void verify_combine(VerifyParams p) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int q0 = p.cu_seqlens_q[b], q_len = seq_q_len(p, b, q0);
  const int kv = min(p.kv_lens[b], p.max_kv);
  const int ntiles = (kv + 63) / 64 - first_tile(p, q_len, kv);
  const int nsplit = num_splits(p, ntiles);
  if (nsplit <= 1) return;
  const int64_t sbase = (int64_t)b * p.max_splits;
  // one (row, 4 columns) item per thread; blockIdx.z picks the chunk of items
  for (int idx = blockIdx.z * blockDim.x + threadIdx.x; idx < q_len * (D / 4); idx += blockDim.x * gridDim.z) {
    const int t = idx / (D / 4), c4 = idx % (D / 4);
    float mx = neg_inf();
    for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, p.ws_lse[((sbase + s) * p.hq + h) * p.qs + t]);
    float wsum = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (mx != neg_inf()) {
      for (int s = 0; s < nsplit; ++s) {
        const int64_t slot = ((sbase + s) * p.hq + h) * p.qs + t;
        const float wgt = __expf(p.ws_lse[slot] - mx);
        const f32x4 o = *(const f32x4 *)(p.ws_o + slot * D + 4 * c4);
        acc += wgt * o;
        wsum += wgt;
      }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    const int64_t tok = (int64_t)q0 + t;
    store4<OutT>((OutT *)p.out + (tok * p.hq + h) * D + 4 * c4, acc[0] * inv, acc[1] * inv, acc[2] * inv,
                 acc[3] * inv);
    if (p.lse && c4 == 0) p.lse[tok * p.hq + h] = wsum > 0.f ? mx + __logf(wsum) : neg_inf();
  }
}


// ---------------------------------------------------------------------------
// Tree verify over a balanced partition of the tiles (custom masks, d <= 128)
// ---------------------------------------------------------------------------
// A unit is (sequence b, head block hb): GH query heads of one GQA group and
// their q_len queries, at most 256 row slots (eight waves of 32), head-major,
// so that each K/V tile gathered serves the whole group.  Its k-tiles are
// 0 .. n_b - 1, n_b = ceil(kv_len / 64).  A unit is cut into k_b =
// ceil(n_b / T) pieces of near-equal length, one workgroup each, where T is
// the smallest tile count for which all pieces fit the grid (sum over units
// of k_b <= G): every workgroup then has at most T tiles and a single piece,
// however unevenly the contexts are spread.  T and the piece of each
// workgroup are computed on the device from the device-resident lengths (a
// binary search over T and prefix sums across a wave).  A unit in one piece
// is written directly; the pieces of a cut unit leave partial (O, LSE) rows
// in their workgroups' slots, which verify_pipe_combine merges in piece
// order (deterministic, no atomics).
//
// Inside a piece the loop is software-pipelined: step j issues the S^T
// products of tile j + 1 beside the masking and softmax of tile j, then
// O^T += V^T P^T of tile j.  Four LDS stages hold tiles j .. j + 3: step j
// gathers tile j + 3 (K, V and the rows' packed mask words, all by LDS DMA)
// into the stage tile j - 1 has left, and ends waiting only for tile j + 2,
// so a tile's gathers have two steps to land.  No compiler-visible load is
// in flight in the loop, so every wait is an explicit vmcnt.
constexpr int kPipeGrid = 256;   // one 8-wave workgroup per CU
constexpr int kPipeRows = 256;   // row slots of a unit
constexpr int kPipeWaves = 8;
constexpr int kPipeStages = 4;

template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const T u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint64_t u = (uint64_t)v;
  return (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(u >> 32)) << 32) |
                   (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)u));
}

// The piece of workgroup `wg`: unit (b, hb), its tiles [kt0, kt1) of n, its
// index k among the unit's npieces pieces, and the sequence's first mask
// word.  b < 0: the workgroup has no piece.
struct Piece {
  int b, hb, kt0, kt1, n, k, npieces;
  int64_t moff;
  int q0, q_len, kv_len;   // the sequence's first query row, rows (seq_q_len), keys
  int64_t doff;            // the sequence's first byte in the dense layout
  int plen;                // the sequence's prefix (prefix masks; 0 otherwise)
};

// Every lane returns the same (scalar) values.  Batches of up to 64
// sequences keep each sequence's lengths in its lane for the whole search,
// loaded at once (one round trip); larger ones reread them per chunk.
__device__ Piece locate_piece(const VerifyParams &p, int wg, int lane) {
  const bool one_chunk = p.batch <= 64;
  // lane's sequence from its lengths (and its prefix under a prefix mask),
  // all loaded before any is used: its tiles (every unit of the sequence has
  // them; a sequence with queries but no keys keeps one tile so that its rows
  // are written, O = 0 and LSE = -inf), its packed mask words and its dense
  // mask bytes (true lengths: the caller's layouts)
  struct Lens {
    int n, q0, ql, kv;
    int64_t words, bytes;
    int pl;
  };
  auto lens = [&](int b) -> Lens {
    if (b >= p.batch) return Lens{0, 0, 0, 0, 0, 0, 0};
    const int q0 = p.cu_seqlens_q[b], q1 = p.cu_seqlens_q[b + 1], kv_true = p.kv_lens[b];
    const int pl = p.mode == kPrefix ? p.prefix_len[b] : 0;
    const int ql = max(0, min(q1 - q0, p.qs));
    const int kv = min(kv_true, p.max_kv);
    return Lens{ql <= 0 ? 0 : (kv > 0 ? (kv + 63) / 64 : 1), q0, ql, kv_true,
                (int64_t)(q1 - q0) * ((kv_true + 63) / 64), (int64_t)(q1 - q0) * kv_true, pl};
  };
  const Lens mine = one_chunk ? lens(lane) : Lens{0, 0, 0, 0, 0, 0, 0};
  auto tiles_at = [&](int b) { return one_chunk ? (b < p.batch ? mine.n : 0) : lens(b).n; };
  // Smallest T in [1, max n_b] with need(T) = sum_b nhb * ceil(n_b / T) <= G
  // (T = max n_b always fits: the host sizes G to at least the number of
  // units).  With S = sum_b nhb * n_b and U units holding tiles, need(T) >=
  // S / T exceeds G below ceil(S / G), and need(T) <= S / T + U is at most G
  // from ceil(S / (G - U)) on, so the search starts in that bracket.
  int maxn = 0, tot = 0, used = 0;
  for (int c0 = 0; c0 < p.batch; c0 += 64) {
    const int n = tiles_at(c0 + lane);
    maxn = max(maxn, n);
    tot += n;
    used += n > 0;
  }
  maxn = wave_max(maxn);
  tot = wave_sum(tot) * p.nhb;
  used = wave_sum(used) * p.nhb;
  int hi_t = max(maxn, 1);
  if (p.grid > used) hi_t = min(hi_t, max(1, (tot + (p.grid - used) - 1) / (p.grid - used)));
  int lo_t = max(1, min(hi_t, (tot + p.grid - 1) / p.grid));
  while (lo_t < hi_t) {
    const int mid = (lo_t + hi_t) >> 1;
    int need = 0;
    for (int c0 = 0; c0 < p.batch; c0 += 64) {
      const int n = tiles_at(c0 + lane);
      need += wave_sum(p.nhb * (int)(((unsigned)n + (unsigned)mid - 1u) / (unsigned)mid));
    }
    if (need <= p.grid) hi_t = mid;
    else lo_t = mid + 1;
  }
  const int T = __builtin_amdgcn_readfirstlane(lo_t);
  // the sequence whose units hold workgroup wg: prefix sums of nhb * k_b
  int base = 0;
  int64_t mbase = 0, dbase = 0;
  Piece r{-1, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  for (int c0 = 0; c0 < p.batch; c0 += 64) {
    const int b = c0 + lane;
    const Lens ln = one_chunk ? (b < p.batch ? mine : Lens{0, 0, 0, 0, 0, 0, 0}) : lens(b);
    const int n = ln.n;
    const int64_t me = ln.words, de = ln.bytes;
    const int wgs = p.nhb * ((n + T - 1) / T);
    const int incl = wave_incl_scan(wgs, lane);
    const int64_t mincl = wave_incl_scan(me, lane);
    const int64_t dincl = wave_incl_scan(de, lane);
    if (r.b < 0) {
      const uint64_t hit = __ballot(b < p.batch && base + incl > wg);
      if (hit) {
        const int l = __builtin_ctzll(hit);
        r.b = c0 + l;
        const int first = base + __shfl(incl - wgs, l, 64);
        r.n = __shfl(n, l, 64);
        r.npieces = (r.n + T - 1) / T;
        const int off = wg - first;
        r.hb = off / r.npieces;
        r.k = off - r.hb * r.npieces;
        r.moff = mbase + __shfl(mincl - me, l, 64);
        r.doff = dbase + __shfl(dincl - de, l, 64);
        r.q0 = __shfl(ln.q0, l, 64);
        r.q_len = __shfl(ln.ql, l, 64);
        r.kv_len = __shfl(ln.kv, l, 64);
        r.plen = __shfl(ln.pl, l, 64);
      }
    }
    base += __shfl(incl, 63, 64);
    mbase += __shfl(mincl, 63, 64);
    dbase += __shfl(dincl, 63, 64);
  }
  r.b = __builtin_amdgcn_readfirstlane(r.b);
  r.n = __builtin_amdgcn_readfirstlane(r.n);
  r.npieces = __builtin_amdgcn_readfirstlane(r.npieces);
  r.hb = __builtin_amdgcn_readfirstlane(r.hb);
  r.k = __builtin_amdgcn_readfirstlane(r.k);
  r.moff = uniform64(r.moff);
  r.doff = uniform64(r.doff);
  r.q0 = __builtin_amdgcn_readfirstlane(r.q0);
  r.q_len = __builtin_amdgcn_readfirstlane(r.q_len);
  r.kv_len = __builtin_amdgcn_readfirstlane(r.kv_len);
  r.plen = __builtin_amdgcn_readfirstlane(r.plen);
  r.kt0 = r.k * r.n / r.npieces;
  r.kt1 = (r.k + 1) * r.n / r.npieces;
  return r;
}

__device__ __forceinline__ Piece uniform_piece(const Piece &x) {
  Piece r;
  r.b = __builtin_amdgcn_readfirstlane(x.b);
  r.hb = __builtin_amdgcn_readfirstlane(x.hb);
  r.kt0 = __builtin_amdgcn_readfirstlane(x.kt0);
  r.kt1 = __builtin_amdgcn_readfirstlane(x.kt1);
  r.n = __builtin_amdgcn_readfirstlane(x.n);
  r.k = __builtin_amdgcn_readfirstlane(x.k);
  r.npieces = __builtin_amdgcn_readfirstlane(x.npieces);
  r.moff = uniform64(x.moff);
  r.doff = uniform64(x.doff);
  r.q0 = __builtin_amdgcn_readfirstlane(x.q0);
  r.q_len = __builtin_amdgcn_readfirstlane(x.q_len);
  r.kv_len = __builtin_amdgcn_readfirstlane(x.kv_len);
  r.plen = __builtin_amdgcn_readfirstlane(x.plen);
  return r;
}

// What a unit's first piece leaves for the merge: its workgroup (the pieces
// are workgroups slot, slot + 1, ...) and how many pieces the unit has.
struct UnitRec {
  int32_t slot, npieces;
};

// Workgroups are dispatched to the 8 XCDs round-robin.  When the grid is a
// multiple of 8, dispatch slot x runs logical workgroup (x % 8) * (G / 8) +
// x / 8, so consecutive workgroups - the pieces of one unit, which read the
// same query rows - share one XCD's L2.
__device__ __forceinline__ int pipe_logical(int x, int g) {
  return (g & 7) == 0 ? (x & 7) * (g >> 3) + (x >> 3) : x;
}

// Direct global -> LDS load of 4 bytes per lane (LDS address M0 + 4 lane).
__device__ __forceinline__ void lds_load4(const void *src, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}

template <int D>
struct PipeStage {
  static constexpr uint32_t KV = (uint32_t)dma::Stage<D>::BYTES;   // K then V
  static constexpr uint32_t WLO = KV;                               // low dwords of the rows' words
  static constexpr uint32_t WHI = KV + 4 * kPipeRows;               // high dwords
  static constexpr uint32_t BYTES = KV + 8 * kPipeRows;
};

// POS: a mask given by position (causal, or causal after a per-sequence
// prefix): each row's word is computed, not loaded, and a tile moves only K
// and V.
template <int D, typename OutT, bool POS>
__global__ __launch_bounds__(kPipeWaves * 64, 1) void verify_pipe_kernel(VerifyParams p, UnitRec *units) {
  extern __shared__ __align__(16) uint16_t lds[];
  constexpr int NW = kPipeWaves;
  using KV = dma::KvDma<D, NW>;
  using PS = PipeStage<D>;
  constexpr int IPW = KV::IPW;
  constexpr int N_TILE = 2 * IPW + (POS ? 0 : 1);   // vector memory instructions per wave and tile
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int wg = pipe_logical(blockIdx.x, p.grid);

  // One wave finds the piece (the other waves would only share its SIMDs
  // doing the same search) and hands it on through LDS.
  __shared__ Piece piece_lds;
  if (wave == 0) {
    const Piece w0 = locate_piece(p, wg, lane);
    if (lane == 0) piece_lds = w0;
  }
  __syncthreads();
  const Piece pc = uniform_piece(piece_lds);
  if (pc.b < 0) return;
  const int b = pc.b, hb = pc.hb, kt0 = pc.kt0, kt1 = pc.kt1;
  const bool complete = pc.npieces == 1;
  const int kv_true = pc.kv_len;
  const int kv = min(kv_true, p.max_kv);
  // The words' layout: the caller's packed rows (the sequence's first word,
  // ceil(kv_len / 64) per row), or for dense rows, which the workgroup turns
  // into words itself, a fixed one (sequence b at b * max_q * W, W words per
  // row, W = ceil(max_kv / 64)) that the workspace always holds, whatever
  // the device lengths.
  const int64_t wmax = (p.max_kv + 63) / 64;
  const int64_t moff = p.dense ? (int64_t)b * p.qs * wmax : pc.moff;
  const int nwords = p.dense ? (int)wmax : (kv_true + 63) / 64;

  const dma::LaneOffsets<D> lo(lane);
  const uint32_t lds0 = dma::lds_addr(lds);
  const dma::LaneGather<D, NW, dma::SwzK<D>> lgk(wave, lane, p.s_slot);
  const dma::LaneGather<D, NW, dma::SwzV<D>> lgv(wave, lane, p.s_slot);
  const uint32_t page_bytes = (uint32_t)(p.s_page * 2), slot_bytes = (uint32_t)(p.s_slot * 2);
  constexpr int kPageRunShift = __builtin_ctz(KV::RPI * KV::IPW);
  const int r = wave * 32 + l32;            // this lane's row slot
  const int rd = 64 * (wave & 3) + lane;    // the row whose word half this lane's DMA moves
  const uint64_t *mask64 = (const uint64_t *)p.mask;

  const int q0 = pc.q0, q_len = pc.q_len, plen = pc.plen;
  if (tid == 0 && pc.k == 0) units[b * p.nhb + hb] = UnitRec{wg, pc.npieces};
  const int hh = min(r / p.qs, p.gh - 1), t = r % p.qs;
  const bool row_ok = r / p.qs < p.gh && t < q_len;
  const int h = hb * p.gh + hh;
  const int g = (hb * p.gh) / p.group;
  const int64_t tok = (int64_t)q0 + t;
  const int td = rd % p.qs;
  const bool rd_ok = rd / p.qs < p.gh && td < q_len;
  const int64_t wrow = moff + (int64_t)td * nwords;   // word index of k-tile 0 of the DMA row
  const int64_t lrow = moff + (int64_t)t * nwords;     // the same for this lane's own row
  bf16x8 qf[D / 16];
  load_q<D>(qf, (const uint16_t *)p.q + (tok * p.hq + h) * D, row_ok, hi);
  f32x16 oacc[D / 32];
#pragma unroll
  for (int m = 0; m < D / 32; ++m) oacc[m] = f32x16{};
  float m_ref = neg_inf();
  float lsum = 0.f;
  const float c = p.scale_log2;
  if (kv > 0 && kt0 < kt1) {
    const uint16_t *kbase = (const uint16_t *)p.k + (int64_t)g * p.s_head;
    const uint16_t *vbase = (const uint16_t *)p.v + (int64_t)g * p.s_head;
    const int32_t *pt = p.page_table + (int64_t)b * p.max_pages;
    const int nt = kt1 - kt0;
    // Page ids of tile kt0 + j (scalar loads, read a step before their
    // gathers: next to the gathers' inline asm each would be waited for)
    auto pages = [&](int j) { return KV::pages_uniform(pt, p.page_shift, kt0 + j, kv, wave); };
    // Tile kt0 + j into stage j % 4: K and V, then one half of 64 rows'
    // words.
    auto issue_kv = [&](int j, const typename KV::Pages &pg) {
      const int kt = kt0 + j;
      const uint32_t st = lds0 + (uint32_t)(j & 3) * PS::BYTES;
      if (kt * 64 + 64 <= kv) {
        if (p.page_shift >= kPageRunShift) {
          dma::issue_mat_page<D, NW, dma::SwzK<D>>(kbase, pg.id[0], lgk, p.page_shift, page_bytes, slot_bytes, kt,
                                                   st, wave);
          dma::issue_mat_page<D, NW, dma::SwzV<D>>(vbase, pg.id[0], lgv, p.page_shift, page_bytes, slot_bytes, kt,
                                                   st + 2u * dma::Stage<D>::V_OFF, wave);
        } else {
          dma::issue_mat_fast<D, NW, dma::SwzK<D>, false>(kbase, pg, lgk, p.page_shift, page_bytes, slot_bytes, kt,
                                                          kv, st, wave, lane);
          dma::issue_mat_fast<D, NW, dma::SwzV<D>, false>(vbase, pg, lgv, p.page_shift, page_bytes, slot_bytes, kt,
                                                          kv, st + 2u * dma::Stage<D>::V_OFF, wave, lane);
        }
      } else {
        dma::issue_mat_fast<D, NW, dma::SwzK<D>, true>(kbase, pg, lgk, p.page_shift, page_bytes, slot_bytes, kt, kv,
                                                       st, wave, lane);
        dma::issue_mat_fast<D, NW, dma::SwzV<D>, true>(vbase, pg, lgv, p.page_shift, page_bytes, slot_bytes, kt, kv,
                                                       st + 2u * dma::Stage<D>::V_OFF, wave, lane);
      }
    };
    auto issue_words = [&](int j) {
      if constexpr (POS) return;
      const int64_t idx = wrow + kt0 + j;
      const uint64_t *src = rd_ok && idx < p.mask_numel ? mask64 + idx : mask64;
      lds_load4((const uint32_t *)src + (wave >> 2), lds0 + (uint32_t)(j & 3) * PS::BYTES +
                                                         ((wave >> 2) ? PS::WHI : PS::WLO) + 256u * (uint32_t)(wave & 3));
    };
    auto issue = [&](int j, const typename KV::Pages &pg) {
      issue_kv(j, pg);
      issue_words(j);
    };
    // This lane's row word of tile kt0 + j (after the barrier that publishes
    // its stage); rows outside the unit or past mask_numel read 0.
    auto word_of = [&](int j) -> uint64_t {
      if constexpr (POS) {
        // query t is key position kv - q_len + t of its sequence
        const int pos = t + kv - q_len;
        return row_ok ? interval_word(0, p.mode == kPrefix ? max(pos, plen - 1) : pos, kt0 + j) : 0ull;
      }
      const uint32_t *w32 = (const uint32_t *)((const char *)lds + (uint32_t)(j & 3) * PS::BYTES);
      const uint32_t lo_w = w32[PS::WLO / 4 + r], hi_w = w32[PS::WHI / 4 + r];
      const bool ok = row_ok && lrow + kt0 + j < p.mask_numel;
      return ok ? ((uint64_t)hi_w << 32) | lo_w : 0ull;
    };
    f32x16 sa[2], sb[2];
    typename KV::Pages pg0 = pages(0), pg1, pg2, pgn;
    if (nt > 1) pg1 = pages(1);
    if (nt > 2) pg2 = pages(2);
    if (nt > 3) pgn = pages(3);
    if (p.dense) {
      // Dense rows: with K and V of the first three tiles in flight, the
      // workgroup writes the words of the rows and tiles it reads (its own
      // piece's; the pieces of the sequence's other head blocks write the
      // same values).  The stores are waited for and the barrier makes them
      // visible to every wave's word gathers.  Bytes at or past dense_numel
      // read as 0.
      issue_kv(0, pg0);
      if (nt > 1) issue_kv(1, pg1);
      if (nt > 2) issue_kv(2, pg2);
      const uint8_t *d8 = (const uint8_t *)p.dense;
      uint64_t *wout = (uint64_t *)p.mask;
      for (int i = tid; i < q_len * nt; i += kPipeWaves * 64) {
        const int t = i / nt, kt = kt0 + i % nt;
        const int nb = min(64, kv_true - 64 * kt);
        if (nb > 0)
          wout[moff + (int64_t)t * nwords + kt] =
              dense_word(d8, p.dense_numel, pc.doff + (int64_t)t * kv_true + 64 * kt, nb);
      }
      dma::wait_vmem();
      __syncthreads();
      issue_words(0);
      if (nt > 1) issue_words(1);
      if (nt > 2) issue_words(2);
      dma::wait_vmem();   // tiles 0 .. 2 have landed
    } else {
      issue(0, pg0);
      if (nt > 1) issue(1, pg1);
      if (nt > 2) {
        issue(2, pg2);
        wait_vmem_n<N_TILE>();   // tiles 0 and 1 have landed
      } else {
        dma::wait_vmem();
      }
    }
    __syncthreads();
    uint64_t word_cur = word_of(0);
    dma::qk_tile<D, (D > 64 ? 4 : D / 16)>(lds, lo, qf, sa);
    auto step = [&](f32x16 (&scur)[2], f32x16 (&snxt)[2], int j) {
      const int kt = kt0 + j;
      const uint64_t wcur = word_cur;
      if (j + 3 < nt) {
        issue(j + 3, pgn);
        if (j + 4 < nt) pgn = pages(j + 4);
      }
      const int kin = kv - kt * 64;
      const uint64_t inb = low_bits(kin);
      const uint64_t wm = wcur & inb;
      // no masking when every row of the wave sees the whole tile
      if (kin < 64 || __ballot(row_ok && wm != inb) != 0ull) apply_word(scur, wm, hi);
      dma::qk_tile_free<D>((const uint16_t *)((const char *)lds + (uint32_t)((j + 1) & 3) * PS::BYTES), lo, qf,
                           snxt);
      float alpha, ps;
      const bool any = softmax_tile(scur, m_ref, c, alpha);
      bf16x8 pb[4];
      dma::pack_p(scur, pb, ps);
      asm volatile("" : "+v"(pb[0]), "+v"(pb[1]), "+v"(pb[2]), "+v"(pb[3]), "+v"(ps));
      if (any) {
#pragma unroll
        for (int m = 0; m < D / 32; ++m) oacc[m] *= alpha;
        lsum *= alpha;
      }
      lsum += ps;
      dma::pv_tile_packed<D>((const uint16_t *)((const char *)lds + (uint32_t)(j & 3) * PS::BYTES), lo, pb, oacc);
      // tile j + 2 has landed (tile j + 3 may still be in flight)
      if (j + 3 < nt)
        wait_vmem_n<N_TILE>();
      else
        dma::wait_vmem();
      __syncthreads();
      if (j + 1 < nt) word_cur = word_of(j + 1);
    };
    for (int j = 0; j < nt; j += 2) {
      step(sa, sb, j);
      if (j + 1 < nt) step(sb, sa, j + 1);
    }
  }
  const float lt = sum_halves(lsum);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse = lt > 0.f ? (m_ref + __log2f(lt)) * kLn2 : neg_inf();
  if (!row_ok) return;
  if (complete) {
    store_row<D, OutT>((OutT *)p.out + (tok * p.hq + h) * D, oacc, inv, hi);
    if (p.lse && hi == 0) p.lse[tok * p.hq + h] = lse;
  } else {
    // partial O in the output's type: a bf16 output is rounded to bf16 at
    // the end anyway, so its partials need not carry more (and move half the
    // bytes); an fp32 output keeps fp32 partials
    const int64_t row = (int64_t)wg * kPipeRows + r;
    store_row<D, OutT>((OutT *)p.ws_o + row * D, oacc, inv, hi);
    if (hi == 0) p.ws_lse[row] = lse;
  }
}

// Merges the pieces of a cut unit: block (u, c) takes unit u's first piece
// i from its record and 256 (row, 8 columns) items of the unit's 256 x D
// outputs (item = c * 256 + thread, D / 8 items per row) and merges the
// pieces i, i + 1, ... in order:
// O = sum_s exp(LSE_s - M) O_s / sum_s exp(LSE_s - M), LSE = M + ln(sum).
// The records keep entries of earlier launches for units that have no piece
// in this one.  A unit has pieces exactly when its sequence has query rows,
// and then its first piece rewrote the record in this launch, so the
// sequence's row count, loaded beside the record, tells a current entry from
// a stale one.  A unit of one piece wrote its output itself.
// Each pass issues the loads of kMergeBatch pieces before using them.
constexpr int kMergeBatch = 8;

// Four consecutive partial values as fp32 (bf16 widened exactly).
__device__ __forceinline__ f32x4 load4f(const float *src) { return *(const f32x4 *)src; }
__device__ __forceinline__ f32x4 load4f(const uint16_t *src) {
  const u32x2 v = *(const u32x2 *)src;
  return f32x4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xFFFF0000u), __uint_as_float(v[1] << 16),
               __uint_as_float(v[1] & 0xFFFF0000u)};
}

template <int D, typename OutT>
__global__ __launch_bounds__(256) void verify_pipe_combine(VerifyParams p, const UnitRec *units) {
  const int u = blockIdx.x;
  const int b = u / p.nhb, hb = u % p.nhb;
  const UnitRec rec = units[u];
  const int q0 = p.cu_seqlens_q[b], q_len = seq_q_len(p, b, q0);
  const int wg = rec.slot, np = rec.npieces;
  if (q_len == 0 || np < 2 || wg < 0 || wg > p.grid - np) return;
  const int item = blockIdx.y * 256 + threadIdx.x;
  const int r = item / (D / 8), c8 = item % (D / 8);
  const int t = r % p.qs;
  if (r / p.qs >= p.gh || t >= q_len) return;
  const int h = hb * p.gh + r / p.qs;
  float m_run = neg_inf(), l_run = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < np; k0 += kMergeBatch) {
    float lse_k[kMergeBatch];
    f32x4 o_k[kMergeBatch], o2_k[kMergeBatch];
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const bool has = k0 + k < np;
      const int64_t row = (int64_t)(wg + k0 + k) * kPipeRows + r;
      lse_k[k] = has ? p.ws_lse[row] : neg_inf();
      o_k[k] = has ? load4f((const OutT *)p.ws_o + row * D + 8 * c8) : f32x4{0.f, 0.f, 0.f, 0.f};
      o2_k[k] = has ? load4f((const OutT *)p.ws_o + row * D + 8 * c8 + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float mx = m_run;
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) mx = fmaxf(mx, lse_k[k]);
    if (mx == neg_inf()) continue;
    const float sc = __expf(m_run - mx);   // 0 while nothing was merged
    l_run *= sc;
    acc *= sc;
    acc2 *= sc;
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const float wgt = __expf(lse_k[k] - mx);
      l_run += wgt;
      acc += wgt * o_k[k];
      acc2 += wgt * o2_k[k];
    }
    m_run = mx;
  }
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  const int64_t tok = (int64_t)q0 + t;
  store4<OutT>((OutT *)p.out + (tok * p.hq + h) * D + 8 * c8, acc[0] * inv, acc[1] * inv, acc[2] * inv,
               acc[3] * inv);
  store4<OutT>((OutT *)p.out + (tok * p.hq + h) * D + 8 * c8 + 4, acc2[0] * inv, acc2[1] * inv, acc2[2] * inv,
               acc2[3] * inv);
  if (p.lse && c8 == 0) p.lse[tok * p.hq + h] = l_run > 0.f ? m_run + __logf(l_run) : neg_inf();
}

// Launches kern over the (split, head group, sequence) grid with nw waves
// per workgroup, then the merge of the split partials.
template <int D, typename OutT, typename Kern>
ma_status launch_split(const VerifyArgs &a, const VerifyParams &prm, const Shape &sh, Kern kern, int nw,
                       size_t lds) {
  hipError_t e = hipSuccess;
  if (lds > 64 * 1024) e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return set_error(MA_ERR_HIP, "hipFuncSetAttribute: %s", hipGetErrorString(e));
  hipStream_t s = (hipStream_t)a.stream;
  hipLaunchKernelGGL(kern, dim3(sh.sp.max_splits, a.hq / sh.gh, a.batch), dim3(nw * 64), lds, s, prm);
  e = hipGetLastError();
  if (e != hipSuccess) return set_error(MA_ERR_HIP, "verify launch: %s", hipGetErrorString(e));
  if (sh.sp.max_splits > 1) {
    const int chunks = (a.max_q * (D / 4) + 255) / 256;
    hipLaunchKernelGGL((verify_combine<D, OutT>), dim3(a.hq, a.batch, chunks), dim3(256), 0, s, prm);
    e = hipGetLastError();
    if (e != hipSuccess) return set_error(MA_ERR_HIP, "verify combine launch: %s", hipGetErrorString(e));
  }
  return MA_OK;
}

template <int D, int NW, typename OutT>
ma_status run(const VerifyArgs &a, const VerifyParams &prm, const Shape &sh) {
  size_t lds = 2 * Stage<D>::BYTES;
  // Uniform pages: the rows of one gather instruction share a page whose
  // bytes a 32-bit offset reaches.
  const bool up = (1 << a.page_shift) >= KvDma<D, NW>::RPI &&
                  ((int64_t)1 << a.page_shift) * a.s_slot * 2 < ((int64_t)1 << 31);
  auto kern = up ? verify_kernel<D, NW, OutT, true> : verify_kernel<D, NW, OutT, false>;
  if (a.kv8) {
    // two fp8 stages (K, V bytes) and one bf16 stage; the host checked the
    // page size (at least 1024 / d keys) and the 32-bit offsets
    kern = verify_kernel<D, NW, OutT, true, true>;
    lds = 2 * (2 * 64 * D) + Stage<D>::BYTES;
  }
  return launch_split<D, OutT>(a, prm, sh, kern, NW, lds);
}

// The wave-split decode kernel with NW waves: one stage per wave (bf16), or
// per wave fp8 K and V tiles and a one-matrix bf16 buffer (e4m3); the merge
// reuses them.
template <int D, int NW, typename OutT>
ma_status run_waves(const VerifyArgs &a, const VerifyParams &prm, const Shape &sh) {
  if (a.kv8)
    return launch_split<D, OutT>(a, prm, sh, decode_waves_kernel<D, NW, OutT, true>, NW, (size_t)NW * 4 * 64 * D);
  return launch_split<D, OutT>(a, prm, sh, decode_waves_kernel<D, NW, OutT, false>, NW, (size_t)NW * Stage<D>::BYTES);
}

template <int D, typename OutT>
ma_status run_nw(const VerifyArgs &a, const VerifyParams &prm, const Shape &sh) {
  if constexpr (D == 256) {
    if (sh.nw != 4) return set_error(MA_ERR_UNSUPPORTED, "%d waves at head_dim 256", sh.nw);
    return run<D, 4, OutT>(a, prm, sh);
  } else {
    if (sh.waves_split) {
      if (sh.nw == kDecodeWaves128) return run_waves<D, kDecodeWaves128, OutT>(a, prm, sh);
      if (sh.nw != 4) return set_error(MA_ERR_UNSUPPORTED, "%d decode waves", sh.nw);
      return run_waves<D, 4, OutT>(a, prm, sh);
    }
    switch (sh.nw) {
      case 1: return run<D, 1, OutT>(a, prm, sh);
      case 2: return run<D, 2, OutT>(a, prm, sh);
      case 4: return run<D, 4, OutT>(a, prm, sh);
    }
    return run<D, 8, OutT>(a, prm, sh);
  }
}

template <int D>
ma_status run_d(const VerifyArgs &a, const VerifyParams &prm, const Shape &sh) {
  if (a.out_dtype == MA_F32) return run_nw<D, float>(a, prm, sh);
  return run_nw<D, uint16_t>(a, prm, sh);
}

int mode_of(int32_t kind) {
  switch (kind) {
    case MA_KIND_DENSE_BOOL: return kDense;
    case MA_KIND_PACKED_U64: return kPacked;
    case MA_KIND_CAUSAL: return kCausal;
    case MA_KIND_SLIDING_WINDOW: return kWindow;
    default: return kPrefix;
  }
}

// The workspace a launch uses: max_splits x max_q partial rows per head and
// sequence (none when one split suffices).  The window only shortens the
// walk, so the bound for the whole context holds for every kind.
size_t workspace_bytes(const Shape &sh, int32_t batch, int32_t max_q, int32_t hq, int32_t d) {
  if (sh.sp.max_splits <= 1) return 0;
  return (size_t)batch * sh.sp.max_splits * hq * max_q * (d + 1) * sizeof(float);
}

// Shape of a balanced tree-verify launch (verify_pipe_kernel): custom masks
// (dense or packed rows) and the causal and prefix masks (computed per row;
// a sliding window keeps the split kernels, whose walks start at the window)
// over bf16 caches at d <= 128 whose pages hold a gather instruction's rows
// (`pages_ok`), with GH query heads x max_q rows per unit filling more than
// half of its eight waves (smaller row sets, e.g. decode, keep the split
// kernels).
struct PipeShape {
  bool ok;
  int gh, nhb, grid;
};

PipeShape pipe_shape(int batch, int hq, int hkv, int d, int max_q, int max_kv, int mode, bool pages_ok, bool kv8) {
  PipeShape s{false, 1, 1, 1};
  if ((mode != kDense && mode != kPacked && mode != kCausal && mode != kPrefix) || kv8 || d > 128 || !pages_ok)
    return s;
  const int group = hq / hkv;
  int gh = 1;
  for (int c = group; c >= 1; --c)
    if (group % c == 0 && c * max_q <= kPipeRows) {
      gh = c;
      break;
    }
  if (gh * max_q <= kPipeRows / 2) return s;
  const int64_t units = (int64_t)batch * (hq / gh);
  const int64_t wmax = units * ((max_kv + 63) / 64);
  if (wmax >= ((int64_t)1 << 30)) return s;
  // at least one workgroup per unit (the partition needs it), else one per
  // CU, never more than there are tiles
  int64_t grid = units > kPipeGrid ? units : kPipeGrid;
  if (grid > wmax) grid = wmax;
  s.ok = true;
  s.gh = gh;
  s.nhb = hq / gh;
  s.grid = (int)grid;
  return s;
}

// Workspace of a balanced launch: one partial (O, LSE) slot of 256 rows per
// workgroup, one record per unit, and room for the words the kernel makes
// from dense rows ([batch][max_q][ceil(max_kv / 64)]).
struct PipeWs {
  size_t o, lse, units, words, total;
};

PipeWs pipe_ws(const PipeShape &s, int32_t batch, int32_t max_q, int32_t max_kv, int32_t d) {
  PipeWs w{0, 0, 0, 0, 0};
  if (!s.ok) return w;
  const size_t slots = (size_t)s.grid;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  w.o = 0;
  w.lse = up(slots * kPipeRows * d * sizeof(float));
  w.units = w.lse + up(slots * kPipeRows * sizeof(float));
  w.words = w.units + up((size_t)batch * s.nhb * sizeof(UnitRec));
  w.total = w.words + (size_t)batch * max_q * ((max_kv + 63) / 64) * sizeof(uint64_t);
  return w;
}

template <int D, typename OutT>
ma_status run_pipe(const VerifyArgs &a, VerifyParams prm, const PipeShape &ps) {
  hipStream_t s = (hipStream_t)a.stream;
  const PipeWs w = pipe_ws(ps, a.batch, a.max_q, a.max_kv, a.d);
  char *ws = (char *)a.workspace;
  prm.ws_o = (float *)(ws + w.o);
  prm.ws_lse = (float *)(ws + w.lse);
  UnitRec *units = (UnitRec *)(ws + w.units);
  hipError_t e = hipSuccess;
  prm.dense = nullptr;
  prm.dense_numel = 0;
  if (prm.mode == kDense) {
    // the main kernel turns the dense rows it reads into packed words in the
    // workspace and reads those (words at or past cap are never written)
    prm.dense = prm.mask;
    prm.dense_numel = prm.mask_numel;
    prm.mask = ws + w.words;
    prm.mask_numel = (int64_t)a.batch * a.max_q * ((a.max_kv + 63) / 64);
    prm.mode = kPacked;
  }
  const size_t lds = (size_t)kPipeStages * PipeStage<D>::BYTES;
  const bool pos = prm.mode == kCausal || prm.mode == kPrefix;
  auto kern = pos ? verify_pipe_kernel<D, OutT, true> : verify_pipe_kernel<D, OutT, false>;
  if (lds > 64 * 1024) {
    e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return set_error(MA_ERR_HIP, "hipFuncSetAttribute: %s", hipGetErrorString(e));
  }
  hipLaunchKernelGGL(kern, dim3(ps.grid), dim3(kPipeWaves * 64), lds, s, prm, units);
  e = hipGetLastError();
  if (e != hipSuccess) return set_error(MA_ERR_HIP, "verify launch: %s", hipGetErrorString(e));
  hipLaunchKernelGGL((verify_pipe_combine<D, OutT>), dim3(a.batch * ps.nhb, kPipeRows * (D / 8) / 256), dim3(256), 0,
                     s, prm, (const UnitRec *)units);
  e = hipGetLastError();
  if (e != hipSuccess) return set_error(MA_ERR_HIP, "verify combine launch: %s", hipGetErrorString(e));
  return MA_OK;
}

}  // namespace

// Scratch for callers that cannot allocate (attn_verify_tree_noalloc): one
// array of kVerifyScratchBytes per GPU, held until the process ends.  Host
// code never uses the array's name as an address: it asks the runtime for
// each device's copy once (hipGetSymbolAddress, with that device current)
// and passes that pointer to the kernels.
static __device__ __align__(256) unsigned char scratch[kVerifyScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

ma_status verify_scratch(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(MA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return set_error(MA_ERR_UNSUPPORTED, "device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return set_error(MA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MA_OK;
}

size_t verify_workspace(int32_t batch, int32_t max_q, int32_t max_kv, int32_t hq, int32_t hkv, int32_t d) {
  const Shape sh = shape_for(batch, hq, hkv, d, max_q, max_walk_tiles(kDense, 0, max_q, max_kv));
  const size_t split = workspace_bytes(sh, batch, max_q, hq, d);
  const size_t pipe = pipe_ws(pipe_shape(batch, hq, hkv, d, max_q, max_kv, kDense, true, false), batch, max_q,
                              max_kv, d).total;
  return split > pipe ? split : pipe;
}

ma_status launch_verify(const VerifyArgs &a) {
  const int mode = mode_of(a.mask_kind);
  const bool positional = mode == kCausal || mode == kWindow || mode == kPrefix;
  // pages of at least one gather instruction's rows (512 / d keys) whose
  // bytes a 32-bit offset reaches
  const bool uniform = (1 << a.page_shift) >= 512 / a.d &&
                       ((int64_t)1 << a.page_shift) * a.s_slot * 2 < ((int64_t)1 << 31);
  Shape sh = shape_for(a.batch, a.hq, a.hkv, a.d, a.max_q, max_walk_tiles(mode, a.window, a.max_q, a.max_kv),
                       positional, uniform, a.kv8 != 0);
  // Never more splits than the whole-context shape the workspace was sized for.
  const Shape full = shape_for(a.batch, a.hq, a.hkv, a.d, a.max_q, max_walk_tiles(kDense, 0, a.max_q, a.max_kv));
  if (sh.sp.max_splits > full.sp.max_splits) sh.sp = full.sp;
  VerifyParams prm{};
  prm.q = a.q;
  prm.k = a.k;
  prm.v = a.v;
  prm.page_table = a.page_table;
  prm.cu_seqlens_q = a.cu_seqlens_q;
  prm.kv_lens = a.kv_lens;
  prm.mask = a.mask;
  prm.mask_numel = a.mask_numel;
  prm.prefix_len = a.prefix_len;
  prm.out = a.out;
  prm.lse = a.lse;
  prm.ws_o = (float *)a.workspace;
  prm.ws_lse = sh.sp.max_splits > 1 ? prm.ws_o + (size_t)a.batch * sh.sp.max_splits * a.hq * a.max_q * a.d : nullptr;
  prm.s_page = a.s_page;
  prm.s_slot = a.s_slot;
  prm.s_head = a.s_head;
  prm.max_pages = a.max_pages;
  prm.page_shift = a.page_shift;
  prm.hq = a.hq;
  prm.group = a.hq / a.hkv;
  prm.gh = sh.gh;
  prm.qs = a.max_q;
  prm.mode = mode;
  prm.window = a.window;
  prm.tiles_per_split = sh.sp.tiles_per_split;
  prm.max_splits = sh.sp.max_splits;
  prm.max_kv = a.max_kv;
  prm.scale = a.scale;
  prm.scale_log2 = a.scale * (a.kv8 ? a.k_descale : 1.f) * kLog2e;
  prm.v_scale = a.kv8 ? a.v_descale : 1.f;
  const bool pipe_pages = uniform && a.s_page * 2 < ((int64_t)1 << 32);
  const PipeShape ps = pipe_shape(a.batch, a.hq, a.hkv, a.d, a.max_q, a.max_kv, mode, pipe_pages, a.kv8 != 0);
  if (ps.ok) {
    prm.gh = ps.gh;
    prm.nhb = ps.nhb;
    prm.grid = ps.grid;
    prm.batch = a.batch;
    const bool f32 = a.out_dtype == MA_F32;
    if (a.d == 64) return f32 ? run_pipe<64, float>(a, prm, ps) : run_pipe<64, uint16_t>(a, prm, ps);
    return f32 ? run_pipe<128, float>(a, prm, ps) : run_pipe<128, uint16_t>(a, prm, ps);
  }
  switch (a.d) {
    case 64: return run_d<64>(a, prm, sh);
    case 128: return run_d<128>(a, prm, sh);
    case 256: return run_d<256>(a, prm, sh);
  }
  return set_error(MA_ERR_UNSUPPORTED, "head_dim %d", a.d);
}

}  // namespace maskattn
