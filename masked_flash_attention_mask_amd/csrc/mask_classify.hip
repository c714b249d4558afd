// Device classification of a device-resident custom mask (dense uint8 or
// bit-packed uint64 rows) into a plan, stream-ordered, with no host round
// trip for the mask itself.  An HBM scan: the mask is read once, coalesced,
// and only PARTIAL tiles' words are written.
//
// One workgroup (4 waves) per q-tile row, walking the row's k-tiles in chunks
// of 64.  Per chunk:
//  1. the words of every (row, tile) go to LDS.  Packed rows: a wave reads 64
//     consecutive words of one row per load (512 B).  Dense rows: lanes 2i and
//     2i + 1 read the two 32-byte halves of wave row i's 64 bytes of a tile,
//     turn them into bits (SWAR), and two shuffles give row i's word to lane
//     i; eight tiles are in flight per wave.
//  2. each wave scans a quarter of the rows of all 64 tiles in LDS for "some
//     bit set" and "every in-bounds row full"; wave 0 combines the quarters
//     into FULL / SKIP / PARTIAL and appends the non-SKIP tiles, in ascending
//     k order, to the row's entry list.
//  3. the workgroup writes the PARTIAL tiles' word blocks (tile_q words each,
//     one block per tile position).
#include <hip/hip_runtime.h>

#include "internal.h"
#include "kernels_common.h"

namespace maskattn {
namespace {

constexpr int kTiles = 64;     // k-tiles per chunk
constexpr int kThreads = 256;  // 4 waves
constexpr int kDenseBatch = 8; // dense tiles in flight per wave

struct ClassifyParams {
  const SeqInfo *seqs;
  const SeqAux *aux;
  Item *items;
  Entry *entries;
  uint64_t *words;
  const void *mask;
  int64_t mask_numel;
  int32_t batch, num_rows, tile_q, packed;
  int32_t window;   // > 0: the mask is ANDed with the band pos - window < j <= pos
};

// Bits of k-tile c (keys 64 c .. 64 c + 63) inside the sliding-window band of
// local query row `row` (all ones without a window).
__device__ __forceinline__ uint64_t band_bits(int row, int c, int q_len, int kv, int window) {
  if (window <= 0) return ~0ull;
  const int64_t pos = (int64_t)row + kv - q_len;
  const int64_t lo = max((int64_t)0, pos - window + 1 - 64 * (int64_t)c);
  const int64_t hi = min((int64_t)64, pos + 1 - 64 * (int64_t)c);
  if (hi <= lo) return 0ull;
  const uint64_t upper = hi >= 64 ? ~0ull : ((1ull << hi) - 1ull);
  return upper & ~((1ull << lo) - 1ull);
}

// Bits (LSB = lowest address) of the nonzero bytes of a dword: per byte the
// high bit is set iff the byte is nonzero (SWAR), then one multiply moves the
// four high bits to bits 21..24 (distinct partial products, no carries).
__device__ __forceinline__ uint32_t nonzero_bytes4(uint32_t x) {
  const uint32_t t = ((((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x) >> 7) & 0x01010101u;
  return ((t * 0x00204081u) >> 21) & 0xFu;
}

// 32 bits for the bytes [base, base + nb) of a dense mask (nb <= 32).
__device__ __forceinline__ uint32_t dense_half(const uint8_t *m8, int64_t base, int nb, int64_t numel) {
  uint32_t bits = 0;
  if (nb == 32 && base + 32 <= numel) {
    dev::u32x4 v0, v1;
    __builtin_memcpy(&v0, m8 + base, 16);
    __builtin_memcpy(&v1, m8 + base + 16, 16);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bits |= nonzero_bytes4(v0[c]) << (4 * c);
      bits |= nonzero_bytes4(v1[c]) << (16 + 4 * c);
    }
  } else {
    for (int j = 0; j < nb; ++j)
      if (base + j < numel && m8[base + j] != 0) bits |= 1u << j;
  }
  return bits;
}

__global__ __launch_bounds__(kThreads) void classify_kernel(ClassifyParams p) {
  extern __shared__ uint64_t wl[];                 // [kTiles][tile_q + 1] words of the chunk
  __shared__ uint32_t any_q[4][kTiles], full_q[4][kTiles];
  __shared__ uint8_t cls_s[kTiles];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.x;
  int b = 0;
  while (b + 1 < p.batch && r >= p.aux[b + 1].row_base) ++b;
  const SeqInfo sq = p.seqs[b];
  const SeqAux ax = p.aux[b];
  const int a = r - ax.row_base;
  const int nkt = sq.nkt, kv = sq.kv_len;
  const int tq = p.tile_q, ws = p.tile_q + 1;      // LDS row stride (words), padded
  const int ngroups = tq / 32;
  const int rows_in = min(tq, sq.q_len - a * tq);  // in-bounds rows of this q-tile
  const int64_t ebase = ax.tile_base + (int64_t)a * nkt;  // entries / word blocks of this row
  const int64_t nw = (kv + 63) / 64;
  const uint8_t *m8 = (const uint8_t *)p.mask;
  const uint64_t *m64 = (const uint64_t *)p.mask;
  int32_t count = 0;

  for (int c0 = 0; c0 < nkt; c0 += kTiles) {
    const int cn = min(kTiles, nkt - c0);
    // ---- 1. words of the chunk -> LDS
    for (int rg = wave; rg < ngroups; rg += 4) {
      const int row0 = a * tq + rg * 32;
      if (p.packed) {
        // lane l: tile c0 + l of row row0 + i, for the wave's 32 rows
        const int c = c0 + lane;
        const int keys = kv - 64 * c;
        const uint64_t inb = keys >= 64 ? ~0ull : (keys <= 0 ? 0ull : ((1ull << keys) - 1ull));
        // all 32 loads in flight before the first LDS store
        uint64_t w[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const int row = row0 + i;
          const int64_t idx = ax.moff + (int64_t)row * nw + c;
          w[i] = (lane < cn && row < sq.q_len && idx < p.mask_numel) ? m64[idx] : 0ull;
        }
        if (lane < cn) {
#pragma unroll
          for (int i = 0; i < 32; ++i)
            wl[lane * ws + rg * 32 + i] = w[i] & inb & band_bits(row0 + i, c, sq.q_len, kv, p.window);
        }
      } else {
        const int i = lane >> 1, half = lane & 1;
        const int row = row0 + i;
        const bool rv = row < sq.q_len;
        const int64_t rbase = ax.moff + (int64_t)row * kv + 32 * half;
        for (int ci0 = 0; ci0 < cn; ci0 += kDenseBatch) {
          // Interior halves: two 16-byte loads each, all issued before any
          // is used (other lanes load the mask's last 32 bytes and discard
          // them).  Halves cut by kv_len, and masks under 32 bytes, take the
          // byte loop.
          dev::u32x4 v0[kDenseBatch], v1[kDenseBatch];
          bool fast[kDenseBatch];
          const bool can_fast = p.mask_numel >= 32;
          const uint8_t *dummy = m8 + (can_fast ? p.mask_numel - 32 : 0);
#pragma unroll
          for (int u = 0; u < kDenseBatch; ++u) {
            const int c = c0 + ci0 + u;
            const int64_t base = rbase + 64 * c;
            fast[u] = can_fast && rv && ci0 + u < cn && kv - 64 * c - 32 * half >= 32 && base + 32 <= p.mask_numel;
            if (can_fast) {
              const uint8_t *src = fast[u] ? m8 + base : dummy;
              __builtin_memcpy(&v0[u], src, 16);
              __builtin_memcpy(&v1[u], src + 16, 16);
            } else {
              v0[u] = dev::u32x4{0, 0, 0, 0};
              v1[u] = dev::u32x4{0, 0, 0, 0};
            }
          }
          uint32_t bits[kDenseBatch];
#pragma unroll
          for (int u = 0; u < kDenseBatch; ++u) {
            uint32_t x = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              x |= nonzero_bytes4(v0[u][c]) << (4 * c);
              x |= nonzero_bytes4(v1[u][c]) << (16 + 4 * c);
            }
            bits[u] = fast[u] ? x : 0u;
            const int c = c0 + ci0 + u;
            const int nb = min(32, kv - 64 * c - 32 * half);
            if (!fast[u] && rv && ci0 + u < cn && nb > 0) bits[u] = dense_half(m8, rbase + 64 * c, nb, p.mask_numel);
          }
#pragma unroll
          for (int u = 0; u < kDenseBatch; ++u) {
            const int src = 2 * (lane & 31);
            const uint32_t lo = __shfl(bits[u], src, 64), hi = __shfl(bits[u], src + 1, 64);
            if (lane < 32 && ci0 + u < cn)
              wl[(ci0 + u) * ws + rg * 32 + lane] =
                  (((uint64_t)hi << 32) | lo) & band_bits(row0 + lane, c0 + ci0 + u, sq.q_len, kv, p.window);
          }
        }
      }
    }
    __syncthreads();
    // ---- 2. per tile: some bit set / every in-bounds row full (wave = row quarter)
    {
      const int t = lane;
      uint32_t any = 0, full = 1;
      if (t < cn) {
        const int keys = kv - 64 * (c0 + t);
        const uint64_t inb = keys >= 64 ? ~0ull : ((1ull << keys) - 1ull);
        const int q0 = wave * (tq / 4), q1 = min(q0 + tq / 4, rows_in);
        for (int q = q0; q < q1; ++q) {
          const uint64_t w = wl[t * ws + q];
          any |= w != 0 ? 1u : 0u;
          full &= w == inb ? 1u : 0u;
        }
      }
      any_q[wave][t] = any;
      full_q[wave][t] = full;
    }
    __syncthreads();
    if (wave == 0) {
      int cls = MA_TILE_SKIP;
      if (lane < cn) {
        const bool any = (any_q[0][lane] | any_q[1][lane] | any_q[2][lane] | any_q[3][lane]) != 0;
        const bool full = (full_q[0][lane] & full_q[1][lane] & full_q[2][lane] & full_q[3][lane]) != 0;
        cls = !any ? MA_TILE_SKIP : (full ? MA_TILE_FULL : MA_TILE_PARTIAL);
      }
      cls_s[lane] = (uint8_t)cls;
      const uint64_t bal = __ballot(cls != MA_TILE_SKIP);
      if (cls != MA_TILE_SKIP) {
        const int c = c0 + lane;
        const int before = __popcll(bal & ((1ull << lane) - 1ull));
        p.entries[ebase + count + before] =
            Entry{c | (cls << kClsShift), cls == MA_TILE_PARTIAL ? (int32_t)(ebase + c) : -1};
      }
      count += __popcll(bal);
    }
    __syncthreads();
    // ---- 3. word blocks of the PARTIAL tiles
    for (int idx = tid; idx < cn * tq; idx += kThreads) {
      const int t = idx / tq, q = idx - t * tq;
      if (cls_s[t] == MA_TILE_PARTIAL) p.words[(ebase + c0 + t) * tq + q] = wl[t * ws + q];
    }
    __syncthreads();
  }
  if (tid == 0)
    p.items[p.num_rows - 1 - r] = Item{b, a, (int32_t)ebase, (int32_t)(ebase + count)};
}

}  // namespace

ma_status launch_classify(ma_plan *p, const void *mask, int32_t kind, int64_t mask_numel, int32_t window,
                          void *stream) {
  if (p->num_tiles > INT32_MAX) return set_error(MA_ERR_UNSUPPORTED, "too many tiles for a device-built plan");
  ma_status st = plan_alloc_device(p, p->num_tiles, p->num_tiles);
  if (st != MA_OK) return st;
  std::vector<SeqInfo> seqs;
  std::vector<SeqAux> aux;
  fill_seqinfo(p, kind, seqs, aux);
  hipStream_t s = (hipStream_t)stream;
  char *base = (char *)p->dbuf;
  hipError_t e = hipMemcpyAsync(base + p->off_seqs, seqs.data(), sizeof(SeqInfo) * seqs.size(),
                                hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(base + p->off_aux, aux.data(), sizeof(SeqAux) * aux.size(), hipMemcpyHostToDevice, s);
  // The host vectors die with this call: wait for the two small copies.
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return set_error(MA_ERR_HIP, "plan metadata upload: %s", hipGetErrorString(e));
  p->on_device = true;
  p->device_built = true;
  if (p->num_rows == 0) return MA_OK;
  ClassifyParams prm{};
  prm.seqs = (const SeqInfo *)(base + p->off_seqs);
  prm.aux = (const SeqAux *)(base + p->off_aux);
  prm.items = (Item *)(base + p->off_items);
  prm.entries = (Entry *)(base + p->off_entries);
  prm.words = (uint64_t *)(base + p->off_words);
  prm.mask = mask;
  prm.mask_numel = mask_numel;
  prm.batch = p->batch;
  prm.num_rows = p->num_rows;
  prm.tile_q = p->tile_q;
  prm.packed = kind == MA_KIND_PACKED_U64 ? 1 : 0;
  prm.window = window;
  const size_t lds = (size_t)kTiles * (p->tile_q + 1) * sizeof(uint64_t);
  e = hipSuccess;
  if (lds > 64 * 1024)
    e = hipFuncSetAttribute((const void *)classify_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return set_error(MA_ERR_HIP, "hipFuncSetAttribute: %s", hipGetErrorString(e));
  hipLaunchKernelGGL(classify_kernel, dim3(p->num_rows), dim3(kThreads), lds, s, prm);
  e = hipGetLastError();
  if (e != hipSuccess) return set_error(MA_ERR_HIP, "classify launch: %s", hipGetErrorString(e));
  return MA_OK;
}

}  // namespace maskattn
