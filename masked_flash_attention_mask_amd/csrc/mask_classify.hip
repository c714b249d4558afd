// Device classification of a device-resident custom mask (dense uint8 or
// bit-packed uint64 rows) into a plan, stream-ordered, with no host round
// trip for the mask itself.  An HBM scan: the mask is read once, coalesced,
// and only PARTIAL tiles' words are written.
//
// Pass 1: one workgroup (4 waves) per (q-tile row, chunk of 64 k-tiles for
// packed rows, 48 for dense ones), all chunks of all rows at once, gives
// each tile position its class byte and
// writes the PARTIAL tiles' word blocks (tile_q words each, one block per
// tile position):
//  * packed rows (classify_packed_kernel): wave w takes 32 rows of the
//    q-tile, lane l tile l of the chunk; a lane loads its tile's 32 words (a
//    row's 64 words are one 512-byte load across the wave) and reduces them
//    in registers; the four row groups combine through LDS flags.
//  * dense rows (classify_kernel): wave w takes a quarter of the q-tile's
//    rows and reads them one after another,
//    each row's chunk (up to 3 KB) in 1 KB loads along the row, turns each
//    lane's 16 bytes into bits (SWAR), and the four lanes of a tile put its
//    word together (four rows in flight per wave); the words go through
//    LDS, where each wave scans a quarter of the rows for "some bit set" and
//    "every in-bounds row full".
// Pass 2 (compact_kernel): one wave per q-tile row appends the row's non-SKIP
// tiles, in ascending k order, to its entry list.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <type_traits>

#include "internal.h"
#include "kernels_common.h"

namespace maskattn {
namespace {

constexpr int kTiles = 64;     // k-tiles per chunk (packed rows)
constexpr int kDenseTiles = 48;                   // k-tiles per chunk (dense rows): 49.5 KB of LDS
constexpr int kDenseLoads = kDenseTiles * 64 / 1024;   // 1 KB loads per row and chunk
static_assert(kDenseTiles % 16 == 0 && kDenseTiles <= 64, "a chunk is whole 1 KB loads, one tile per lane at most");
constexpr int kThreads = 256;  // 4 waves
constexpr int kDenseRows = 4;  // dense rows in flight per wave (3 KB each)

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

// The sequence holding q-tile row r (aux row bases ascend): binary search.
__device__ __forceinline__ int seq_of_row(const ClassifyParams &p, int r) {
  int lo = 0, hi = p.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.aux[mid].row_base <= r) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Pass 1 (dense masks): workgroup (q-tile row r, chunk ch) classifies k-tiles
// [48 ch, 48 ch + 48) of row r: their classes go to cls (one byte per tile
// position) and the PARTIAL tiles' word blocks to their tile positions.
// Every chunk of every row runs at once, so the whole mask is in flight; the
// chunk's words (49.5 KB at tile_q 128) leave room for three workgroups per
// CU.
__global__ __launch_bounds__(kThreads) void classify_kernel(ClassifyParams p, uint8_t *cls) {
  extern __shared__ uint64_t wl[];                 // [kDenseTiles][tile_q + 1] words of the chunk
  __shared__ uint32_t any_q[4][kDenseTiles], full_q[4][kDenseTiles];
  __shared__ uint8_t cls_s[kDenseTiles];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.x;
  const int b = seq_of_row(p, r);
  const SeqInfo sq = p.seqs[b];
  const SeqAux ax = p.aux[b];
  const int a = r - ax.row_base;
  const int nkt = sq.nkt, kv = sq.kv_len;
  const int c0 = blockIdx.y * kDenseTiles;
  if (c0 >= nkt) return;
  const int tq = p.tile_q, ws = p.tile_q + 1;      // LDS row stride (words), padded
  const int rows_in = min(tq, sq.q_len - a * tq);  // in-bounds rows of this q-tile
  const int64_t ebase = ax.tile_base + (int64_t)a * nkt;  // tile positions of this row
  const uint8_t *m8 = (const uint8_t *)p.mask;
  const int cn = min(kDenseTiles, nkt - c0);
  // ---- 1. words of the chunk -> LDS: wave w takes rows [w tq / 4, (w + 1) tq / 4)
  {
    const int rpw = tq / 4, q0w = wave * rpw;
    const int row0 = a * tq + q0w;
    {
      // One row at a time, read along the row: lane l of load k takes the
      // row's bytes [64 c0 + 1024 k + 16 l, + 16), keys 16 (l % 4) .. + 15
      // of tile c0 + 16 k + l / 4; the four lanes of a quad hold one tile,
      // whose word their first lane assembles (quad permutes) and stores.
      // Every load is issued (lanes past the row or the mask read the mask's
      // last 16 bytes and discard them), so the compiler's waits cover whole
      // batches.  Bytes past kv_len belong to the next row and are masked.
      const int nbytes = min(64 * cn, kv - 64 * c0);   // the row's bytes in this chunk
      const int lofs = 16 * lane;
      // FAST: the mask holds at least 16 bytes, so its last 16 are a valid
      // stand-in address for lanes that read nothing
      auto rows = [&](auto fast_tag) {
        constexpr bool FAST = decltype(fast_tag)::value;
        const uint8_t *dummy = m8 + (FAST ? p.mask_numel - 16 : 0);
        for (int i0 = 0; i0 < rpw; i0 += kDenseRows) {
          dev::u32x4 v[kDenseRows][kDenseLoads];
          bool ok[kDenseRows][kDenseLoads];
#pragma unroll
          for (int ii = 0; ii < kDenseRows; ++ii)
#pragma unroll
            for (int k = 0; k < kDenseLoads; ++k) {
              const int row = row0 + i0 + ii;
              const int off = 1024 * k + lofs;
              const int64_t base = ax.moff + (int64_t)row * kv + 64 * c0 + off;
              ok[ii][k] = FAST && row < sq.q_len && off < nbytes && base + 16 <= p.mask_numel;
              if constexpr (FAST) __builtin_memcpy(&v[ii][k], ok[ii][k] ? m8 + base : dummy, 16);
            }
#pragma unroll
          for (int ii = 0; ii < kDenseRows; ++ii) {
            const int row = row0 + i0 + ii;
#pragma unroll
            for (int k = 0; k < kDenseLoads; ++k) {
              const int off = 1024 * k + lofs;
              uint32_t bits = 0;
              if (ok[ii][k]) {
#pragma unroll
                for (int c = 0; c < 4; ++c) bits |= nonzero_bytes4(v[ii][k][c]) << (4 * c);
              }
              // a lane whose 16 bytes run past the end of the mask reads its
              // row's bytes one by one (only at the mask's end), in a branch
              // the wave skips when no lane needs it
              const bool slow = row < sq.q_len && off < nbytes && !ok[ii][k];
              if (__any(slow)) {
                if (slow) {
                  const int64_t base = ax.moff + (int64_t)row * kv + 64 * c0 + off;
                  for (int j = 0; j < 16; ++j)
                    if (base + j < p.mask_numel && m8[base + j] != 0) bits |= 1u << j;
                }
              }
              const int nb = nbytes - off;   // bytes of this lane inside the row
              if (nb < 16) bits &= nb <= 0 ? 0u : (1u << nb) - 1u;
              // the quad's other three lanes (quad permutes: lane j of a
              // quad reads lane j + 1, j + 2, j + 3 modulo 4)
              const uint32_t b1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)bits, 0x39, 0xF, 0xF, false);
              const uint32_t b2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)bits, 0x4E, 0xF, 0xF, false);
              const uint32_t b3 = (uint32_t)__builtin_amdgcn_mov_dpp((int)bits, 0x93, 0xF, 0xF, false);
              const int t = 16 * k + (lane >> 2);
              if ((lane & 3) == 0 && t < cn)
                wl[t * ws + q0w + i0 + ii] =
                    (((uint64_t)(b2 | (b3 << 16)) << 32) | (bits | (b1 << 16))) &
                    band_bits(row, c0 + t, sq.q_len, kv, p.window);
            }
          }
        }
      };
      if (p.mask_numel >= 16)
        rows(std::true_type{});
      else
        rows(std::false_type{});
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
    if (t < kDenseTiles) {   // a chunk has fewer tiles than a wave has lanes
      any_q[wave][t] = any;
      full_q[wave][t] = full;
    }
  }
  __syncthreads();
  if (wave == 0) {
    int c = MA_TILE_SKIP;
    if (lane < cn) {
      const bool any = (any_q[0][lane] | any_q[1][lane] | any_q[2][lane] | any_q[3][lane]) != 0;
      const bool full = (full_q[0][lane] & full_q[1][lane] & full_q[2][lane] & full_q[3][lane]) != 0;
      c = !any ? MA_TILE_SKIP : (full ? MA_TILE_FULL : MA_TILE_PARTIAL);
      cls[ebase + c0 + lane] = (uint8_t)c;
    }
    if (lane < kDenseTiles) cls_s[lane] = (uint8_t)c;
  }
  __syncthreads();
  // ---- 3. word blocks of the PARTIAL tiles
  for (int idx = tid; idx < cn * tq; idx += kThreads) {
    const int t = idx / tq, q = idx - t * tq;
    if (cls_s[t] == MA_TILE_PARTIAL) p.words[(ebase + c0 + t) * tq + q] = wl[t * ws + q];
  }
}

// Pass 1 for packed masks, without LDS staging: workgroup (q-tile row r,
// chunk ch), wave w takes the rows [32 w, 32 w + 32) of the q-tile and lane l
// tile 64 ch + l: the lane loads its tile's 32 words (row-contiguous across
// lanes: one 512-byte load per row) and reduces them in registers to "some
// bit set" / "every in-bounds row full"; the row quarters combine through a
// few LDS flags, and the lanes of PARTIAL tiles write their words from
// registers.
__global__ __launch_bounds__(kThreads) void classify_packed_kernel(ClassifyParams p, uint8_t *cls) {
  __shared__ uint32_t any_q[4][kTiles], full_q[4][kTiles];
  __shared__ uint8_t cls_s[kTiles];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.x;
  const int b = seq_of_row(p, r);
  const SeqInfo sq = p.seqs[b];
  const SeqAux ax = p.aux[b];
  const int a = r - ax.row_base;
  const int nkt = sq.nkt, kv = sq.kv_len;
  const int c0 = blockIdx.y * kTiles;
  if (c0 >= nkt) return;
  const int tq = p.tile_q;
  const int cn = min(kTiles, nkt - c0);
  const int64_t ebase = ax.tile_base + (int64_t)a * nkt;
  const int64_t nw = (kv + 63) / 64;
  const uint64_t *m64 = (const uint64_t *)p.mask;
  const int c = c0 + lane;
  const int keys = kv - 64 * c;
  const uint64_t inb = keys >= 64 ? ~0ull : (keys <= 0 ? 0ull : ((1ull << keys) - 1ull));
  const int row0 = a * tq + wave * 32;
  const bool wave_rows = wave * 32 < tq;
  uint64_t w[32];
  uint32_t any = 0, full = 1;
  if (wave_rows) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int row = row0 + i;
      const int64_t idx = ax.moff + (int64_t)row * nw + c;
      w[i] = (lane < cn && row < sq.q_len && idx < p.mask_numel) ? m64[idx] : 0ull;
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      w[i] &= inb & band_bits(row0 + i, c, sq.q_len, kv, p.window);
      if (row0 + i < sq.q_len) {
        any |= w[i] != 0 ? 1u : 0u;
        full &= w[i] == inb ? 1u : 0u;
      }
    }
  }
  any_q[wave][lane] = any;
  full_q[wave][lane] = full;
  __syncthreads();
  if (wave == 0) {
    int k = MA_TILE_SKIP;
    if (lane < cn) {
      const bool an = (any_q[0][lane] | any_q[1][lane] | any_q[2][lane] | any_q[3][lane]) != 0;
      const bool fu = (full_q[0][lane] & full_q[1][lane] & full_q[2][lane] & full_q[3][lane]) != 0;
      k = !an ? MA_TILE_SKIP : (fu ? MA_TILE_FULL : MA_TILE_PARTIAL);
      cls[ebase + c] = (uint8_t)k;
    }
    cls_s[lane] = (uint8_t)k;
  }
  __syncthreads();
  if (wave_rows && lane < cn && cls_s[lane] == MA_TILE_PARTIAL) {
    uint64_t *dst = p.words + (ebase + c) * tq + wave * 32;
#pragma unroll
    for (int i = 0; i < 32; ++i) dst[i] = w[i];
  }
}

// Pass 2: one wave per q-tile row appends the row's non-SKIP tiles, in
// ascending k order, to its entry list and writes its work item (rows in
// reverse order: the longest rows of causal-like masks first).
__global__ __launch_bounds__(64) void compact_kernel(ClassifyParams p, const uint8_t *cls) {
  const int lane = threadIdx.x;
  const int r = blockIdx.x;
  const int b = seq_of_row(p, r);
  const SeqInfo sq = p.seqs[b];
  const SeqAux ax = p.aux[b];
  const int a = r - ax.row_base;
  const int nkt = sq.nkt;
  const int64_t ebase = ax.tile_base + (int64_t)a * nkt;
  int32_t count = 0;
  for (int c0 = 0; c0 < nkt; c0 += 64) {
    const int c = c0 + lane;
    const int k = c < nkt ? cls[ebase + c] : MA_TILE_SKIP;
    const uint64_t bal = __ballot(k != MA_TILE_SKIP);
    if (k != MA_TILE_SKIP) {
      const int before = __popcll(bal & ((1ull << lane) - 1ull));
      p.entries[ebase + count + before] = Entry{c | (k << kClsShift), k == MA_TILE_PARTIAL ? (int32_t)(ebase + c) : -1};
    }
    count += __popcll(bal);
  }
  if (lane == 0) p.items[p.num_rows - 1 - r] = Item{b, a, (int32_t)ebase, (int32_t)(ebase + count)};
}

}  // namespace

ma_status launch_classify(ma_plan *p, const void *mask, int32_t kind, int64_t mask_numel, int32_t window,
                          void *stream) {
  if (p->num_tiles > INT32_MAX) return set_error(MA_ERR_UNSUPPORTED, "too many tiles for a device-built plan");
  // one class byte per tile position after the word blocks (pass 1 -> pass 2)
  ma_status st = plan_alloc_device(p, p->num_tiles, p->num_tiles, (size_t)p->num_tiles);
  if (st != MA_OK) return st;
  std::vector<SeqInfo> seqs;
  std::vector<SeqAux> aux;
  fill_seqinfo(p, kind, seqs, aux);
  // The metadata goes through a pinned staging buffer the plan keeps until
  // it is destroyed: the copy is stream-ordered and nothing waits for it.
  const size_t meta = sizeof(SeqInfo) * seqs.size() + sizeof(SeqAux) * aux.size();
  if ((st = plan_staging(p, meta)) != MA_OK) return st;
  char *h = (char *)p->staging;
  memcpy(h, seqs.data(), sizeof(SeqInfo) * seqs.size());
  memcpy(h + sizeof(SeqInfo) * seqs.size(), aux.data(), sizeof(SeqAux) * aux.size());
  hipStream_t s = (hipStream_t)stream;
  char *base = (char *)p->dbuf;
  hipError_t e = hipMemcpyAsync(base + p->off_seqs, h, sizeof(SeqInfo) * seqs.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(base + p->off_aux, h + sizeof(SeqInfo) * seqs.size(), sizeof(SeqAux) * aux.size(),
                       hipMemcpyHostToDevice, s);
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
  uint8_t *cls = (uint8_t *)(base + p->off_extra);
  int32_t max_nkt = 1;
  for (int b = 0; b < p->batch; ++b) max_nkt = std::max(max_nkt, p->nkt[b]);
  if (prm.packed) {
    const dim3 grid(p->num_rows, (max_nkt + kTiles - 1) / kTiles);
    hipLaunchKernelGGL(classify_packed_kernel, grid, dim3(kThreads), 0, s, prm, cls);
  } else {
    const dim3 grid(p->num_rows, (max_nkt + kDenseTiles - 1) / kDenseTiles);
    const size_t lds = (size_t)kDenseTiles * (p->tile_q + 1) * sizeof(uint64_t);
    e = hipSuccess;
    if (lds > 64 * 1024)
      e = hipFuncSetAttribute((const void *)classify_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return set_error(MA_ERR_HIP, "hipFuncSetAttribute: %s", hipGetErrorString(e));
    hipLaunchKernelGGL(classify_kernel, grid, dim3(kThreads), lds, s, prm, cls);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return set_error(MA_ERR_HIP, "classify launch: %s", hipGetErrorString(e));
  hipLaunchKernelGGL(compact_kernel, dim3(p->num_rows), dim3(64), 0, s, prm, (const uint8_t *)cls);
  e = hipGetLastError();
  if (e != hipSuccess) return set_error(MA_ERR_HIP, "classify compaction launch: %s", hipGetErrorString(e));
  return MA_OK;
}

}  // namespace maskattn
