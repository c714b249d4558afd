// Device classification of a device-resident custom mask (dense uint8 or
// bit-packed uint64 rows) into a plan, stream-ordered, with no host round
// trip for the mask itself.
//
// One workgroup per q-tile row.  Each wave owns 32 rows of the tile.  For
// every k-tile, the wave forms each row's 64-bit word (a packed mask is read
// one word per row; a dense mask is read one byte per lane and turned into a
// word with a wavefront ballot, so a row's 64 bytes are one coalesced load),
// stores it in the plan's per-tile word layout, and records with ballots
// whether all its in-bounds rows are full or empty.  A second pass combines
// the waves' flags into FULL / SKIP / PARTIAL and compacts the non-SKIP tiles,
// in ascending k order, into the row's entry list with a block scan.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "kernels_common.h"

namespace maskattn {
namespace {

constexpr int kChunk = 256;  // k-tiles per pass; also the block size

struct ClassifyParams {
  const SeqInfo *seqs;
  const SeqAux *aux;
  Item *items;
  Entry *entries;
  uint64_t *words;
  const void *mask;
  int64_t mask_numel;
  int32_t batch, num_rows, tile_q, packed;
};

__global__ __launch_bounds__(kChunk) void classify_kernel(ClassifyParams p) {
  __shared__ uint8_t flags[4][kChunk];
  __shared__ int32_t wave_tot[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.x;
  int b = 0;
  while (b + 1 < p.batch && r >= p.aux[b + 1].row_base) ++b;
  const SeqInfo sq = p.seqs[b];
  const SeqAux ax = p.aux[b];
  const int a = r - ax.row_base;
  const int nkt = sq.nkt, kv = sq.kv_len;
  const int nwave_rows = p.tile_q / 32;
  const int64_t ebase = ax.tile_base + (int64_t)a * nkt;  // entries / word blocks of this row
  const int64_t nw = (kv + 63) / 64;
  int32_t count = 0;

  for (int c0 = 0; c0 < nkt; c0 += kChunk) {
    const int cn = min(kChunk, nkt - c0);
    if (wave < nwave_rows) {
      for (int ci = 0; ci < cn; ++ci) {
        const int c = c0 + ci;
        const int keys = min(64, kv - 64 * c);
        const uint64_t inb = keys >= 64 ? ~0ull : ((1ull << keys) - 1ull);
        uint64_t w = 0;  // word of row (wave*32 + lane) for lanes < 32
        const int row0 = a * p.tile_q + wave * 32;
        if (p.packed) {
          const int row = row0 + lane;
          if (lane < 32 && row < sq.q_len) {
            const int64_t idx = ax.moff + (int64_t)row * nw + c;
            if (idx < p.mask_numel) w = ((const uint64_t *)p.mask)[idx] & inb;
          }
        } else {
          const uint8_t *m8 = (const uint8_t *)p.mask;
          for (int i = 0; i < 32; ++i) {
            const int row = row0 + i;
            bool bit = false;
            if (row < sq.q_len && lane < keys) {
              const int64_t idx = ax.moff + (int64_t)row * kv + 64 * c + lane;
              bit = idx < p.mask_numel && m8[idx] != 0;
            }
            const uint64_t word = __ballot(bit);
            if (lane == i) w = word;
          }
        }
        const bool valid = lane < 32 && row0 + lane < sq.q_len;
        if (lane < 32) p.words[(ebase + c) * p.tile_q + wave * 32 + lane] = w;
        const uint64_t vmask = __ballot(valid);
        const uint64_t fullm = __ballot(valid && w == inb);
        const uint64_t nzm = __ballot(valid && w != 0);
        if (lane == 0) flags[wave][ci] = (uint8_t)((nzm != 0 ? 1 : 0) | (fullm == vmask ? 2 : 0));
      }
    }
    __syncthreads();
    int cls = MA_TILE_SKIP;
    if (tid < cn) {
      bool any = false, all = true;
      for (int wv = 0; wv < nwave_rows; ++wv) {
        any |= (flags[wv][tid] & 1) != 0;
        all &= (flags[wv][tid] & 2) != 0;
      }
      cls = !any ? MA_TILE_SKIP : (all ? MA_TILE_FULL : MA_TILE_PARTIAL);
    }
    const bool keep = cls != MA_TILE_SKIP;
    const uint64_t bal = __ballot(keep);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wave_tot[wave] = __popcll(bal);
    __syncthreads();
    int off = count;
    for (int wv = 0; wv < wave; ++wv) off += wave_tot[wv];
    if (keep) {
      const int c = c0 + tid;
      p.entries[ebase + off + before] =
          Entry{c | (cls << kClsShift), cls == MA_TILE_PARTIAL ? (int32_t)(ebase + c) : -1};
    }
    count += wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
    __syncthreads();
  }
  if (tid == 0)
    p.items[p.num_rows - 1 - r] = Item{b, a, (int32_t)ebase, (int32_t)(ebase + count)};
}

}  // namespace

ma_status launch_classify(ma_plan *p, const void *mask, int32_t kind, int64_t mask_numel, void *stream) {
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
  hipLaunchKernelGGL(classify_kernel, dim3(p->num_rows), dim3(kChunk), 0, s, prm);
  e = hipGetLastError();
  if (e != hipSuccess) return set_error(MA_ERR_HIP, "classify launch: %s", hipGetErrorString(e));
  return MA_OK;
}

}  // namespace maskattn
