// Speculative tree verify (gfx950): every sequence's draft-tree queries
// (q_len <= 64) against its cached context plus the draft tokens, under a
// full-row custom mask that changes every decoding step (tree attention
// through a custom mask, flashinfer issue 724).
//
// The mask is classified on the fly, per tile and per wave, instead of in a
// separate pass: each lane fetches its query row's 64-bit word for the tile
// (one word per row of a packed mask; for a dense mask a wavefront ballot
// over 64 contiguous bytes of the row), and a wave whose rows all see the
// whole tile (every context tile) skips masking.
//
// Work split: a workgroup takes GH query heads of one GQA group (two waves of
// 32 rows per head), so each K/V tile gathered from the paged cache serves
// GH heads.  Long contexts are cut into contiguous k-tile ranges handled by
// separate workgroups; each writes a partial (O, LSE) and a second kernel
// merges the partials in fixed split order (deterministic, no atomics).
#include <hip/hip_runtime.h>

#include "internal.h"
#include "kernels_common.h"
#include "tile_dma_bf16.h"

namespace maskattn {
using namespace dev;
using namespace dev::dma;

namespace {

constexpr int kTargetWorkgroups = 512;

struct SplitShape {
  int tiles_per_split;
  int max_splits;
};

SplitShape split_shape(int batch, int max_kv, int hkv) {
  const int max_nkt = (max_kv + 63) / 64;
  int want = (kTargetWorkgroups + batch * hkv - 1) / (batch * hkv);
  want = want < 1 ? 1 : (want > max_nkt ? max_nkt : want);
  const int t = (max_nkt + want - 1) / want;
  return SplitShape{t, (max_nkt + t - 1) / t};
}

// Query heads per workgroup: the largest of 4, 2, 1 that divides the GQA
// group (2 at most for d = 256, whose accumulators fill the register file).
int heads_per_workgroup(int group, int d) {
  const int cap = d == 256 ? 2 : 4;
  for (int gh = cap; gh > 1; gh >>= 1)
    if (group % gh == 0) return gh;
  return 1;
}

struct VerifyParams {
  const void *q, *k, *v;
  const int32_t *page_table;
  const int32_t *cu_seqlens_q, *kv_lens;
  const void *mask;
  int64_t mask_numel;
  void *out;
  float *lse;
  float *ws_o;    // [batch][max_splits][hq][64][d]
  float *ws_lse;  // [batch][max_splits][hq][64]
  int64_t s_page, s_slot, s_head;
  int32_t max_pages, page_shift;
  int32_t hq, group, packed;
  int32_t tiles_per_split, max_splits, max_kv;
  float scale, scale_log2;
};

__device__ __forceinline__ int64_t mask_offset(const VerifyParams &p, int b) {
  int64_t off = 0;
  for (int i = 0; i < b; ++i) {
    const int64_t ql = p.cu_seqlens_q[i + 1] - p.cu_seqlens_q[i], kv = p.kv_lens[i];
    off += p.packed ? ql * ((kv + 63) / 64) : ql * kv;
  }
  return off;
}

// The lane's row word for k-tile kt (rows of this wave: base + 0..31; lanes
// l and l + 32 hold the same row).
__device__ __forceinline__ uint64_t fetch_word(const VerifyParams &p, int64_t moff, int row_base, int q_len,
                                               int kv, int kt, int lane) {
  const int l32 = lane & 31;
  const int keys = min(64, kv - 64 * kt);
  if (p.packed) {
    const int row = row_base + l32;
    if (row >= q_len) return 0ull;
    const int64_t idx = moff + (int64_t)row * ((kv + 63) / 64) + kt;
    return idx < p.mask_numel ? ((const uint64_t *)p.mask)[idx] : 0ull;
  }
  const uint8_t *m8 = (const uint8_t *)p.mask;
  uint64_t w = 0;
  for (int i = 0; i < 32; ++i) {
    const int row = row_base + i;
    bool bit = false;
    if (row < q_len && lane < keys) {
      const int64_t idx = moff + (int64_t)row * kv + 64 * kt + lane;
      bit = idx < p.mask_numel && m8[idx] != 0;
    }
    const uint64_t word = __ballot(bit);
    if (l32 == i) w = word;
  }
  return w;
}

template <int D, int GH, typename OutT>
__global__ __launch_bounds__(GH * 128, 1) void verify_kernel(VerifyParams p) {
  constexpr int NT = GH * 128;
  extern __shared__ __align__(16) uint16_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int split = blockIdx.x, b = blockIdx.z;
  const int q0 = p.cu_seqlens_q[b], q_len = p.cu_seqlens_q[b + 1] - q0;
  const int kv = min(p.kv_lens[b], p.max_kv);  // the page table covers max_kv keys
  const int nkt = (kv + 63) / 64;
  const int nsplit = (nkt + p.tiles_per_split - 1) / p.tiles_per_split;
  if (split >= nsplit && !(split == 0 && nkt == 0)) return;
  const int kt0 = split * p.tiles_per_split;
  const int kt1 = min(nkt, kt0 + p.tiles_per_split);
  const int h = blockIdx.y * GH + (wave >> 1);
  const int g = h / p.group;
  const int row_base = (wave & 1) * 32;
  const int t = row_base + l32;
  const bool row_ok = t < q_len;
  const int64_t tok = (int64_t)q0 + t;
  const int64_t moff = mask_offset(p, b);

  bf16x8 qf[D / 16];
  load_q<D>(qf, (const uint16_t *)p.q + (tok * p.hq + h) * D, row_ok, hi);
  const uint16_t *kbase = (const uint16_t *)p.k + (int64_t)g * p.s_head;
  const uint16_t *vbase = (const uint16_t *)p.v + (int64_t)g * p.s_head;
  const int32_t *pt = p.page_table + (int64_t)b * p.max_pages;
  using KV = KvDma<D, 2 * GH>;
  const LaneOffsets<D> lo(lane);
  const int wave_id = wave;
  typename KV::Pages pg_nxt;

  f32x16 oacc[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n) oacc[n] = f32x16{};
  float m_ref = neg_inf();
  f32x16 lsum = f32x16{};
  const float c = p.scale_log2;

  uint64_t word_nxt = 0;
  if (kt0 < kt1) {
    const typename KV::Pages pg0 = KV::pages(pt, p.page_shift, kt0, kv, wave_id, lane);
    KV::issue(kbase, vbase, pg0, p.page_shift, p.s_page, p.s_slot, kt0, kv, lds, wave_id, lane);
    word_nxt = fetch_word(p, moff, row_base, q_len, kv, kt0, lane);
    if (kt0 + 1 < kt1) pg_nxt = KV::pages(pt, p.page_shift, kt0 + 1, kv, wave_id, lane);
    wait_vmem();
    __syncthreads();
  }
  for (int kt = kt0; kt < kt1; ++kt) {
    const int cur = (kt - kt0) & 1;
    const uint64_t wcur = word_nxt;
    if (kt + 1 < kt1) {
      // The mask word first: a dense mask's ballots wait for its loads, and
      // that wait would otherwise include the gather.
      word_nxt = fetch_word(p, moff, row_base, q_len, kv, kt + 1, lane);
      KV::issue(kbase, vbase, pg_nxt, p.page_shift, p.s_page, p.s_slot, kt + 1, kv,
                lds + (cur ^ 1) * Stage<D>::ELEMS, wave_id, lane);
      if (kt + 2 < kt1) pg_nxt = KV::pages(pt, p.page_shift, kt + 2, kv, wave_id, lane);
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

  const float lt = lsum[0];
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse = lt > 0.f ? (m_ref + __log2f(lt)) * kLn2 : neg_inf();
  if (!row_ok) return;
  if (nsplit <= 1) {
    store_row<D, OutT>((OutT *)p.out + (tok * p.hq + h) * D, oacc, inv, hi);
    if (p.lse && hi == 0) p.lse[tok * p.hq + h] = lse;
  } else {
    const int64_t slot = (((int64_t)b * p.max_splits + split) * p.hq + h) * 64 + t;
    store_row<D, float>(p.ws_o + slot * D, oacc, inv, hi);
    if (hi == 0) p.ws_lse[slot] = lse;
  }
}

// Merges the split partials of one (sequence, query head) in split order:
// O = sum_s exp(LSE_s - M) O_s / sum_s exp(LSE_s - M), LSE = M + ln(sum).
template <int D, typename OutT>
__global__ __launch_bounds__(256) void verify_combine(VerifyParams p) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int q0 = p.cu_seqlens_q[b], q_len = p.cu_seqlens_q[b + 1] - q0;
  const int kv = min(p.kv_lens[b], p.max_kv);
  const int nkt = (kv + 63) / 64;
  const int nsplit = (nkt + p.tiles_per_split - 1) / p.tiles_per_split;
  if (nsplit <= 1) return;
  const int64_t sbase = (int64_t)b * p.max_splits;
  for (int idx = threadIdx.x; idx < q_len * (D / 4); idx += blockDim.x) {
    const int t = idx / (D / 4), c4 = idx % (D / 4);
    float mx = neg_inf();
    for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, p.ws_lse[((sbase + s) * p.hq + h) * 64 + t]);
    float wsum = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (mx != neg_inf()) {
      for (int s = 0; s < nsplit; ++s) {
        const int64_t slot = ((sbase + s) * p.hq + h) * 64 + t;
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

template <int D, int GH, typename OutT>
ma_status run(const VerifyArgs &a, const VerifyParams &prm, const SplitShape &sp) {
  const size_t lds = 2 * Stage<D>::BYTES;
  auto kern = verify_kernel<D, GH, OutT>;
  hipError_t e = hipSuccess;
  if (lds > 64 * 1024) e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return set_error(MA_ERR_HIP, "hipFuncSetAttribute: %s", hipGetErrorString(e));
  hipStream_t s = (hipStream_t)a.stream;
  hipLaunchKernelGGL(kern, dim3(sp.max_splits, a.hq / GH, a.batch), dim3(GH * 128), lds, s, prm);
  e = hipGetLastError();
  if (e != hipSuccess) return set_error(MA_ERR_HIP, "verify launch: %s", hipGetErrorString(e));
  if (sp.max_splits > 1) {
    hipLaunchKernelGGL((verify_combine<D, OutT>), dim3(a.hq, a.batch), dim3(256), 0, s, prm);
    e = hipGetLastError();
    if (e != hipSuccess) return set_error(MA_ERR_HIP, "verify combine launch: %s", hipGetErrorString(e));
  }
  return MA_OK;
}

template <int D, typename OutT>
ma_status run_gh(const VerifyArgs &a, const VerifyParams &prm, const SplitShape &sp) {
  switch (heads_per_workgroup(a.hq / a.hkv, D)) {
    case 1: return run<D, 1, OutT>(a, prm, sp);
    case 2: return run<D, 2, OutT>(a, prm, sp);
    default: return run<D, 4, OutT>(a, prm, sp);
  }
}

template <int D>
ma_status run_d(const VerifyArgs &a, const VerifyParams &prm, const SplitShape &sp) {
  if (a.out_dtype == MA_F32) return run_gh<D, float>(a, prm, sp);
  return run_gh<D, uint16_t>(a, prm, sp);
}

}  // namespace

size_t verify_workspace(int32_t batch, int32_t max_q, int32_t max_kv, int32_t hq, int32_t hkv, int32_t d) {
  (void)max_q;
  const SplitShape sp = split_shape(batch, max_kv, hkv);
  if (sp.max_splits <= 1) return 0;
  return (size_t)batch * sp.max_splits * hq * 64 * (d + 1) * sizeof(float);
}

ma_status launch_verify(const VerifyArgs &a) {
  const int group = a.hq / a.hkv;
  const SplitShape sp = split_shape(a.batch, a.max_kv, a.hkv);
  VerifyParams prm{};
  prm.q = a.q;
  prm.k = a.k;
  prm.v = a.v;
  prm.page_table = a.page_table;
  prm.cu_seqlens_q = a.cu_seqlens_q;
  prm.kv_lens = a.kv_lens;
  prm.mask = a.mask;
  prm.mask_numel = a.mask_numel;
  prm.out = a.out;
  prm.lse = a.lse;
  prm.ws_o = (float *)a.workspace;
  prm.ws_lse = sp.max_splits > 1 ? prm.ws_o + (size_t)a.batch * sp.max_splits * a.hq * 64 * a.d : nullptr;
  prm.s_page = a.s_page;
  prm.s_slot = a.s_slot;
  prm.s_head = a.s_head;
  prm.max_pages = a.max_pages;
  prm.page_shift = a.page_shift;
  prm.hq = a.hq;
  prm.group = group;
  prm.packed = a.mask_kind == MA_KIND_PACKED_U64 ? 1 : 0;
  prm.tiles_per_split = sp.tiles_per_split;
  prm.max_splits = sp.max_splits;
  prm.max_kv = a.max_kv;
  prm.scale = a.scale;
  prm.scale_log2 = a.scale * kLog2e;
  switch (a.d) {
    case 64: return run_d<64>(a, prm, sp);
    case 128: return run_d<128>(a, prm, sp);
    case 256: return run_d<256>(a, prm, sp);
  }
  return set_error(MA_ERR_UNSUPPORTED, "head_dim %d", a.d);
}

}  // namespace maskattn
