// Device helpers shared by the gfx950 attention kernels.
//
// Matrix-core layout used throughout (v_mfma_f32_32x32x16_bf16 and
// v_mfma_f32_32x32x2_f32, wave64):
//   A (32 x K):  lane l holds row l % 32, K-slots of half l / 32
//   B (K x 32):  lane l holds column l % 32, the same K-slots
//   C (32 x 32): lane l holds column l % 32; accumulator register r holds
//                row 8 * (r / 4) + 4 * (l / 32) + r % 4
// The kernels compute S^T = K Q^T and O^T = V^T P^T, so a lane's C column is
// one query row: the row max and row sum of the online softmax stay inside a
// lane (plus one exchange with lane l ^ 32), and P leaves the S accumulator
// already in B-operand form for the P.V product, with the key order of the
// V^T operand permuted to match.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace maskattn {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float lane_swap32(float x) { return __shfl_xor(x, 32, 64); }

// bf16 <-> raw bits
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round-to-nearest-even fp32 -> bf16 via the native converter.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  f32x2 v = {lo, hi};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// Byte permute of two dwords (v_perm_b32): result byte i = byte sel_i of
// {hi:lo} where bytes 0-3 are `lo` and 4-7 are `hi`.
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

// Q rows as B operands: lane l holds Q[row][16 s + 8 (l / 32) .. + 7].
template <int D>
__device__ __forceinline__ void load_q(bf16x8 (&qf)[D / 16], const uint16_t *qrow, bool ok, int hi) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const u32x4 raw = ok ? *(const u32x4 *)(qrow + 16 * s + 8 * hi) : u32x4{0, 0, 0, 0};
    qf[s] = __builtin_bit_cast(bf16x8, raw);
  }
}

__device__ __forceinline__ uint64_t low_bits(int n) {  // n in [0, 64]
  return n >= 64 ? ~0ull : (n <= 0 ? 0ull : ((1ull << n) - 1ull));
}

// Masks the two 32-key score blocks of a lane with its row's tile word.
// Score (kb, r) of lane l is key 32 kb + 8 (r / 4) + 4 (l / 32) + r % 4.
__device__ __forceinline__ void apply_word(f32x16 (&s)[2], uint64_t word, int hi) {
  const uint64_t ws = word >> (4 * hi);
  const uint32_t w0 = (uint32_t)ws, w1 = (uint32_t)(ws >> 32);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int bit = 8 * (r >> 2) + (r & 3);
    if (!((w0 >> bit) & 1u)) s[0][r] = neg_inf();
    if (!((w1 >> bit) & 1u)) s[1][r] = neg_inf();
  }
}

// acc + the sum of the 8 bf16 values of x (v_dot2_f32_bf16 against (1, 1),
// fp32 accumulation).
__device__ __forceinline__ float row_sum_bf16(const bf16x8 &x, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = __builtin_bit_cast(bf16x2, 0x3F803F80u);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 pr = {x[2 * i], x[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
  }
  return acc;
}

// Both 32-lane halves of a wave hold the same 32 query rows (other keys):
// combine a per-lane value with its partner lane l ^ 32.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Online softmax in the log2 domain with a lazily raised reference.
// m_ref (scaled by scale * log2 e) only moves when a tile's row max exceeds
// it by more than kRescaleSlack; until then probabilities are exp2(s c -
// m_ref) <= 2^kRescaleSlack and the accumulators keep their scale.  The
// result is unchanged (O and its normaliser share the reference), and most
// tiles skip the rescale.  Returns true when some row of the wave changed
// its reference; alpha is then that row's rescale factor (1 for the others).
constexpr float kRescaleSlack = 8.f;

__device__ __forceinline__ bool softmax_tile(f32x16 (&s)[2], float &m_ref, float c, float &alpha) {
  float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
  for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
  const float mxc = max_halves(mx) * c;
  const bool raise = mxc > m_ref + kRescaleSlack;
  // selects, not a branch: the kernels schedule matrix products across this
  const float a = fast_exp2(m_ref - mxc);   // 0 when m_ref is still -inf
  alpha = raise ? a : 1.f;
  m_ref = raise ? mxc : m_ref;
  const bool any = __builtin_amdgcn_ballot_w64(raise) != 0ull;
  const float mu = m_ref == neg_inf() ? 0.f : m_ref;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = fast_exp2(__builtin_fmaf(s[kb][r], c, -mu));
  return any;
}

template <typename OutT>
__device__ __forceinline__ void store4(OutT *dst, float a, float b, float c, float d);

template <>
__device__ __forceinline__ void store4<float>(float *dst, float a, float b, float c, float d) {
  *(f32x4 *)dst = f32x4{a, b, c, d};
}

template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t *dst, float a, float b, float c, float d) {
  *(u32x2 *)dst = u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}

// Writes a lane's normalised output row slice (O^T register layout: register
// r of block n is head-dim 32 n + 8 (r / 4) + 4 (l / 32) + r % 4).
template <int D, typename OutT>
__device__ __forceinline__ void store_row(OutT *dst, const f32x16 (&o)[D / 32], float inv, int hi) {
#pragma unroll
  for (int n = 0; n < D / 32; ++n)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d0 = 32 * n + 8 * r4 + 4 * hi;
      store4<OutT>(dst + d0, o[n][4 * r4] * inv, o[n][4 * r4 + 1] * inv, o[n][4 * r4 + 2] * inv,
                   o[n][4 * r4 + 3] * inv);
    }
}

}  // namespace dev
}  // namespace maskattn
