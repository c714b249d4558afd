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

}  // namespace dev
}  // namespace maskattn
