// Device-side building blocks for gfx950 (CDNA4, wave64).
//
// MFMA used throughout: v_mfma_f32_16x16x32_bf16.  One wave multiplies a
// 16x32 bf16 tile A by a 32x16 bf16 tile B into a 16x16 fp32 tile D.  Lane l
// (row/col index i = l % 16, lane group g = l / 16) supplies A[i][slots of g]
// and B[slots of g][i] as eight bf16 each, and receives D[4g + r][i], r = 0..3.
// The eight "slots" of group g are eight positions of the 32-long contraction;
// which actual contraction indices they stand for is up to the caller, as long
// as A and B agree.  The kernels use that freedom to make every operand a
// single 16-byte load or a register-resident accumulator.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gha {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ f32x4 mfma_bf16(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two floats -> packed bf16 pair (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Sum of the two bf16 values packed in one word, widened exactly to fp32.
// The softmax normaliser is summed from the same bf16-rounded probabilities
// that the P.V MFMA consumes, so that weights and normaliser agree (a row
// with one visible key returns that value exactly).
__device__ __forceinline__ float bf16_pair_sum(uint32_t w) {
  return __builtin_bit_cast(float, w << 16) + __builtin_bit_cast(float, w & 0xffff0000u);
}
__device__ __forceinline__ float bf16x8_sum(const u32x4& w) {
  return (bf16_pair_sum(w[0]) + bf16_pair_sum(w[1])) + (bf16_pair_sum(w[2]) + bf16_pair_sum(w[3]));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Max / sum over the four lanes l, l^16, l^32, l^48 (the four lane groups
// that hold one MFMA column).
__device__ __forceinline__ float group4_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float group4_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

// Interleave the low (or high) bf16 halves of two words: result = (a.x, b.x).
__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

// Work-group id remapped so that consecutive logical ids run on the same
// XCD: the dispatcher deals work-groups round-robin over the 8 XCDs, each with
// its own L2, so logical neighbours (which share K/V or latent tiles) should
// sit on one XCD.  `padded` is the grid size, a multiple of 8.
__device__ __forceinline__ uint32_t xcd_logical_id(uint32_t bid, uint32_t padded) {
  return (bid & 7u) * (padded >> 3) + (bid >> 3);
}

}  // namespace gha
