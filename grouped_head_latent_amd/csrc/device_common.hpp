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
// that hold one MFMA column), with gfx950's permlane swaps.
// v_permlane16_swap a, b exchanges the odd 16-lane rows of a with the even
// rows of b; applied to two copies of x it leaves, per lane, x in one
// register and x of lane l^16 in the other (v_permlane32_swap likewise for
// l^32), so the max or sum of the two registers is the pair reduction.
// Written as inline asm because the compiler builtin exposes only the first
// of the two results; the s_nop pads cover the VALU-write-to-permlane
// hazard, since the hazard checker does not look inside inline asm.
__device__ __forceinline__ void permlane16_swap(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void permlane32_swap(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float xor16_max(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  permlane16_swap(a, b);
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float xor32_max(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  permlane32_swap(a, b);
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float xor16_sum(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  permlane16_swap(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}
__device__ __forceinline__ float xor32_sum(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  permlane32_swap(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}
__device__ __forceinline__ float group4_max(float x) { return xor32_max(xor16_max(x)); }

// Maxima of finite or infinite floats as single instructions.  Written as
// inline asm because fmaxf on values the compiler cannot prove canonical
// (MFMA results, asm outputs) costs an extra v_max per operand in IEEE mode;
// neither helper is meant for NaN inputs.  Volatile, so that a maximum
// woven between MFMAs stays where it is written: moved to its use, it would
// keep the raw scores it reads alive beside the probabilities made from them.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm volatile("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max2f(float a, float b) {
  float r;
  asm volatile("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float group4_sum(float x) { return xor32_sum(xor16_sum(x)); }

// An MFMA A operand of all-ones bf16: multiplying it into P^T sums P over the
// contraction (key) axis in every output row, i.e. the softmax normaliser of
// exactly the bf16 probabilities that the P.V product consumes.
constexpr uint32_t kBf16OnePair = 0x3F803F80u;

// Interleave the low (or high) bf16 halves of two words: result = (a.x, b.x).
__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Wait until every vector-memory load issued so far has landed (vmcnt = 0,
// other counters untouched).  Kernels call it once after loading their
// resident query fragments: otherwise the first MFMA of the main loop waits
// on vmcnt(0) every iteration, i.e. on the prefetch of the next tile too.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Inclusive prefix sum over the lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d *= 2) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

// True in every lane if any lane's predicate holds (wave-uniform branch).
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Online softmax with a lazily updated running maximum.  Scores are kept in
// log2 units (score * scale * log2 e).  The running maximum m only moves when
// a tile's maximum exceeds it by more than kRescaleSlack, so most tiles skip
// rescaling the output accumulator; probabilities are then at most
// 2^kRescaleSlack, far inside fp32 and bf16 range.  The result is the same
// softmax: numerator and normaliser share whatever m was used.
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// a 16-byte global load marked non-temporal (data read once: it need not stay in L2)
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

// Work-group id remapped so that consecutive logical ids run on the same
// XCD: the dispatcher deals work-groups round-robin over the 8 XCDs, each with
// its own L2, so logical neighbours (which share K/V or latent tiles) should
// sit on one XCD.  `padded` is the grid size, a multiple of 8.
__device__ __forceinline__ uint32_t xcd_logical_id(uint32_t bid, uint32_t padded) {
  return (bid & 7u) * (padded >> 3) + (bid >> 3);
}

}  // namespace gha
