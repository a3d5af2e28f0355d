// Building blocks of the kernels that stream K/V or latent tiles from HBM
// straight into LDS and feed MFMAs from there (gfx950).
#pragma once
#include <type_traits>

#include "device_common.hpp"

namespace gha {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Buffer resource word 3 for raw (unswizzled, untyped) dword access.
constexpr int kBufferFlags = 0x00020000;
// A buffer offset past any range the kernels build: such loads read zeros.
constexpr uint32_t kOutOfRange = 0x80000000u;

// f(integral_constant<int, I>) for I = B .. E - 1, unrolled at compile time
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// 16 bytes per lane from buffer `rs` at voff + soff into LDS at lds + 16 lane
// (buffer_load_dwordx4 ... lds); bytes past the buffer's range come back as
// zeros.  Inline asm so that the compiler sees no LDS write it would have to
// order every LDS read after (with the builtin it waits for every outstanding
// tile load before each LDS read, which serialises the prefetch); the kernels
// order these loads themselves (vmcnt wait + barrier).  The instruction has no
// destination register; M0 needs one wait state after it is written.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(rs), "s"(soff) : "memory", "m0");
}
// The same load marked non-temporal, for data that one work-group reads once
// (a decode step's cache): it streams past the caches, and a stream of such
// loads reads HBM faster (a read probe of 4 GiB on MI355X: about 7.1 TB/s
// against 6.3 with the default policy).  Data that other work-groups read
// again through L2 (prefill tiles, a key part shared by groups) keeps the
// default policy.
__device__ __forceinline__ void lds_dma16_nt(__amdgpu_buffer_rsrc_t rs, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
               :: "s"(lds), "v"(voff), "s"(rs), "s"(soff) : "memory", "m0");
}
#ifndef GHA_DECODE_NT
#define GHA_DECODE_NT 1  // decode caches streamed with non-temporal loads
#endif
// a decode cache tile: non-temporal unless switched off
__device__ __forceinline__ void lds_dma16_stream(__amdgpu_buffer_rsrc_t rs, uint32_t lds, uint32_t voff, uint32_t soff) {
  if constexpr (GHA_DECODE_NT != 0) lds_dma16_nt(rs, lds, voff, soff);
  else lds_dma16(rs, lds, voff, soff);
}
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// ds_read_b64_tr_b16: within each 16-lane group, destination lane d receives
// as element j the element d % 4 of the 8 bytes that source lane 4 j + d / 4
// points at (a 4 x 4 transpose of 16-bit elements per lane quad).
__device__ __forceinline__ u32x2 ld_tr(const unsigned char* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p));
}

// ds_read_b64_tr_b8: within each 16-lane group, destination lane t receives
// as byte j the byte t % 8 of the 8 bytes that source lane 2 j + t / 8
// points at (the layout an LDS probe of the instruction showed).
typedef int i32x2_lds __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_lds lds_i32x2;
__device__ __forceinline__ u32x2 ld_tr8(const unsigned char* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)p));
}

// s_waitcnt with only the vector-memory counter limited to N (N < 64)
template <int N>
__device__ __forceinline__ void wait_vmem_at_most() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// MFMAs written as inline asm to pin register classes: output accumulators
// in AGPRs (mfma_acc), scores, normalisers and every operand in VGPRs.  Left
// to itself the compiler puts every MFMA result, scores included, in AGPRs
// and spills.  The asm is volatile so that the MFMAs keep their program order.
// The compiler does not see these as MFMAs, so the kernels pad the two hazards
// it would otherwise cover: VALU writes of an operand need two wait states
// before an MFMA reads it, and an MFMA result needs more than eight before a
// VALU reads it.  MFMA to MFMA accumulator chains need none.
__device__ __forceinline__ void mfma_acc(f32x4& acc, const u32x4& a, const u32x4& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v(f32x4& acc, const u32x4& a, const u32x4& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v0(f32x4& acc, const u32x4& a, const u32x4& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "v"(b));
}

}  // namespace gha
