// Absorbed latent decode (MLA / GQLA MQA-absorb path), bf16, split-KV with a
// log-sum-exp merge.
//
// "GQLA: Group-Query Latent Attention ...", section 1 and Figure 2 (right):
// with W^UK folded into the query and W^UV into the output, every query head
// attends directly over the cached latent.  Each cached token is one row of
// r_kv + d_r = 576 bf16 (the latent c^KV followed by the shared RoPE key k^R).
// For head i and token u the score is q_lat_i . c_u + q_rope_i . k^R_u (a
// 576-long dot product) and the value is c_u (the first 512 features).
//
// One work-group takes 128 query rows (all heads of one token at s_q = 1),
// one wave per SIMD and 32 rows per wave, and walks a split of the cache in
// tiles of 64 tokens.  Every tile goes from HBM straight into LDS (buffer
// DMA, no VGPR staging) once and serves all 128 rows:
//   S^T (tokens x rows) = C Q^T over 576 features: K-side fragments are 16 B
//   LDS reads, Q^T (32 rows x 576) stays in VGPRs;
//   O^T (512 x rows) += C^T P^T: C^T fragments come from transposing LDS
//   reads (ds_read_b64_tr_b16) and the score accumulator is P^T.
// The O^T accumulator (512 x 32 fp32 per wave) lives in AGPRs.
//
// LDS tile layout, unit-major: the 72 units (8 features, 16 B) of the 64
// tokens; unit u of token k sits at byte 1024 u + 16 (k ^ 8 (u & 1)).  One
// DMA instruction fills one unit of all 64 tokens (lane = slot).  The XOR of
// odd units makes the transposing reads, which touch units 2 dt and 2 dt + 1
// of 8 tokens per half-wave, land in distinct banks; score reads touch 16
// consecutive tokens of one unit.
#include "device_common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace gha {
namespace {

constexpr int RKV = 512, DR = 64, DL = RKV + DR;  // 576
constexpr int T = 32;                             // tokens per tile
constexpr int NU = DL / 8;                        // 72 units per token
constexpr int NUC = RKV / 8;                      // 64 latent units; the rest are RoPE units
constexpr int UNITB = T * 16;                     // 512 bytes: one unit of every token
constexpr int TILEB = NU * UNITB;                 // 36 KiB
constexpr int ROWS = 128;                         // query rows per work-group
constexpr int DS = DL / 32;                       // 18 score contraction steps
constexpr int DT = RKV / 16;                      // 32 output column tiles
constexpr int kBufferFlags = 0x00020000;          // raw dword buffer access
constexpr float kLatentSlack = 96.f;              // see the running state below

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// 16 bytes per lane from buffer `rs` at voff + soff into LDS at lds + 16 lane;
// bytes past the buffer's range come back as zeros.  Inline asm so that the
// compiler sees no LDS write it would have to order every LDS read after;
// the kernel orders these loads itself (vmcnt wait + barrier).  M0 needs one
// wait state after it is written.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(rs), "s"(soff) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// The MFMAs are written as inline asm to pin register classes: the O^T
// accumulator (512 x 32 fp32 per wave) in AGPRs, the scores, the normaliser
// and every operand in VGPRs.  Left to itself the compiler puts every MFMA
// result, scores included, in AGPRs and spills.  The asm is volatile so that
// the MFMAs keep their program order.  The compiler does not see these as
// MFMAs, so the kernel pads the two hazards it would otherwise cover: VALU
// writes of an operand need two wait states before an MFMA reads it, and an
// MFMA result needs more than eight before a VALU reads it.  MFMA to MFMA
// accumulator chains need none.
__device__ __forceinline__ void mfma_acc(f32x4& acc, const u32x4& a, const u32x4& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v(f32x4& acc, const u32x4& a, const u32x4& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v0(f32x4& acc, const u32x4& a, const u32x4& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ u32x2 ld_tr(const unsigned char* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p));
}

__global__ __launch_bounds__(256, 1) void latent_split_kernel(LatentArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * TILEB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;

  const uint32_t lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const int n_units = a.B * a.n_splits * a.n_rb;
  if (lid >= (uint32_t)n_units) return;
  // work-group-uniform indices, kept in scalar registers
  const int rb = __builtin_amdgcn_readfirstlane(lid % a.n_rb);
  const int split = __builtin_amdgcn_readfirstlane((lid / a.n_rb) % a.n_splits);
  const int b = __builtin_amdgcn_readfirstlane(lid / (a.n_rb * a.n_splits));
  const int L = __builtin_amdgcn_readfirstlane(a.seqlens[b]);
  const int start = split * a.split_len;
  if (start >= L) return;
  const int end = min(L, start + a.split_len);

  // ---- this lane's two query rows (q-tiles): R = t * h_q + head ------------
  const int n_rows = a.s_q * a.h_q;
  int kvis[2];
  bool row_ok[2];
  u32x4 qf[2][DS];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int R = rb * ROWS + 32 * wave + 16 * qt + li;
    row_ok[qt] = R < n_rows;
    const int tq = R / a.h_q, head = R % a.h_q;
    kvis[qt] = L - a.s_q + tq;  // last visible token (bottom-right causal)
    const __bf16* qp = (const __bf16*)a.q + (int64_t)b * a.q_sb + (int64_t)head * a.q_sh + (int64_t)tq * a.q_ss;
    const __bf16* qrp = (const __bf16*)a.qr + (int64_t)b * a.qr_sb + (int64_t)head * a.qr_sh + (int64_t)tq * a.qr_ss;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      if (!row_ok[qt]) qf[qt][s] = u32x4{0u, 0u, 0u, 0u};
      else if (s < RKV / 32) qf[qt][s] = ld16(qp + 32 * s + 8 * lg);
      else qf[qt][s] = ld16(qrp + 32 * (s - RKV / 32) + 8 * lg);
    }
  }
  wait_vmem_all();
  const float c2 = a.scale * kLog2e;

  // ---- tile loads ------------------------------------------------------------
  // One DMA instruction (64 lanes x 16 B) fills two units of 32 tokens:
  // lane l writes slot l % 32 of unit u0 + l / 32 (u0 even), i.e. token
  // (l % 32) ^ 8 (l / 32).  Wave w fills latent units 16 w .. 16 w + 15 and
  // RoPE units 64 + 2 w, 65 + 2 w.  Rows at or past the sequence end read as
  // zeros (range check).
  const uint32_t c_row = (uint32_t)a.c_ss * 2u, r_row = (uint32_t)a.kr_ss * 2u;
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const __bf16*)a.c + (int64_t)b * a.c_sb), 0, (int)((uint32_t)(L - 1) * c_row + 2u * RKV), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const __bf16*)a.kr + (int64_t)b * a.kr_sb), 0, (int)((uint32_t)(L - 1) * r_row + 2u * DR), kBufferFlags);
  static_assert(T == 32 && UNITB == 512, "a DMA instruction covers two units");
  const int dma_tok = (lane & 31) ^ (8 * (lane >> 5)), dma_u = lane >> 5;
  const uint32_t c_off = (uint32_t)dma_tok * c_row + 16u * dma_u;
  const uint32_t r_off = (uint32_t)dma_tok * r_row + 16u * dma_u;
  const uint32_t lds0 = lds_offset(smem);
  auto issue_tile = [&](int k0, int buf) __attribute__((always_inline)) {
    const uint32_t dst = lds0 + buf * TILEB;
    const uint32_t cs = (uint32_t)k0 * c_row + 16u * (16 * wave), rsft = (uint32_t)k0 * r_row + 16u * (2 * wave);
#pragma unroll
    for (int j = 0; j < 8; ++j) lds_dma16(crs, dst + (16 * wave + 2 * j) * UNITB, c_off, cs + 32u * j);
    lds_dma16(rrs, dst + (NUC + 2 * wave) * UNITB, r_off, rsft);
  };

  // ---- fragment addresses (bytes within a tile) -----------------------------
  // score A operand: token 16 kt + li, unit 4 s + lg (parity lg & 1)
  const uint32_t sfrag = lg * UNITB + ((li ^ (8 * (lg & 1))) * 16);
  // value A operand (transposing read), source lane li of group lg: token
  // 32 k2 + 16 h + 4 lg + li / 4, unit 2 dt + b with b = (li / 2) % 2, byte
  // 8 (li % 2) of it
  const int vb = (li >> 1) & 1;
  const uint32_t vfrag = vb * UNITB + (((4 * lg + (li >> 2)) ^ (8 * vb)) * 16) + 8 * (li & 1);

  // ---- running state -----------------------------------------------------------
  // Scores are taken against a per-row reference m2 (log2 units) fixed by
  // the first visible tile: probabilities 2^(s - m2) up to 2^kLatentSlack stay
  // far inside bf16 and fp32 range, so the accumulators never need
  // rescaling (they live in AGPRs, where rescaling would be costly).  A tile
  // whose maximum exceeds m2 + kLatentSlack restarts the split with the new
  // maximum as reference; the result is the same softmax either way.
  f32x4 oacc[DT][2], lacc[2];
  float m2[2] = {kNegInf, kNegInf};
  __shared__ int restart_flag[2][4];
  const u32x4 ones = {kBf16OnePair, kBf16OnePair, kBf16OnePair, kBf16OnePair};

  const int n_t = (end - start + T - 1) / T;

  // Tiles wholly before `end` and before every row's causal limit need no
  // mask; only the last one or two may.
  int t_mask = (end - start) / T;
  {
    int lim = L - a.s_q;  // smallest last-visible token over the rows (tq = 0)
    t_mask = min(t_mask, max(0, (lim + 1 - start) / T));
  }

  auto tile = [&](int it, auto masked) __attribute__((always_inline)) -> bool {
    constexpr bool kMasked = decltype(masked)::value;
    const int buf = it & 1;
    const int k0 = start + it * T;
    if (it + 1 < n_t) issue_tile(k0 + T, buf ^ 1);
    const unsigned char* ts = smem + buf * TILEB;

    // S^T tiles: token tile kt (16 tokens) x q-tile qt, one contraction step
    // (32 features) per scheduling region, K fragments read one step ahead
    f32x4 sacc[2][2];
    u32x4 kf[2][2];
    auto load_k = [&](int s, u32x4 (&f)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) f[kt] = ld16(ts + sfrag + (4 * s) * UNITB + 256 * kt);
    };
    load_k(0, kf[0]);
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      if (s + 1 < DS) load_k(s + 1, kf[(s + 1) & 1]);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          if (s == 0) mfma_v0(sacc[kt][qt], kf[s & 1][kt], qf[qt][s]);
          else mfma_v(sacc[kt][qt], kf[s & 1][kt], qf[qt][s]);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
    // scores retire before the softmax reads them
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(sacc[0][0]), "+v"(sacc[0][1]), "+v"(sacc[1][0]), "+v"(sacc[1][1]));

    // softmax per row (= per lane and q-tile) against a fixed reference;
    // sacc[kt][qt][r] is token k0 + 16 kt + 4 lg + r
    u32x4 pf[2];
    bool restart_row = false;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      if (kMasked) {
        const int kmax = min(end - 1, kvis[qt]);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (k0 + 16 * kt + 4 * lg + r > kmax) sacc[kt][qt][r] = kNegInf;
      }
      float mx = fmaxf(fmaxf(sacc[0][qt][0], sacc[0][qt][1]), sacc[0][qt][2]);
      mx = fmaxf(fmaxf(mx, sacc[0][qt][3]), sacc[1][qt][0]);
      mx = fmaxf(fmaxf(mx, sacc[1][qt][1]), sacc[1][qt][2]);
      mx = fmaxf(mx, sacc[1][qt][3]);
      const float mx2 = group4_max(mx) * c2;
      if (m2[qt] == kNegInf) {
        m2[qt] = mx2;  // first visible scores of this row: nothing accumulated yet
      } else if (mx2 > m2[qt] + kLatentSlack) {
        m2[qt] = mx2;
        restart_row = true;
      }
      const float msub = (m2[qt] == kNegInf) ? 0.f : m2[qt];
      float p[2][4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) p[kt][r] = fast_exp2(__builtin_fmaf(sacc[kt][qt][r], c2, -msub));
      pf[qt] = u32x4{pack_bf16(p[0][0], p[0][1]), pack_bf16(p[0][2], p[0][3]), pack_bf16(p[1][0], p[1][1]),
                     pack_bf16(p[1][2], p[1][3])};
    }

    // O^T += C^T P^T (accumulators in AGPRs) and the normaliser += 1^T P^T,
    // four column tiles per scheduling region, C^T fragments read one region
    // ahead.  Two wait states between the VALU writes of P^T (and of any
    // rescaled accumulator) and the first MFMA that reads them.
    asm volatile("s_nop 1" : "+v"(pf[0]), "+v"(pf[1]));
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) mfma_v(lacc[qt], ones, pf[qt]);
    u32x4 vf[2][4];
    auto load_v = [&](int j, u32x4 (&f)[4]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const unsigned char* vp = ts + vfrag + (2 * (4 * j + i)) * UNITB;
        const u32x2 h0 = ld_tr(vp);
        const u32x2 h1 = ld_tr(vp + 256);
        f[i] = u32x4{h0[0], h0[1], h1[0], h1[1]};
      }
    };
    load_v(0, vf[0]);
#pragma unroll
    for (int j = 0; j < DT / 4; ++j) {
      if (j + 1 < DT / 4) load_v(j + 1, vf[(j + 1) & 1]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) mfma_acc(oacc[4 * j + i][qt], vf[j & 1][i], pf[qt]);
      __builtin_amdgcn_sched_barrier(0);
    }

    // a wave whose rows outgrew their reference asks the whole work-group
    // to start the split again (every wave must run the same tiles and
    // barriers)
    if (lane == 0) restart_flag[it & 1][wave] = wave_any(restart_row) ? 1 : 0;
    wait_vmem_all();
    __syncthreads();
    const int* f = restart_flag[it & 1];
    return (f[0] | f[1] | f[2] | f[3]) != 0;
  };
  for (;;) {
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      lacc[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    issue_tile(start, 0);
    wait_vmem_all();
    __syncthreads();
    bool restart = false;
    int it = 0;
    for (; it < t_mask && !restart; ++it) restart = tile(it, std::false_type{});
    for (; it < n_t && !restart; ++it) restart = tile(it, std::true_type{});
    if (!restart) break;
  }

  // ---- partial of this split: normalised output and log2-sum-exp ---------
  // the last accumulator MFMAs must retire before the VALU reads them
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(oacc[DT - 1][0]), "+a"(oacc[DT - 1][1]), "+v"(lacc[0]), "+v"(lacc[1]));
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float l = lacc[qt][0];
    if (!row_ok[qt]) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t pidx = (((int64_t)b * a.n_rb + rb) * a.n_splits + split) * ROWS + 32 * wave + 16 * qt + li;
    float* wo = a.ws_o + pidx * RKV;
    // oacc[dt][qt][r] is feature 16 dt + 4 lg + r
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      *reinterpret_cast<f32x4*>(wo + 16 * dt + 4 * lg) = oacc[dt][qt] * inv;
      if ((dt & 3) == 3) __builtin_amdgcn_sched_barrier(0);
    }
    if (lg == 0) a.ws_lse[pidx] = l > 0.f ? m2[qt] + fast_log2(l) : kNegInf;
  }
}

// Merge the splits of 4 query rows per work-group (64 threads per row, 8
// features per thread): each split s holds its normalised output O_s and its
// log2-sum-exp l_s; the result is sum_s 2^(l_s - M) O_s / sum_s 2^(l_s - M).
template <bool OUT_F32>
__global__ __launch_bounds__(256) void latent_merge_kernel(LatentArgs a) {
  const int unit = blockIdx.x / (ROWS / 4);  // b * n_rb + rb
  const int rb = unit % a.n_rb, b = unit / a.n_rb;
  const int tid = threadIdx.x;
  const int row = (blockIdx.x % (ROWS / 4)) * 4 + (tid >> 6);
  const int f = (tid & 63) * 8;
  const int R = rb * ROWS + row;
  if (R >= a.s_q * a.h_q) return;
  const int L = a.seqlens[b];
  // lengths above the plan's bound are a precondition violation; never read
  // partials the plan did not allot
  const int ns = min((L + a.split_len - 1) / a.split_len, a.n_splits);
  const int64_t base = (int64_t)unit * a.n_splits * ROWS + row;
  float M = kNegInf;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, a.ws_lse[base + (int64_t)s * ROWS]);
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float ls = a.ws_lse[base + (int64_t)s * ROWS];
    const float w = (ls == kNegInf) ? 0.f : fast_exp2(ls - M);
    den += w;
    const float* src = a.ws_o + (base + (int64_t)s * ROWS) * RKV + f;
    acc0 += w * *reinterpret_cast<const f32x4*>(src);
    acc1 += w * *reinterpret_cast<const f32x4*>(src + 4);
  }
  const float inv = 1.f / den;
  acc0 *= inv;
  acc1 *= inv;
  const int tq = R / a.h_q, head = R % a.h_q;
  const int64_t obase = (int64_t)b * a.o_sb + (int64_t)head * a.o_sh + (int64_t)tq * a.o_ss + f;
  if constexpr (OUT_F32) {
    *reinterpret_cast<f32x4*>((float*)a.o + obase) = acc0;
    *reinterpret_cast<f32x4*>((float*)a.o + obase + 4) = acc1;
  } else {
    *reinterpret_cast<u32x4*>((__bf16*)a.o + obase) =
        u32x4{pack_bf16(acc0[0], acc0[1]), pack_bf16(acc0[2], acc0[3]), pack_bf16(acc1[0], acc1[1]),
              pack_bf16(acc1[2], acc1[3])};
  }
  if (a.lse != nullptr && (tid & 63) == 0)
    a.lse[((int64_t)b * a.s_q + tq) * a.h_q + head] = (M + fast_log2(den)) * kLn2;
}

}  // namespace

int latent_rows_per_wg() { return ROWS; }
int latent_tile_tokens() { return T; }

hipError_t launch_latent_decode(const LatentArgs& a, bool out_f32, hipStream_t st) {
  const int n_units = a.B * a.n_splits * a.n_rb;
  const int padded = (n_units + 7) / 8 * 8;
  hipLaunchKernelGGL(latent_split_kernel, dim3(padded), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (out_f32)
    hipLaunchKernelGGL(latent_merge_kernel<true>, dim3(a.B * a.n_rb * (ROWS / 4)), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(latent_merge_kernel<false>, dim3(a.B * a.n_rb * (ROWS / 4)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace gha
