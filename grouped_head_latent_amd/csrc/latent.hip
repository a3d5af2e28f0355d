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
// All query heads read the same cache rows, so a work-group stages a tile of
// 32 tokens (36 KiB) in LDS once and lets 64 query rows (4 waves x 16) use it:
//   S^T (16 tokens x 16 rows) = C Q^T over 576 features, C from LDS, Q^T in
//   VGPRs;  O^T (512 x 16 rows) += C^T P^T, where each lane reads an 8-token x
//   8-feature block of the same LDS tile and transposes it in registers, and
//   the score tiles' token order makes the score accumulator the P^T operand.
// Work-groups that cover other query rows of the same (sequence, split) get
// neighbouring logical ids and are placed on the same XCD, so their second
// read of the tile comes from that XCD's L2.
#include "device_common.hpp"
#include "kernels.hpp"

namespace gha {
namespace {

constexpr int RKV = 512, DR = 64, DL = RKV + DR;  // 576
constexpr int TKEYS = 32;                          // tokens per tile
constexpr int LP = DL + 8;                         // LDS row pitch (elements), 16 B pad
constexpr int CHUNKS = TKEYS * DL / 8;             // 16-byte chunks per tile
constexpr int LOADS = CHUNKS / 256;                // per thread
static_assert(CHUNKS % 256 == 0 && TKEYS * 8 == 256 && LOADS == 9 && RKV == 64 * (LOADS - 1) && DR == 64,
              "tile staging: 8 threads per token row, 8 latent chunks + 1 RoPE chunk each");

__global__ __launch_bounds__(256, 1) void latent_split_kernel(LatentArgs a) {
  constexpr int DS = DL / 32;  // 18 score MFMA steps
  __shared__ __attribute__((aligned(16))) __bf16 smem[2][TKEYS * LP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;

  const uint32_t lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const int n_units = a.B * a.n_splits * a.n_rb;
  if (lid >= (uint32_t)n_units) return;
  const int rb = lid % a.n_rb;
  const int split = (lid / a.n_rb) % a.n_splits;
  const int b = lid / (a.n_rb * a.n_splits);
  const int L = a.seqlens[b];
  const int start = split * a.split_len;
  if (start >= L) return;
  const int end = min(L, start + a.split_len);

  // this lane's query row: R = t * h_q + head
  const int R = rb * 64 + wave * 16 + li;
  const int n_rows = a.s_q * a.h_q;
  const bool row_ok = R < n_rows;
  const int tq = R / a.h_q, head = R % a.h_q;
  const int kvis = L - a.s_q + tq;

  u32x4 qf[DS];
  {
    const __bf16* qp = (const __bf16*)a.q + (int64_t)b * a.q_sb + (int64_t)head * a.q_sh + (int64_t)tq * a.q_ss;
    const __bf16* qrp = (const __bf16*)a.qr + (int64_t)b * a.qr_sb + (int64_t)head * a.qr_sh + (int64_t)tq * a.qr_ss;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      if (!row_ok) qf[s] = u32x4{0u, 0u, 0u, 0u};
      else if (s < RKV / 32) qf[s] = ld16(qp + 32 * s + 8 * lg);
      else qf[s] = ld16(qrp + 32 * (s - RKV / 32) + 8 * lg);
    }
  }
  const __bf16* cbase = (const __bf16*)a.c + (int64_t)b * a.c_sb;
  const __bf16* rbase = (const __bf16*)a.kr + (int64_t)b * a.kr_sb;
  const float c2 = a.scale * kLog2e;

  // Staging: thread t owns token row t/8 of the tile and its 16-byte chunks
  // (t%8) + 8m, m = 0..8 (72 chunks per 576-wide row): one row pointer per
  // tile, the chunks at constant offsets.  Rows past `end` are clamped to the
  // last token (masked to -inf below).
  const int s_row = tid >> 3, s_chunk = tid & 7;
  u32x4 stg[LOADS];
  auto load_tile = [&](int k0) {
    const int kk = min(k0 + s_row, end - 1);
    const __bf16* cp = cbase + (int64_t)kk * a.c_ss + 8 * s_chunk;
    const __bf16* rp = rbase + (int64_t)kk * a.kr_ss + 8 * s_chunk;
#pragma unroll
    for (int m = 0; m < LOADS - 1; ++m) stg[m] = ld16(cp + 64 * m);
    stg[LOADS - 1] = ld16(rp);
  };
  auto store_tile = [&](int buf) {
    __bf16* dst = &smem[buf][s_row * LP + 8 * s_chunk];
#pragma unroll
    for (int m = 0; m < LOADS; ++m) st16(dst + 64 * m, stg[m]);
  };

  f32x4 oacc[4][8];
#pragma unroll
  for (int dg = 0; dg < 4; ++dg)
#pragma unroll
    for (int e = 0; e < 8; ++e) oacc[dg][e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m2 = kNegInf, lsum = 0.f;

  const int n_t = (end - start + TKEYS - 1) / TKEYS;
  load_tile(start);
  store_tile(0);
  wait_vmem_all();
  __syncthreads();

  for (int it = 0; it < n_t; ++it) {
    const int buf = it & 1;
    const int k0 = start + it * TKEYS;
    if (it + 1 < n_t) load_tile(k0 + TKEYS);
    const __bf16* ts = smem[buf];

    // S^T: score tile t row i <-> token k0 + 8*(i/4) + 4*t + i%4
    f32x4 sacc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      const __bf16* rowp = ts + (8 * (li >> 2) + 4 * t + (li & 3)) * LP + 8 * lg;
#pragma unroll
      for (int s = 0; s < DS; ++s) sacc[t] = mfma_bf16(ld16(rowp + 32 * s), qf[s], sacc[t]);
    }
    // lane group lg, tile t, element r <-> token k0 + 8*lg + 4*t + r
    float mx = kNegInf;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + 8 * lg + 4 * t + r;
        if (key >= end || key > kvis) sacc[t][r] = kNegInf;
        mx = fmaxf(mx, sacc[t][r]);
      }
    const float mx2 = group4_max(mx) * c2;
    if (wave_any(mx2 > m2 + kRescaleSlack)) {
      const float mnew = fmaxf(m2, mx2);
      const float alpha = (mnew == kNegInf) ? 1.f : fast_exp2(m2 - mnew);
      m2 = mnew;
      lsum *= alpha;
#pragma unroll
      for (int dg = 0; dg < 4; ++dg)
#pragma unroll
        for (int e = 0; e < 8; ++e) oacc[dg][e] *= alpha;
    }
    const float msub = (m2 == kNegInf) ? 0.f : m2;
    float p[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) p[t][r] = fast_exp2(__builtin_fmaf(sacc[t][r], c2, -msub));
    const u32x4 pf = {pack_bf16(p[0][0], p[0][1]), pack_bf16(p[0][2], p[0][3]),
                      pack_bf16(p[1][0], p[1][1]), pack_bf16(p[1][2], p[1][3])};
    lsum += bf16x8_sum(pf);

    // O^T += C^T P^T: lane reads tokens 8*lg .. 8*lg+7, features 128*dg + 8*li .. +7
#pragma unroll
    for (int dg = 0; dg < 4; ++dg) {
      u32x4 vr[8];
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) vr[tt] = ld16(ts + (8 * lg + tt) * LP + 128 * dg + 8 * li);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const u32x4 alo = {lo_pair(vr[0][w], vr[1][w]), lo_pair(vr[2][w], vr[3][w]),
                           lo_pair(vr[4][w], vr[5][w]), lo_pair(vr[6][w], vr[7][w])};
        const u32x4 ahi = {hi_pair(vr[0][w], vr[1][w]), hi_pair(vr[2][w], vr[3][w]),
                           hi_pair(vr[4][w], vr[5][w]), hi_pair(vr[6][w], vr[7][w])};
        oacc[dg][2 * w] = mfma_bf16(alo, pf, oacc[dg][2 * w]);
        oacc[dg][2 * w + 1] = mfma_bf16(ahi, pf, oacc[dg][2 * w + 1]);
      }
    }

    if (it + 1 < n_t) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- partial of this split: normalised output and log2-sum-exp ---------
  const float lfull = group4_sum(lsum);
  if (!row_ok) return;
  const float inv = lfull > 0.f ? 1.f / lfull : 0.f;
  const int64_t pidx = (((int64_t)b * a.n_rb + rb) * a.n_splits + split) * 64 + wave * 16 + li;
  float* wo = a.ws_o + pidx * RKV;
  // oacc[dg][e][r] is feature 128*dg + 8*(4*lg + r) + e
#pragma unroll
  for (int dg = 0; dg < 4; ++dg)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int f = 128 * dg + 8 * (4 * lg + r);
      *reinterpret_cast<f32x4*>(wo + f) =
          f32x4{oacc[dg][0][r], oacc[dg][1][r], oacc[dg][2][r], oacc[dg][3][r]} * inv;
      *reinterpret_cast<f32x4*>(wo + f + 4) =
          f32x4{oacc[dg][4][r], oacc[dg][5][r], oacc[dg][6][r], oacc[dg][7][r]} * inv;
    }
  if (lg == 0) a.ws_lse[pidx] = lfull > 0.f ? m2 + fast_log2(lfull) : kNegInf;
}

// Merge the splits of 4 query rows per work-group (64 threads per row, 8
// features per thread): each split s holds its normalised output O_s and its
// log2-sum-exp l_s; the result is sum_s 2^(l_s - M) O_s / sum_s 2^(l_s - M).
template <bool OUT_F32>
__global__ __launch_bounds__(256) void latent_merge_kernel(LatentArgs a) {
  const int unit = blockIdx.x / 16;  // b * n_rb + rb
  const int rb = unit % a.n_rb, b = unit / a.n_rb;
  const int tid = threadIdx.x;
  const int row = (blockIdx.x % 16) * 4 + (tid >> 6);
  const int f = (tid & 63) * 8;
  const int R = rb * 64 + row;
  if (R >= a.s_q * a.h_q) return;
  const int L = a.seqlens[b];
  // lengths above the plan's bound are a precondition violation; never read
  // partials the plan did not allot
  const int ns = min((L + a.split_len - 1) / a.split_len, a.n_splits);
  const int64_t base = (int64_t)unit * a.n_splits * 64 + row;
  float M = kNegInf;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, a.ws_lse[base + (int64_t)s * 64]);
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float ls = a.ws_lse[base + (int64_t)s * 64];
    const float w = (ls == kNegInf) ? 0.f : fast_exp2(ls - M);
    den += w;
    const float* src = a.ws_o + (base + (int64_t)s * 64) * RKV + f;
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

hipError_t launch_latent_decode(const LatentArgs& a, bool out_f32, hipStream_t st) {
  const int n_units = a.B * a.n_splits * a.n_rb;
  const int padded = (n_units + 7) / 8 * 8;
  hipLaunchKernelGGL(latent_split_kernel, dim3(padded), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (out_f32)
    hipLaunchKernelGGL(latent_merge_kernel<true>, dim3(a.B * a.n_rb * 16), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(latent_merge_kernel<false>, dim3(a.B * a.n_rb * 16), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace gha
