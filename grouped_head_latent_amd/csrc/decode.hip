// Grouped-query attention decode over a contiguous KV cache, bf16, split-KV
// with a log-sum-exp merge.
//
// Decode reads every cached key and value once per step ("GQLA ...", section
// 1: each generated token must read the whole cached history from off-chip
// memory), so the kernel is HBM-bound and is built around keeping loads wide
// and in flight:
//  * A work-group owns one (sequence, KV head, 16-row block, key split).  Its
//    16 MFMA rows are the group's query heads times the s_q new tokens (4 or 8
//    real rows at 4 heads per group), so each K/V byte is read from HBM once
//    and used by the whole group.
//  * K and V go straight from global memory into MFMA operand registers with
//    16-byte loads; nothing is staged in LDS.  For S^T = K Q^T each lane loads
//    8 consecutive features of one key.  For O^T = V^T P^T each lane loads
//    8 consecutive keys' 8-feature chunks (four full 256-byte rows per load
//    instruction) and transposes the 8x8 block in registers with v_perm; the
//    key order of the score tiles is chosen so that the score accumulator is,
//    without any data movement, the P^T operand matching those keys.
//  * The four waves of a work-group stride over 64-key chunks of the split
//    and combine their (max, sum, output) through LDS at the end; a second
//    kernel merges the splits with their log-sum-exp.
#include "device_common.hpp"
#include "kernels.hpp"

namespace gha {
namespace {

constexpr int CH = 64;  // keys per wave iteration

template <int D>
__global__ __launch_bounds__(256, 2) void gqa_decode_split_kernel(DecodeArgs a) {
  constexpr int DS = D / 32;       // score MFMA contraction steps
  constexpr int NCH = D / 8;       // 8-feature chunks per row (16 or 8)
  __shared__ __attribute__((aligned(16))) float s_o[4][16][D + 4];  // +4: spread rows over banks
  __shared__ float s_m[4][16];
  __shared__ float s_l[4][16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;

  const int split = blockIdx.x % a.n_splits;
  const int unit = blockIdx.x / a.n_splits;
  const int rb = unit % a.n_rb;
  const int j = (unit / a.n_rb) % a.h_kv;
  const int b = unit / (a.n_rb * a.h_kv);
  // a length outside [0, L_cap] breaks the documented precondition; clamping
  // keeps every read inside the sequence's slice of the cache
  const int L = min(max(a.seqlens[b], 0), a.L_cap);
  const int start = split * a.split_len;
  if (start >= L) return;  // the merge ignores splits past the sequence end
  const int end = min(L, start + a.split_len);

  // this lane's query row (MFMA column li): row R = head_in_group * s_q + t
  const int R = rb * 16 + li;
  const bool row_ok = R < a.rows;
  const int hh = R / a.s_q, tq = R % a.s_q;
  const int kvis = L - a.s_q + tq;  // last key this row may see

  u32x4 qf[DS];
  {
    const __bf16* qp = (const __bf16*)a.q + (int64_t)b * a.q_sb +
                       (int64_t)(j * a.group + hh) * a.q_sh + (int64_t)tq * a.q_ss;
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[s] = row_ok ? ld16(qp + 32 * s + 8 * lg) : u32x4{0u, 0u, 0u, 0u};
  }
  const __bf16* kbase = (const __bf16*)a.k + (int64_t)b * a.k_sb + (int64_t)j * a.k_sh;
  const __bf16* vbase = (const __bf16*)a.v + (int64_t)b * a.v_sb + (int64_t)j * a.v_sh;
  const float c2 = a.scale * kLog2e;

  f32x4 oacc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) oacc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m2 = kNegInf, lsum = 0.f;
  wait_vmem_all();

  // Loads are clamped to the last key of the split instead of branched on:
  // keys at or past `end` are masked to -inf below, so they get zero weight.
  // With head dim 64, lanes li >= 8 feed MFMA rows whose outputs are
  // discarded; they re-read a valid chunk.
  const int vcol = 8 * (li % NCH);
  u32x4 kf[4][DS];
  u32x4 vr[2][8];
  auto load_k = [&](int k0) {
    // score tile t, row i  <->  key k0 + 32*(t/2) + 8*(i/4) + 4*(t%2) + i%4
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int key = min(k0 + 32 * (t >> 1) + 8 * (li >> 2) + 4 * (t & 1) + (li & 3), end - 1);
#pragma unroll
      for (int s = 0; s < DS; ++s) kf[t][s] = ld16(kbase + (int64_t)key * a.k_ss + 32 * s + 8 * lg);
    }
  };
  auto load_v = [&](int k0) {
#pragma unroll
    for (int hk = 0; hk < 2; ++hk)
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const int key = min(k0 + 32 * hk + 8 * lg + tt, end - 1);
        vr[hk][tt] = ld16(vbase + (int64_t)key * a.v_ss + vcol);
      }
  };

  // Pipeline per wave: K(c) was loaded during the previous chunk's P.V;
  // V(c) is loaded while S(c) and its softmax run.
  int k0 = start + wave * CH;
  if (k0 < end) load_k(k0);
  for (; k0 < end; k0 += 4 * CH) {
    load_v(k0);

    // ---- S^T = K Q^T ------------------------------------------------------
    f32x4 sacc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < DS; ++s) sacc[t] = mfma_bf16(kf[t][s], qf[s], sacc[t]);
    }
    if (k0 + 4 * CH < end) load_k(k0 + 4 * CH);

    // lane group lg, tile t, element r  <->  key k0 + 32*(t/2) + 8*lg + 4*(t%2) + r
    float mx = kNegInf;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + 32 * (t >> 1) + 8 * lg + 4 * (t & 1) + r;
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
      for (int e = 0; e < 8; ++e) oacc[e] *= alpha;
    }
    const float msub = (m2 == kNegInf) ? 0.f : m2;
    float p[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) p[t][r] = fast_exp2(__builtin_fmaf(sacc[t][r], c2, -msub));
    u32x4 pfs[2];
#pragma unroll
    for (int hk = 0; hk < 2; ++hk)
      pfs[hk] = u32x4{pack_bf16(p[2 * hk][0], p[2 * hk][1]), pack_bf16(p[2 * hk][2], p[2 * hk][3]),
                      pack_bf16(p[2 * hk + 1][0], p[2 * hk + 1][1]),
                      pack_bf16(p[2 * hk + 1][2], p[2 * hk + 1][3])};
    lsum += bf16x8_sum(pfs[0]) + bf16x8_sum(pfs[1]);

    // ---- O^T += V^T P^T ---------------------------------------------------
#pragma unroll
    for (int hk = 0; hk < 2; ++hk) {
      const u32x4 pf = pfs[hk];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // features 8*li + 2w (low halves) and 8*li + 2w + 1 (high halves)
        const u32x4 alo = {lo_pair(vr[hk][0][w], vr[hk][1][w]), lo_pair(vr[hk][2][w], vr[hk][3][w]),
                           lo_pair(vr[hk][4][w], vr[hk][5][w]), lo_pair(vr[hk][6][w], vr[hk][7][w])};
        const u32x4 ahi = {hi_pair(vr[hk][0][w], vr[hk][1][w]), hi_pair(vr[hk][2][w], vr[hk][3][w]),
                           hi_pair(vr[hk][4][w], vr[hk][5][w]), hi_pair(vr[hk][6][w], vr[hk][7][w])};
        oacc[2 * w] = mfma_bf16(alo, pf, oacc[2 * w]);
        oacc[2 * w + 1] = mfma_bf16(ahi, pf, oacc[2 * w + 1]);
      }
    }
  }

  // ---- combine the four waves -------------------------------------------
  // oacc[e][r] of lane (li, lg) is feature 8*(4*lg + r) + e of query row li.
  const float lfull = group4_sum(lsum);
  if (lg == 0) {
    s_m[wave][li] = m2;
    s_l[wave][li] = lfull;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int f0 = 8 * (4 * lg + r);
    if (f0 < D) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_o[wave][li][f0 + e] = oacc[e][r];
    }
  }
  __syncthreads();
  constexpr int TPR = 16;           // threads per row
  constexpr int FPT = D / TPR;      // features per thread
  const int row = tid / TPR, f0 = (tid % TPR) * FPT;
  const int Rw = rb * 16 + row;
  if (Rw >= a.rows) return;
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][row]);
  float wt[4], Lsum = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    wt[w] = (s_m[w][row] == kNegInf) ? 0.f : fast_exp2(s_m[w][row] - M);
    Lsum += wt[w] * s_l[w][row];
  }
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
  const int64_t pidx = ((int64_t)unit * a.n_splits + split) * 16 + row;
  float* wo = a.ws_o + pidx * D + f0;
#pragma unroll
  for (int f = 0; f < FPT; f += 4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(&s_o[w][row][f0 + f]);
      acc += wt[w] * x;
    }
    *reinterpret_cast<f32x4*>(wo + f) = acc * inv;
  }
  if (tid % TPR == 0) a.ws_lse[pidx] = (Lsum > 0.f) ? M + fast_log2(Lsum) : kNegInf;
}

// Merge the splits of one (sequence, KV head, row block): each split s holds
// its normalised output O_s and log2-sum-exp l_s over its keys; the full
// result is sum_s 2^(l_s - M) O_s / sum_s 2^(l_s - M) with M = max_s l_s.
template <int D, bool OUT_F32>
__global__ __launch_bounds__(256) void gqa_decode_merge_kernel(DecodeArgs a) {
  constexpr int TPR = 16, FPT = D / TPR;
  const int unit = blockIdx.x;
  const int rb = unit % a.n_rb;
  const int j = (unit / a.n_rb) % a.h_kv;
  const int b = unit / (a.n_rb * a.h_kv);
  const int tid = threadIdx.x;
  const int row = tid / TPR, f0 = (tid % TPR) * FPT;
  const int R = rb * 16 + row;
  if (R >= a.rows) return;
  const int L = min(max(a.seqlens[b], 0), a.L_cap);
  // lengths above the plan's bound are a precondition violation; never read
  // partials the plan did not allot
  const int ns = min((L + a.split_len - 1) / a.split_len, a.n_splits);
  const int64_t base = (int64_t)unit * a.n_splits * 16 + row;
  float M = kNegInf;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, a.ws_lse[base + (int64_t)s * 16]);
  float acc[FPT];
#pragma unroll
  for (int f = 0; f < FPT; ++f) acc[f] = 0.f;
  float den = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float ls = a.ws_lse[base + (int64_t)s * 16];
    const float w = (ls == kNegInf) ? 0.f : fast_exp2(ls - M);
    den += w;
    const float* src = a.ws_o + (base + (int64_t)s * 16) * D + f0;
#pragma unroll
    for (int f = 0; f < FPT; f += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(src + f);
      acc[f] += w * x[0]; acc[f + 1] += w * x[1]; acc[f + 2] += w * x[2]; acc[f + 3] += w * x[3];
    }
  }
  // a row with no visible key (only when L_b < s_q) gets zeros and lse -inf
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const int hh = R / a.s_q, tq = R % a.s_q;
  const int head = j * a.group + hh;
  const int64_t obase = (int64_t)b * a.o_sb + (int64_t)head * a.o_sh + (int64_t)tq * a.o_ss + f0;
  if constexpr (OUT_F32) {
#pragma unroll
    for (int f = 0; f < FPT; f += 4)
      *reinterpret_cast<f32x4*>((float*)a.o + obase + f) =
          f32x4{acc[f] * inv, acc[f + 1] * inv, acc[f + 2] * inv, acc[f + 3] * inv};
  } else {
#pragma unroll
    for (int f = 0; f < FPT; f += 4)
      *reinterpret_cast<u32x2*>((__bf16*)a.o + obase + f) =
          u32x2{pack_bf16(acc[f] * inv, acc[f + 1] * inv), pack_bf16(acc[f + 2] * inv, acc[f + 3] * inv)};
  }
  if (a.lse != nullptr && (tid % TPR) == 0)
    a.lse[((int64_t)b * a.h_q + head) * a.s_q + tq] = den > 0.f ? (M + fast_log2(den)) * kLn2 : kNegInf;
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, bool out_f32, hipStream_t st) {
  const int units = a.B * a.h_kv * a.n_rb;
  hipLaunchKernelGGL(gqa_decode_split_kernel<D>, dim3(units * a.n_splits), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (out_f32)
    hipLaunchKernelGGL((gqa_decode_merge_kernel<D, true>), dim3(units), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((gqa_decode_merge_kernel<D, false>), dim3(units), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gqa_decode(const DecodeArgs& a, int d, bool out_f32, hipStream_t st) {
  if (d == 128) return launch_d<128>(a, out_f32, st);
  if (d == 64) return launch_d<64>(a, out_f32, st);
  return hipErrorInvalidValue;
}

}  // namespace gha
