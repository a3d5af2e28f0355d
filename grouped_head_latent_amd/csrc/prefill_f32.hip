// Grouped-query attention prefill with fp32 inputs and outputs ("Grouped
// Query Attention (GQA)", Ultralytics glossary, "How GQA works": the worked
// example runs in fp32 at 8 query heads over 2 key/value heads).
//
// These are small problems, so what matters is latency: one wave per
// (batch, query head, 16 query rows), and both contractions on the fp32
// matrix cores (v_mfma_f32_16x16x4_f32, full fp32 products and sums) instead
// of long chains of dependent VALU multiply-adds.  Per 16-key tile:
//   S^T = K Q^T: 16 keys x 16 rows, D / 4 MFMAs.  Lane (group g, index i)
//     supplies K[key i][dim] and Q[row i][dim] for the contraction slot g of
//     each step, slot g of step s being dim (D / 4) g + s, so that a lane's
//     K and Q values are D / 4 consecutive dims (vector loads, Q resident).
//     The accumulator holds S^T[key 4 g + r][row i] in lane (g, i).
//   online softmax per row (the four lane groups of column i), in log2 units;
//   O^T += V^T P^T: the contraction slot g of step s is key 4 g + s, so that
//     the B operand P^T[key 4 g + s][row i] is the lane's own probability r = s
//     and nothing moves between lanes; V^T[dim][key] is read from the tile in
//     LDS.  The accumulator holds O[row i][dim 16 t + 4 g + r].
#include "device_common.hpp"
#include "kernels.hpp"

namespace gha {
namespace {

constexpr int TK = 16;  // keys per tile

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int D>
__global__ __launch_bounds__(64) void prefill_f32_kernel(PrefillArgs a) {
  constexpr int DPL = D / 4;       // dims per lane group = score MFMA steps
  constexpr int DT = D / 16;       // 16-dim output tiles
  constexpr int VP = D + 16;       // V row pitch in LDS (floats): rows 64 B apart in the banks
  __shared__ __attribute__((aligned(16))) float vs[TK * VP];

  const int lane = threadIdx.x, li = lane & 15, lg = lane >> 4;
  const int qb = blockIdx.x, qhead = blockIdx.y, b = blockIdx.z;
  const int kvh = qhead / a.group;
  const int row = qb * 16 + li;                 // this lane's query row
  const bool valid = row < a.S_q;
  const int off = a.S_k - a.S_q;                // bottom-right causal offset
  const int kmax_row = a.causal ? min(min(row, a.S_q - 1) + off, a.S_k - 1) : a.S_k - 1;
  int k_end = a.S_k;
  if (a.causal) k_end = min(a.S_k, min(qb * 16 + 15, a.S_q - 1) + off + 1);

  const float* kp = (const float*)a.k + (int64_t)b * a.k_sb + (int64_t)kvh * a.k_sh;
  const float* vp = (const float*)a.v + (int64_t)b * a.v_sb + (int64_t)kvh * a.v_sh;
  float qv[DPL];
  {
    const float* qp = (const float*)a.q + (int64_t)b * a.q_sb + (int64_t)qhead * a.q_sh +
                      (int64_t)min(row, a.S_q - 1) * a.q_ss + DPL * lg;
#pragma unroll
    for (int s = 0; s < DPL; s += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(qp + s);
      qv[s] = x[0]; qv[s + 1] = x[1]; qv[s + 2] = x[2]; qv[s + 3] = x[3];
    }
  }

  f32x4 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float c2 = a.scale * kLog2e;
  float m2 = kNegInf;   // running maximum of the row (log2 units)
  float lpart = 0.f;    // this lane's share of the row's normaliser

  for (int k0 = 0; k0 < k_end; k0 += TK) {
    // V tile into LDS (rows past the end read as zeros), K operand straight
    // into registers
    __syncthreads();  // the previous tile's V reads are done
#pragma unroll
    for (int e = 4 * lane; e < TK * D; e += 256) {
      const int key = e / D, dim = e % D;
      const f32x4 x = k0 + key < a.S_k ? *reinterpret_cast<const f32x4*>(vp + (int64_t)(k0 + key) * a.v_ss + dim)
                                       : f32x4{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4*>(&vs[key * VP + dim]) = x;
    }
    float kv[DPL];
    {
      const bool in = k0 + li < a.S_k;
      const float* kr = kp + (int64_t)(k0 + li) * a.k_ss + DPL * lg;
#pragma unroll
      for (int s = 0; s < DPL; s += 4) {
        const f32x4 x = in ? *reinterpret_cast<const f32x4*>(kr + s) : f32x4{0.f, 0.f, 0.f, 0.f};
        kv[s] = x[0]; kv[s + 1] = x[1]; kv[s + 2] = x[2]; kv[s + 3] = x[3];
      }
    }
    // S^T = K Q^T
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < DPL; ++s) sacc = mfma_f32(kv[s], qv[s], sacc);
    // online softmax of row li over keys k0 + 4 lg + r
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = k0 + 4 * lg + r;
      sacc[r] = key <= kmax_row ? sacc[r] * c2 : kNegInf;
      mx = fmaxf(mx, sacc[r]);
    }
    mx = group4_max(mx);
    const float mnew = fmaxf(m2, mx);
    const float alpha = (mnew == kNegInf) ? 1.f : fast_exp2(m2 - mnew);
    const float msub = (mnew == kNegInf) ? 0.f : mnew;
    m2 = mnew;
    lpart *= alpha;
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t] *= alpha;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = fast_exp2(sacc[r] - msub);
      lpart += p[r];
    }
    __syncthreads();  // the V tile is in LDS
    // O^T += V^T P^T, contraction slot g of step s = key 4 g + s
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int s = 0; s < 4; ++s) oacc[t] = mfma_f32(vs[(4 * lg + s) * VP + 16 * t + li], p[s], oacc[t]);
  }

  const float l = group4_sum(lpart);
  if (!valid) return;
  const float inv = 1.f / l;
  float* op = (float*)a.o + (int64_t)b * a.o_sb + (int64_t)qhead * a.o_sh + (int64_t)row * a.o_ss + 4 * lg;
#pragma unroll
  for (int t = 0; t < DT; ++t) *reinterpret_cast<f32x4*>(op + 16 * t) = oacc[t] * inv;
  if (a.lse != nullptr && lg == 0) a.lse[((int64_t)b * a.lse_heads + qhead) * a.S_q + row] = (m2 + fast_log2(l)) * kLn2;
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, int d, hipStream_t st) {
  const int h_q = a.h_kv * a.group;
  dim3 grid((a.S_q + 15) / 16, h_q, a.B);
  if (d == 64)
    hipLaunchKernelGGL(prefill_f32_kernel<64>, grid, dim3(64), 0, st, a);
  else if (d == 128)
    hipLaunchKernelGGL(prefill_f32_kernel<128>, grid, dim3(64), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace gha
