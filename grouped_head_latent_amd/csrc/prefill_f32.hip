// Grouped-query attention prefill with fp32 inputs and outputs ("Grouped
// Query Attention (GQA)", Ultralytics glossary, "How GQA works": the worked
// example runs in fp32 at 8 query heads over 2 key/value heads).
//
// fp32 has no dense-MFMA advantage worth the layout work at these sizes, so
// this path is plain VALU: one lane per query row, the row's q and running
// output in registers, K/V tiles of 32 keys staged in LDS and read as
// broadcasts (every lane reads the same key row, so there are no bank
// conflicts).  A work-group is one wave covering 64 positions of one head.
#include "device_common.hpp"
#include "kernels.hpp"

namespace gha {
namespace {

constexpr int TK = 32;

template <int D>
__global__ __launch_bounds__(64) void prefill_f32_kernel(PrefillArgs a) {
  __shared__ float ks[TK][D];
  __shared__ float vs[TK][D];
  const int lane = threadIdx.x;
  const int qb = blockIdx.x;
  const int qhead = blockIdx.y;
  const int b = blockIdx.z;
  const int kvh = qhead / a.group;
  const int pos = qb * 64 + lane;
  const int off = a.S_k - a.S_q;
  const bool valid = pos < a.S_q;

  const float* qp = (const float*)a.q + (int64_t)b * a.q_sb + (int64_t)qhead * a.q_sh + (int64_t)pos * a.q_ss;
  const float* kp = (const float*)a.k + (int64_t)b * a.k_sb + (int64_t)kvh * a.k_sh;
  const float* vp = (const float*)a.v + (int64_t)b * a.v_sb + (int64_t)kvh * a.v_sh;

  float q[D], o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    q[c] = valid ? qp[c] : 0.f;
    o[c] = 0.f;
  }
  const float c2 = a.scale * kLog2e;
  float m = kNegInf, l = 0.f;
  const int kmax_row = a.causal ? min(pos + off, a.S_k - 1) : a.S_k - 1;
  int k_end = a.S_k;
  if (a.causal) k_end = min(a.S_k, min(qb * 64 + 63, a.S_q - 1) + off + 1);

  for (int k0 = 0; k0 < k_end; k0 += TK) {
    __syncthreads();
    for (int idx = lane; idx < TK * D / 4; idx += 64) {
      const int r = idx / (D / 4), c4 = (idx % (D / 4)) * 4;
      const bool in = k0 + r < a.S_k;
      f32x4 kv = in ? *reinterpret_cast<const f32x4*>(kp + (int64_t)(k0 + r) * a.k_ss + c4) : f32x4{0, 0, 0, 0};
      f32x4 vv = in ? *reinterpret_cast<const f32x4*>(vp + (int64_t)(k0 + r) * a.v_ss + c4) : f32x4{0, 0, 0, 0};
      *reinterpret_cast<f32x4*>(&ks[r][c4]) = kv;
      *reinterpret_cast<f32x4*>(&vs[r][c4]) = vv;
    }
    __syncthreads();
    float s[TK];
    float mx = kNegInf;
#pragma unroll
    for (int u = 0; u < TK; ++u) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) acc = __builtin_fmaf(q[c], ks[u][c], acc);
      s[u] = (k0 + u <= kmax_row) ? acc * c2 : kNegInf;
      mx = fmaxf(mx, s[u]);
    }
    const float mnew = fmaxf(m, mx);
    const float alpha = (mnew == kNegInf) ? 1.f : fast_exp2(m - mnew);
    const float msub = (mnew == kNegInf) ? 0.f : mnew;
    m = mnew;
    l *= alpha;
#pragma unroll
    for (int c = 0; c < D; ++c) o[c] *= alpha;
#pragma unroll
    for (int u = 0; u < TK; ++u) {
      const float p = fast_exp2(s[u] - msub);
      l += p;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] = __builtin_fmaf(p, vs[u][c], o[c]);
    }
  }
  if (!valid) return;
  const float inv = 1.f / l;
  float* op = (float*)a.o + (int64_t)b * a.o_sb + (int64_t)qhead * a.o_sh + (int64_t)pos * a.o_ss;
#pragma unroll
  for (int c = 0; c < D; c += 4)
    *reinterpret_cast<f32x4*>(op + c) = f32x4{o[c] * inv, o[c + 1] * inv, o[c + 2] * inv, o[c + 3] * inv};
  if (a.lse) a.lse[((int64_t)b * a.lse_heads + qhead) * a.S_q + pos] = (m + fast_log2(l)) * kLn2;
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, int d, hipStream_t st) {
  const int h_q = a.h_kv * a.group;
  dim3 grid((a.S_q + 63) / 64, h_q, a.B);
  if (d == 64)
    hipLaunchKernelGGL(prefill_f32_kernel<64>, grid, dim3(64), 0, st, a);
  else if (d == 128)
    hipLaunchKernelGGL(prefill_f32_kernel<128>, grid, dim3(64), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace gha
