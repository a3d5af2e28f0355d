// Debug check of the decode length precondition, s_q <= seqlens_k[b] <= L_cap
// (the new tokens are the last s_q cached positions and a decode step reads
// the whole cached history: "GQLA: Group-Query Latent Attention ...",
// section 1).  Launched by the decode entry points only when debug checks are
// on; the host waits for its two-word answer before launching anything else.
#include <hip/hip_runtime.h>

#include <climits>

#include "kernels.hpp"

namespace gha {
namespace {

__global__ __launch_bounds__(256) void check_lengths_kernel(const int32_t* seqlens, int B, int lo, int hi,
                                                            int32_t* out) {
  __shared__ int first;
  if (threadIdx.x == 0) first = INT_MAX;
  __syncthreads();
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    const int L = seqlens[b];
    if (L < lo || L > hi) atomicMin(&first, b);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const bool bad = first != INT_MAX;
    out[0] = bad ? first : -1;
    out[1] = bad ? seqlens[first] : 0;
  }
}

}  // namespace

hipError_t launch_check_lengths(const int32_t* seqlens, int B, int lo, int hi, int32_t* out, hipStream_t st) {
  hipLaunchKernelGGL(check_lengths_kernel, dim3(1), dim3(256), 0, st, seqlens, B, lo, hi, out);
  return hipGetLastError();
}

}  // namespace gha
