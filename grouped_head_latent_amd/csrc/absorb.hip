// Absorption products around the absorbed latent decode ("GQLA: Group-Query
// Latent Attention ...", section 3.1, Eq. (1), and Figure 2, right): before
// attention the content query of head i in group j = i / (h_q / g) becomes
// q~_i = (W^UK_j)^T q^C_i (width r_kv); after attention the head's output is
// O_i = W^UV_j o_lat_i (width d_h), where W^UK and W^UV stack the groups'
// (d_h x r_kv) blocks.  Both are per-group matrix products over the rows
// (batch x new tokens x heads of the group), on MFMA (bf16 in, fp32
// accumulate).  Every operand fragment is a 16-byte load straight from
// global memory (L2): the output tile is computed transposed, so that both
// operands are read along their contiguous axis; W^UK, whose contiguous axis
// is the output one, is first transposed into the workspace.
#include "device_common.hpp"
#include "kernels.hpp"

namespace gha {
namespace {

constexpr int DH = 128, RKV = 512;

// row rr of group j: (b, t, head) with head = j * qpg + rr % qpg
__device__ __forceinline__ void row_of(const AbsorbArgs& a, int j, int rr, int& b, int& t, int& head) {
  const int qpg = a.h_q / a.g;
  const int bt = rr / qpg;
  head = j * qpg + rr % qpg;
  b = bt / a.s_q;
  t = bt % a.s_q;
}

// w_t[j][n][c] = W^UK[j d_h + c][n]: one 16 x 16 block per thread row
__global__ __launch_bounds__(256) void transpose_wuk_kernel(AbsorbArgs a) {
  __shared__ uint16_t tile[32][33];
  const int j = blockIdx.z, c0 = blockIdx.y * 32, n0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  const uint16_t* w = (const uint16_t*)a.w + (int64_t)j * DH * RKV;
  for (int r = ty; r < 32; r += 8) tile[r][tx] = w[(int64_t)(c0 + r) * RKV + n0 + tx];
  __syncthreads();
  uint16_t* wt = (uint16_t*)a.wt + (int64_t)j * RKV * DH;
  for (int r = ty; r < 32; r += 8) wt[(int64_t)(n0 + r) * DH + c0 + tx] = tile[tx][r];
}

// q~^T tile (16 n x 16 rows) = W^UK_j^T (n x c) q^C^T (c x rows), c = 128:
// a work-group takes 256 n (wave w: n-tiles 4 w .. 4 w + 3) and 32 rows
__global__ __launch_bounds__(256) void absorb_query_kernel(AbsorbArgs a) {
  const int j = blockIdx.z, nh = blockIdx.y, r0 = blockIdx.x * 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int nrows = a.B * a.s_q * (a.h_q / a.g);
  // B operand rows: this lane's row li of each row tile
  const __bf16* qrow[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    int b, t, head;
    row_of(a, j, min(r0 + 16 * rt + li, nrows - 1), b, t, head);
    qrow[rt] = (const __bf16*)a.in + (int64_t)b * a.in_sb + (int64_t)head * a.in_sh + (int64_t)t * a.in_ss;
  }
  const __bf16* wt = (const __bf16*)a.wt + (int64_t)j * RKV * DH;
  const int nt0 = nh * 16 + 4 * wave;  // first n-tile of this wave
  f32x4 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < DH; k += 32) {
    u32x4 bq[2], aw[4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) bq[rt] = ld16(qrow[rt] + k + 8 * lg);
#pragma unroll
    for (int i = 0; i < 4; ++i) aw[i] = ld16(wt + (int64_t)(16 * (nt0 + i) + li) * DH + k + 8 * lg);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) acc[i][rt] = mfma_bf16(aw[i], bq[rt], acc[i][rt]);
  }
  // acc[i][rt][r] = q~[row r0 + 16 rt + li][n = 16 (nt0 + i) + 4 lg + r]
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int rr = r0 + 16 * rt + li;
    if (rr >= nrows) continue;
    int b, t, head;
    row_of(a, j, rr, b, t, head);
    __bf16* o = (__bf16*)a.out + (((int64_t)b * a.s_q + t) * a.h_q + head) * RKV;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = 16 * (nt0 + i) + 4 * lg;
      *reinterpret_cast<u32x2*>(o + n) = u32x2{pack_bf16(acc[i][rt][0], acc[i][rt][1]), pack_bf16(acc[i][rt][2], acc[i][rt][3])};
    }
  }
}

// O^T tile (16 m x 16 rows) = W^UV_j (m x c) o_lat^T (c x rows), c = 512:
// a work-group takes all 128 m (wave w: m-tiles 2 w, 2 w + 1) and 32 rows
template <bool OUT_F32>
__global__ __launch_bounds__(256) void absorb_output_kernel(AbsorbArgs a) {
  const int j = blockIdx.y, r0 = blockIdx.x * 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int nrows = a.B * a.s_q * (a.h_q / a.g);
  const __bf16* lrow[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    int b, t, head;
    row_of(a, j, min(r0 + 16 * rt + li, nrows - 1), b, t, head);
    lrow[rt] = (const __bf16*)a.lat + (((int64_t)b * a.s_q + t) * a.h_q + head) * RKV;
  }
  const __bf16* w = (const __bf16*)a.w + (int64_t)j * DH * RKV;
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int k = 0; k < RKV; k += 32) {
    u32x4 bl[2], aw[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) bl[rt] = ld16(lrow[rt] + k + 8 * lg);
#pragma unroll
    for (int i = 0; i < 2; ++i) aw[i] = ld16(w + (int64_t)(16 * (2 * wave + i) + li) * RKV + k + 8 * lg);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) acc[i][rt] = mfma_bf16(aw[i], bl[rt], acc[i][rt]);
  }
  // acc[i][rt][r] = O[row r0 + 16 rt + li][m = 16 (2 w + i) + 4 lg + r]
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int rr = r0 + 16 * rt + li;
    if (rr >= nrows) continue;
    int b, t, head;
    row_of(a, j, rr, b, t, head);
    const int64_t base = (int64_t)b * a.o_sb + (int64_t)head * a.o_sh + (int64_t)t * a.o_ss;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int m = 16 * (2 * wave + i) + 4 * lg;
      if constexpr (OUT_F32)
        *reinterpret_cast<f32x4*>((float*)a.out + base + m) = acc[i][rt];
      else
        *reinterpret_cast<u32x2*>((__bf16*)a.out + base + m) =
            u32x2{pack_bf16(acc[i][rt][0], acc[i][rt][1]), pack_bf16(acc[i][rt][2], acc[i][rt][3])};
    }
  }
}

}  // namespace

hipError_t launch_absorb_query(const AbsorbArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(transpose_wuk_kernel, dim3(RKV / 32, DH / 32, a.g), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nrows = a.B * a.s_q * (a.h_q / a.g);
  hipLaunchKernelGGL(absorb_query_kernel, dim3((nrows + 31) / 32, RKV / 256, a.g), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_absorb_output(const AbsorbArgs& a, bool out_f32, hipStream_t st) {
  const int nrows = a.B * a.s_q * (a.h_q / a.g);
  if (out_f32)
    hipLaunchKernelGGL(absorb_output_kernel<true>, dim3((nrows + 31) / 32, a.g), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(absorb_output_kernel<false>, dim3((nrows + 31) / 32, a.g), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace gha
