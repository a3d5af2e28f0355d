// GTA shared-score attention prefill, bf16, fp32 accumulation, on gfx950 MFMA.
//
// "GTA: Grouped-head latenT Attention" news article, grouped shared attention
// matrix mechanism: the heads of a group share one attention matrix, computed
// once and handed to every head of the group.  The kernel mirrors that
// structure.  A work-group owns 64 positions of one group:
//   1. Score phase: wave w computes S for positions 16w..16w+15 against the
//      group's key tile (S^T = K Q^T, K staged in LDS), runs the online
//      softmax for those rows, and publishes the bf16 probabilities P and a
//      per-row rescale factor in LDS.
//   2. Value phase: wave w acts as head w of the group (with fewer than four
//      heads, waves split a head's positions): it applies the shared P of all
//      64 positions to its own head's values.  V never passes through LDS:
//      each lane loads 8 keys x 4 features of its head's V tile with 8-byte
//      loads and transposes them in registers into MFMA operands, and the key
//      order of the score tiles makes P^T line up with those keys.
// Each value fragment feeds four MFMAs (four 16-row position tiles), and the
// score matrix is computed once per group, not once per head.
#include "device_common.hpp"
#include "kernels.hpp"

namespace gha {
namespace {

constexpr int KB = 64;   // keys per iteration
constexpr int PR = 64;   // positions per work-group
constexpr int DVH = 64;  // value width of one head
constexpr int PP = KB + 8;  // P row pitch in LDS (elements), 16 B pad

template <int DQK, int H, bool OUT_F32>
__global__ __launch_bounds__(256, 2) void gta_kernel(PrefillArgs a) {
  constexpr int KP = DQK + 8;
  constexpr int DS = DQK / 32;
  constexpr int KCH = DQK / 8;              // 16-byte chunks per K row
  constexpr int K_LOADS = KB * KCH / 256;   // per thread
  constexpr int K_ROWSTEP = 256 / KCH;
  constexpr int QTV = H;                    // position tiles per wave in the value phase
  static_assert(H == 1 || H == 2 || H == 4, "heads per group");

  __shared__ __attribute__((aligned(16))) __bf16 k_s[KB * KP];
  __shared__ __attribute__((aligned(16))) __bf16 p_s[PR * PP];
  __shared__ float alpha_s[PR];
  __shared__ float l_s[PR];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;

  const uint32_t lid = xcd_logical_id(blockIdx.x, gridDim.x);
  if (lid >= (uint32_t)a.n_blocks) return;
  const int n_qb = a.n_qblocks;
  const int qb = n_qb - 1 - (int)(lid % n_qb);  // heavy (late) blocks first
  const int grp = (int)(lid / n_qb) % a.h_kv;
  const int b = (int)(lid / n_qb) / a.h_kv;
  const int pos_wg = qb * PR;
  const int S = a.S_q;

  // score phase: this wave's 16 positions
  const int spos0 = pos_wg + 16 * wave;
  // value phase: head and position tiles of this wave
  const int vhead = wave / (4 / H);
  const int vq0 = (wave % (4 / H)) * QTV;

  int k_end = S;
  if (a.causal) k_end = min(S, pos_wg + PR);
  const int n_kb = (k_end + KB - 1) / KB;
  const int wave_kmax = a.causal ? min(spos0 + 15, S - 1) : S - 1;

  const __bf16* qbase = (const __bf16*)a.q + (int64_t)b * a.q_sb + (int64_t)grp * a.q_sh;
  const __bf16* kbase = (const __bf16*)a.k + (int64_t)b * a.k_sb + (int64_t)grp * a.k_sh;
  const __bf16* vbase = (const __bf16*)a.v + (int64_t)b * a.v_sb + (int64_t)(grp * a.group + vhead) * a.v_sh;

  u32x4 qf[DS];
  {
    const int pos = min(spos0 + li, S - 1);
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[s] = ld16(qbase + (int64_t)pos * a.q_ss + 32 * s + 8 * lg);
  }

  // K staging (LDS, single buffer: stored after every wave has finished the
  // previous tile's scores)
  const int k_row = tid / KCH, k_col = (tid % KCH) * 8;
  const __bf16* kthr = kbase + (int64_t)k_row * a.k_ss + k_col;
  const int64_t k_rowstep = (int64_t)K_ROWSTEP * a.k_ss;
  u32x4 kreg[K_LOADS];
  // Whole tiles use strided addresses; the tail tile clamps rows to the last
  // position (their scores are masked).
  auto load_k = [&](int kb) {
    const int key0 = kb * KB;
    if (key0 + KB <= S) {
      const __bf16* p = kthr + (int64_t)key0 * a.k_ss;
#pragma unroll
      for (int i = 0; i < K_LOADS; ++i) kreg[i] = ld16(p + i * k_rowstep);
    } else {
#pragma unroll
      for (int i = 0; i < K_LOADS; ++i) {
        const int kk = min(key0 + k_row + K_ROWSTEP * i, S - 1);
        kreg[i] = ld16(kbase + (int64_t)kk * a.k_ss + k_col);
      }
    }
  };
  auto store_k = [&]() {
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) st16(k_s + (k_row + K_ROWSTEP * i) * KP + k_col, kreg[i]);
  };
  // V straight into registers: lane (li, lg) loads keys 32*hk + 8*lg + tt,
  // features 8*(li & 7) + 4*(li >> 3) .. +3 (8 bytes); lanes 0..15 of one load
  // cover a whole 128-byte row.
  const int v_col = 8 * (li & 7) + 4 * (li >> 3);
  const __bf16* vthr = vbase + (int64_t)(8 * lg) * a.v_ss + v_col;
  u32x2 vbuf[2][2][8];  // two tiles in flight: this one and the next
  auto load_v = [&](int kb, u32x2 (&vr)[2][8]) {
    const int key0 = kb * KB;
    if (key0 + KB <= S) {
      const __bf16* p = vthr + (int64_t)key0 * a.v_ss;
#pragma unroll
      for (int hk = 0; hk < 2; ++hk)
#pragma unroll
        for (int tt = 0; tt < 8; ++tt)
          vr[hk][tt] = *reinterpret_cast<const u32x2*>(p + (int64_t)(32 * hk + tt) * a.v_ss);
    } else {
#pragma unroll
      for (int hk = 0; hk < 2; ++hk)
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
          const int kk = min(key0 + 32 * hk + 8 * lg + tt, S - 1);
          vr[hk][tt] = *reinterpret_cast<const u32x2*>(vbase + (int64_t)kk * a.v_ss + v_col);
        }
    }
  };

  f32x4 oacc[4][QTV];
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int q = 0; q < QTV; ++q) oacc[w][q] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 lacc = {0.f, 0.f, 0.f, 0.f};
  float m2 = kNegInf;
  const float c2 = a.scale * kLog2e;
  const u32x4 ones = {kBf16OnePair, kBf16OnePair, kBf16OnePair, kBf16OnePair};

  if (n_kb > 0) {
    load_k(0);
    store_k();
  }
  wait_vmem_all();
  __syncthreads();
  if (n_kb > 0) load_v(0, vbuf[0]);

  // One iteration per key tile; `vr` holds this tile's values (loaded one
  // iteration earlier), `vn` receives the next tile's.  K(t+1) is loaded at
  // the top and stored at the bottom, so both loads have a whole iteration
  // to land.
  auto iteration = [&](int kb, u32x2 (&vr)[2][8], u32x2 (&vn)[2][8]) {
    const int key0 = kb * KB;
    // prefetch unconditionally (the last iteration re-reads its own tile):
    // no branch around the loads keeps the compiler's memory waits exact
    const int kn = min(kb + 1, n_kb - 1);
    load_v(kn, vn);
    load_k(kn);

    // ---- score phase: S^T for this wave's 16 positions -------------------
    // score tile t, row i  <->  key key0 + 32*(t/2) + 8*(i/4) + 4*(t%2) + i%4
    if (key0 <= wave_kmax) {
      f32x4 sacc[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        const __bf16* kr = k_s + (32 * (t >> 1) + 8 * (li >> 2) + 4 * (t & 1) + (li & 3)) * KP + 8 * lg;
#pragma unroll
        for (int s = 0; s < DS; ++s) sacc[t] = mfma_bf16(ld16(kr + 32 * s), qf[s], sacc[t]);
      }
      // lane group lg, tile t, element r  <->  key key0 + 32*(t/2) + 8*lg + 4*(t%2) + r
      const int qpos = spos0 + li;
      const int kmax = a.causal ? min(qpos, S - 1) : S - 1;
      if (key0 + KB - 1 > (a.causal ? spos0 : S - 1)) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (key0 + 32 * (t >> 1) + 8 * lg + 4 * (t & 1) + r > kmax) sacc[t][r] = kNegInf;
      }
      float mx = fmaxf(fmaxf(sacc[0][0], sacc[0][1]), sacc[0][2]);
      mx = fmaxf(fmaxf(mx, sacc[0][3]), sacc[1][0]);
      mx = fmaxf(fmaxf(mx, sacc[1][1]), sacc[1][2]);
      mx = fmaxf(fmaxf(mx, sacc[1][3]), sacc[2][0]);
      mx = fmaxf(fmaxf(mx, sacc[2][1]), sacc[2][2]);
      mx = fmaxf(fmaxf(mx, sacc[2][3]), sacc[3][0]);
      mx = fmaxf(fmaxf(mx, sacc[3][1]), sacc[3][2]);
      mx = fmaxf(mx, sacc[3][3]);
      const float mx2 = group4_max(mx) * c2;
      float alpha = 1.f;
      if (wave_any(mx2 > m2 + kRescaleSlack)) {
        const float mnew = fmaxf(m2, mx2);
        alpha = (mnew == kNegInf) ? 1.f : fast_exp2(m2 - mnew);
        m2 = mnew;
        lacc *= alpha;
      }
      const float msub = (m2 == kNegInf) ? 0.f : m2;
      float p[4][4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) p[t][r] = fast_exp2(__builtin_fmaf(sacc[t][r], c2, -msub));
#pragma unroll
      for (int hk = 0; hk < 2; ++hk) {
        const u32x4 pf = {pack_bf16(p[2 * hk][0], p[2 * hk][1]), pack_bf16(p[2 * hk][2], p[2 * hk][3]),
                          pack_bf16(p[2 * hk + 1][0], p[2 * hk + 1][1]),
                          pack_bf16(p[2 * hk + 1][2], p[2 * hk + 1][3])};
        lacc = mfma_bf16(ones, pf, lacc);
        // P row (16*wave + li), keys 32*hk + 8*lg .. +7
        st16(p_s + (16 * wave + li) * PP + 32 * hk + 8 * lg, pf);
      }
      alpha_s[16 * wave + li] = alpha;  // the four lane groups write the same value
    } else {
      // tile wholly above this wave's diagonal: zero probabilities
#pragma unroll
      for (int hk = 0; hk < 2; ++hk)
        st16(p_s + (16 * wave + li) * PP + 32 * hk + 8 * lg, u32x4{0u, 0u, 0u, 0u});
      alpha_s[16 * wave + li] = 1.f;
    }
    __syncthreads();  // P, alpha visible; every wave is done reading k_s

    // ---- value phase: this wave's head over its position tiles ------------
#pragma unroll
    for (int q = 0; q < QTV; ++q) {
      const int qt = vq0 + q;  // position tile = the score wave that wrote it
      const float al = alpha_s[16 * qt + li];
      if (wave_any(al != 1.f)) {
#pragma unroll
        for (int w = 0; w < 4; ++w) oacc[w][q] *= al;
      }
    }
#pragma unroll
    for (int hk = 0; hk < 2; ++hk) {
      u32x4 pt[QTV];
#pragma unroll
      for (int q = 0; q < QTV; ++q) pt[q] = ld16(p_s + (16 * (vq0 + q) + li) * PP + 32 * hk + 8 * lg);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // features 8*(li&7) + 4*(li>>3) + w: dword w/2 of each key's 4 features
        const int dw = w >> 1;
        const u32x4 av = (w & 1) ? u32x4{hi_pair(vr[hk][0][dw], vr[hk][1][dw]), hi_pair(vr[hk][2][dw], vr[hk][3][dw]),
                                         hi_pair(vr[hk][4][dw], vr[hk][5][dw]), hi_pair(vr[hk][6][dw], vr[hk][7][dw])}
                                 : u32x4{lo_pair(vr[hk][0][dw], vr[hk][1][dw]), lo_pair(vr[hk][2][dw], vr[hk][3][dw]),
                                         lo_pair(vr[hk][4][dw], vr[hk][5][dw]), lo_pair(vr[hk][6][dw], vr[hk][7][dw])};
#pragma unroll
        for (int q = 0; q < QTV; ++q) oacc[w][q] = mfma_bf16(av, pt[q], oacc[w][q]);
      }
    }
    store_k();
    __syncthreads();  // P consumed, next K tile visible
  };
  for (int kb = 0; kb < n_kb; kb += 2) {
    iteration(kb, vbuf[0], vbuf[1]);
    if (kb + 1 < n_kb) iteration(kb + 1, vbuf[1], vbuf[0]);
  }

  // ---- epilogue ------------------------------------------------------------
  if (lg == 0) l_s[16 * wave + li] = lacc[0];
  if (lg == 0 && a.lse != nullptr && spos0 + li < S)
    a.lse[((int64_t)b * a.lse_heads + grp) * S + spos0 + li] = (m2 + fast_log2(lacc[0])) * kLn2;
  __syncthreads();
  // oacc[w][q][r] of lane (li, lg) is feature 8*((4*lg + r) & 7) + 4*((4*lg + r) >> 3) + w
  // of position tile vq0 + q, row li: four consecutive features per (q, r).
  const int head = grp * a.group + vhead;
#pragma unroll
  for (int q = 0; q < QTV; ++q) {
    const int row = 16 * (vq0 + q) + li;
    const int pos = pos_wg + row;
    if (pos >= S) continue;
    const float inv = 1.f / l_s[row];
    const int64_t obase = (int64_t)b * a.o_sb + (int64_t)head * a.o_sh + (int64_t)pos * a.o_ss;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * lg + r;
      const int f = 8 * (i & 7) + 4 * (i >> 3);
      const f32x4 v = f32x4{oacc[0][q][r], oacc[1][q][r], oacc[2][q][r], oacc[3][q][r]} * inv;
      if constexpr (OUT_F32)
        *reinterpret_cast<f32x4*>((float*)a.o + obase + f) = v;
      else
        *reinterpret_cast<u32x2*>((__bf16*)a.o + obase + f) = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
    }
  }
}

template <int DQK, int H>
hipError_t launch_h(const PrefillArgs& a, bool out_f32, hipStream_t st) {
  const uint32_t padded = (uint32_t)((a.n_blocks + 7) / 8 * 8);
  if (out_f32)
    hipLaunchKernelGGL((gta_kernel<DQK, H, true>), dim3(padded), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((gta_kernel<DQK, H, false>), dim3(padded), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

int gta_positions_per_wg() { return PR; }

hipError_t launch_gta(const PrefillArgs& a, int d_qk, int heads_per_group, bool out_f32, hipStream_t st) {
#define GHA_GTA_CASE(DQ, HH) \
  if (d_qk == DQ && heads_per_group == HH) return launch_h<DQ, HH>(a, out_f32, st);
  GHA_GTA_CASE(64, 4)
  GHA_GTA_CASE(64, 2)
  GHA_GTA_CASE(64, 1)
  GHA_GTA_CASE(128, 4)
  GHA_GTA_CASE(128, 2)
  GHA_GTA_CASE(128, 1)
#undef GHA_GTA_CASE
  return hipErrorInvalidValue;
}

}  // namespace gha
