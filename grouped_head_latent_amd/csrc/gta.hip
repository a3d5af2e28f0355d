// GTA shared-score attention prefill, bf16, fp32 accumulation, on gfx950 MFMA.
//
// "GTA: Grouped-head latenT Attention" news article, grouped shared attention
// matrix mechanism: the heads of a group share one attention matrix, computed
// once and handed to every head of the group.  The kernel mirrors that
// structure.  A work-group owns 64 positions of one group:
//   * Score phase: wave w computes S for positions 16w..16w+15 against the
//     group's key tile (S^T = K Q^T, K staged in LDS), runs the online softmax
//     for those rows, and publishes the bf16 probabilities P and a per-row
//     rescale factor in LDS.
//   * Value phase: wave w acts as head w of the group (with fewer than four
//     heads, waves split a head's positions): it applies the shared P of all
//     64 positions to its own head's values.  V never passes through LDS:
//     each lane loads 8 keys x 4 features of its head's V tile with 8-byte
//     loads and transposes them in registers into MFMA operands, and the key
//     order of the score tiles makes P^T line up with those keys.
// The two phases are software-pipelined across key tiles: iteration t runs
// the score phase of tile t+1 and the value phase of tile t, which are
// independent, in one basic block (so one wave's softmax VALU work can fill
// the gaps between its own value MFMAs), with one barrier per tile; K and P
// are double-buffered in LDS and V in registers.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace gha {
namespace {

constexpr int KB = 64;   // keys per iteration
constexpr int PR = 64;   // positions per work-group
constexpr int PP = KB + 8;  // P row pitch in LDS (elements), 16 B pad
static_assert(PR == KB, "every wave sees every tile it visits: tile t <= the diagonal tile");

template <int DQK, int H, bool OUT_F32>
__global__ __launch_bounds__(256, 2) void gta_kernel(PrefillArgs a) {
  constexpr int KP = DQK + 8;
  constexpr int DS = DQK / 32;
  constexpr int KCH = DQK / 8;              // 16-byte chunks per K row
  constexpr int K_LOADS = KB * KCH / 256;   // per thread
  constexpr int K_ROWSTEP = 256 / KCH;
  constexpr int QTV = H;                    // position tiles per wave in the value phase
  static_assert(H == 1 || H == 2 || H == 4, "heads per group");

  __shared__ __attribute__((aligned(16))) __bf16 k_s[2][KB * KP];
  __shared__ __attribute__((aligned(16))) __bf16 p_s[2][PR * PP];
  __shared__ float alpha_s[2][PR];
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

  const int spos0 = pos_wg + 16 * wave;        // score phase: this wave's 16 positions
  const int vhead = wave / (4 / H);            // value phase: this wave's head
  const int vq0 = (wave % (4 / H)) * QTV;      //   and its position tiles

  const int k_end = a.causal ? min(S, pos_wg + PR) : S;
  const int n_kb = (k_end + KB - 1) / KB;

  const __bf16* qbase = (const __bf16*)a.q + (int64_t)b * a.q_sb + (int64_t)grp * a.q_sh;
  const __bf16* kbase = (const __bf16*)a.k + (int64_t)b * a.k_sb + (int64_t)grp * a.k_sh;
  const __bf16* vbase = (const __bf16*)a.v + (int64_t)b * a.v_sb + (int64_t)(grp * a.group + vhead) * a.v_sh;

  u32x4 qf[DS];
  {
    const int pos = min(spos0 + li, S - 1);
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[s] = ld16(qbase + (int64_t)pos * a.q_ss + 32 * s + 8 * lg);
  }

  // ---- K: global -> registers -> LDS (double buffer) -----------------------
  // Whole tiles use strided addresses; the tail tile clamps rows to the last
  // position (their scores are masked).
  const int k_row = tid / KCH, k_col = (tid % KCH) * 8;
  const __bf16* kthr = kbase + (int64_t)k_row * a.k_ss + k_col;
  const int64_t k_rowstep = (int64_t)K_ROWSTEP * a.k_ss;
  u32x4 kreg[K_LOADS];
  auto load_k = [&](int kb) __attribute__((always_inline)) {
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
  auto store_k = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) st16(&k_s[buf][(k_row + K_ROWSTEP * i) * KP + k_col], kreg[i]);
  };

  // ---- V: global -> registers (double buffer) ------------------------------
  // lane (li, lg) loads keys 32*hk + 8*lg + tt, features
  // 8*(li & 7) + 4*(li >> 3) .. +3 (8 bytes); lanes 0..15 of one load cover a
  // whole 128-byte row.
  const int v_col = 8 * (li & 7) + 4 * (li >> 3);
  const __bf16* vthr = vbase + (int64_t)(8 * lg) * a.v_ss + v_col;
  u32x2 vbuf0[2][8], vbuf1[2][8];
  auto load_v = [&](int kb, u32x2 (&vr)[2][8]) __attribute__((always_inline)) {
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

  // ---- state ----------------------------------------------------------------
  f32x4 oacc[4][QTV];
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int q = 0; q < QTV; ++q) oacc[w][q] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 lacc = {0.f, 0.f, 0.f, 0.f};
  float m2 = kNegInf;
  const float c2 = a.scale * kLog2e;
  const u32x4 ones = {kBf16OnePair, kBf16OnePair, kBf16OnePair, kBf16OnePair};
  const int kmax = a.causal ? min(spos0 + li, S - 1) : S - 1;  // last key this lane's row sees

  // score MFMAs of tile t: S^T tile j, row i  <->  key 32*(j/2) + 8*(i/4) + 4*(j%2) + i%4
  auto score_mfma = [&](int t, f32x4 (&sacc)[4]) __attribute__((always_inline)) {
    const __bf16* kb_s = k_s[t & 1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      const __bf16* kr = kb_s + (32 * (j >> 1) + 8 * (li >> 2) + 4 * (j & 1) + (li & 3)) * KP + 8 * lg;
#pragma unroll
      for (int s = 0; s < DS; ++s) sacc[j] = mfma_bf16(ld16(kr + 32 * s), qf[s], sacc[j]);
    }
  };
  // softmax of tile t (lane group lg, tile j, element r <-> key 32*(j/2) + 8*lg
  // + 4*(j%2) + r), publishing P and the rescale factor of this wave's rows.
  // The running maximum moves per row (the four lanes of a row agree), so the
  // phase is branch-free.
  auto score_softmax = [&](int t, f32x4 (&sacc)[4], auto masked) __attribute__((always_inline)) {
    const int key0 = t * KB;
    if constexpr (decltype(masked)::value) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (key0 + 32 * (j >> 1) + 8 * lg + 4 * (j & 1) + r > kmax) sacc[j][r] = kNegInf;
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
    const float mnew = (mx2 > m2 + kRescaleSlack) ? fmaxf(m2, mx2) : m2;
    const float alpha = (m2 == mnew) ? 1.f : fast_exp2(m2 - mnew);
    m2 = mnew;
    lacc *= alpha;
    const float msub = (m2 == kNegInf) ? 0.f : m2;
    float p[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) p[j][r] = fast_exp2(__builtin_fmaf(sacc[j][r], c2, -msub));
    __bf16* pb = p_s[t & 1];
#pragma unroll
    for (int hk = 0; hk < 2; ++hk) {
      const u32x4 pf = {pack_bf16(p[2 * hk][0], p[2 * hk][1]), pack_bf16(p[2 * hk][2], p[2 * hk][3]),
                        pack_bf16(p[2 * hk + 1][0], p[2 * hk + 1][1]),
                        pack_bf16(p[2 * hk + 1][2], p[2 * hk + 1][3])};
      lacc = mfma_bf16(ones, pf, lacc);
      st16(pb + (16 * wave + li) * PP + 32 * hk + 8 * lg, pf);  // row 16*wave + li, keys 32hk + 8lg ..
    }
    alpha_s[t & 1][16 * wave + li] = alpha;  // the four lane groups write the same value
  };
  // value phase of tile t: this wave's head over its position tiles
  auto value_rescale = [&](int t) __attribute__((always_inline)) {
    float al[QTV];
    bool any = false;
#pragma unroll
    for (int q = 0; q < QTV; ++q) {  // all reads first: one LDS round trip
      al[q] = alpha_s[t & 1][16 * (vq0 + q) + li];
      any |= al[q] != 1.f;
    }
    if (wave_any(any)) {
#pragma unroll
      for (int q = 0; q < QTV; ++q)
#pragma unroll
        for (int w = 0; w < 4; ++w) oacc[w][q] *= al[q];
    }
  };
  auto value_mfma = [&](int t, u32x2 (&vr)[2][8]) __attribute__((always_inline)) {
    const __bf16* pb = p_s[t & 1];
#pragma unroll
    for (int hk = 0; hk < 2; ++hk) {
      u32x4 pt[QTV];
#pragma unroll
      for (int q = 0; q < QTV; ++q) pt[q] = ld16(pb + (16 * (vq0 + q) + li) * PP + 32 * hk + 8 * lg);
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
  };

  // ---- prologue: K(0), K(1) staged, score(0) published, V(0) in flight ------
  load_k(0);
  store_k(0);
  wait_vmem_all();
  __syncthreads();
  load_v(0, vbuf0);
  load_k(min(1, n_kb - 1));
  {
    f32x4 sacc[4];
    score_mfma(0, sacc);
    score_softmax(0, sacc, std::true_type{});
  }
  store_k(1);
  __syncthreads();

  // ---- steady state: iteration t = value(t) + score(t+1) ---------------------
  // loads: V(t+1) into the other register set, K(t+2) into k_s[t & 1], which
  // held K(t), last read by score(t) one iteration earlier.
  auto step = [&](int t, u32x2 (&vr)[2][8], u32x2 (&vn)[2][8], auto with_score, auto masked) __attribute__((always_inline)) {
    load_v(min(t + 1, n_kb - 1), vn);
    load_k(min(t + 2, n_kb - 1));
    value_rescale(t);
    if constexpr (decltype(with_score)::value) {
      f32x4 sacc[4];
      score_mfma(t + 1, sacc);
      value_mfma(t, vr);
      score_softmax(t + 1, sacc, masked);
    } else {
      value_mfma(t, vr);
    }
    store_k(t & 1);
    __syncthreads();
  };
  auto rotate_v = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int hk = 0; hk < 2; ++hk)
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) vbuf0[hk][tt] = vbuf1[hk][tt];
  };
  // steady state: the next tile is neither the diagonal nor the ragged tail
  int t = 0;
  for (; t + 1 < n_kb - 1; ++t) {
    step(t, vbuf0, vbuf1, std::true_type{}, std::false_type{});
    rotate_v();
  }
  // the last two tiles, peeled: the next tile is masked, then value only
  if (t + 1 == n_kb - 1) {
    step(t, vbuf0, vbuf1, std::true_type{}, std::true_type{});
    rotate_v();
    ++t;
  }
  step(t, vbuf0, vbuf1, std::false_type{}, std::false_type{});

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
