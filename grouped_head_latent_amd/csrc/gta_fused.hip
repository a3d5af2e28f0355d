// GTA shared-score attention prefill, bf16 in, fp32 accumulation, gfx950:
// one instruction stream per wave, no exchange of probabilities.
//
// "GTA: Grouped-head latenT Attention" news article, grouped shared attention
// matrix mechanism: the heads of a group share one attention matrix, computed
// once and applied to the values of every head in the group.  For one group
// that is a single attention whose value is the group's heads side by side:
// NV value sources of 64 columns each (a head of d_v = 64, 128 or 256 is one,
// two or four sources), i.e. an output 64 NV columns wide.  A group with more
// than four sources is covered by several launches.
//
// A work-group is four waves and owns 128 positions of one group; wave w owns
// positions 32 w .. 32 w + 31 (two 16-row q-tiles) from scores to output, as
// the d = 128 GQA prefill kernel does:
//   S^T = K Q^T (K fragments from LDS, Q^T resident in VGPRs), an online
//   softmax with a lazily moved running maximum, and O^T += V^T P^T for all
//   64 NV output columns, with P^T straight from the score accumulator (no
//   data movement) and V^T from transposing LDS reads.  The normaliser is an
//   MFMA with an all-ones operand over the same bf16 P.
// K and V tiles of 64 keys reach LDS by buffer DMA into two buffers each (K
// one tile ahead of V); one barrier per tile.  With d_qk = 64 and four
// sources a work-group takes 80 KiB of LDS, so two share a CU (two waves per
// SIMD: one's softmax runs beside the other's matrix work).
//
// Iteration t: the softmax of tile t, then one stream of MFMA steps: the
// value steps of tile t (two contraction halves x NV sources, eight MFMAs
// each) with the score steps of tile t + 1 (d_qk / 32 of them) spread among
// them, the LDS reads of each step issued one step ahead.
//
// LDS rows, 16-byte units swizzled so that fragment reads touch distinct
// banks: K rows of 128 B keep unit u at u ^ ((r / 2) % 8), of 256 B at
// u ^ (r % 16); V rows (128 B, one source) keep unit u at u ^ 2 ((r / 2) % 4).
#include "device_common.hpp"
#include "kernels.hpp"
#include "lds_pipe.hpp"

#include <atomic>
#include <type_traits>

namespace gha {
namespace {

constexpr int KB = 64;          // keys per tile
constexpr int QT = 2;           // 16-row q-tiles per wave
constexpr int NW = 4;           // waves per work-group
constexpr int ROWS = NW * QT * 16;  // positions per work-group
constexpr int VROW = 128;       // bytes per V row of one source (64 bf16)
constexpr int VSRC = KB * VROW; // one source's V tile: 8 KiB

template <int DQK, int NV>
struct GfLayout {
  static constexpr int KROW = 2 * DQK;
  static constexpr int KTILE = KB * KROW;
  static constexpr int VTILE = NV * VSRC;
  static constexpr int KBASE = 0;
  static constexpr int VBASE = 2 * KTILE;
  static constexpr int BYTES = 2 * KTILE + 2 * VTILE;
  static constexpr int KDMA = KTILE / 1024 / NW;   // DMA instructions per wave per K tile
  static constexpr int VDMA = VTILE / 1024 / NW;   // ... per V tile (all for one source)
  static constexpr int RPD = 1024 / KROW;          // K rows per DMA instruction
  static constexpr int U = KROW / 16;              // 16-byte units per K row
};

__device__ __forceinline__ int gf_k_swz(int dqk, int r) { return dqk == 64 ? ((r >> 1) & 7) : (r & 15); }

template <int DQK, int NV, bool OUT_F32>
__global__ __launch_bounds__(64 * NW, 2) void gta_fused_kernel(PrefillArgs a) {
  using Ly = GfLayout<DQK, NV>;
  constexpr int DS = DQK / 32;        // score contraction steps
  constexpr int NCT = 4 * NV;         // 16-column output tiles
  constexpr int NPV = 2 * NV;         // value steps per tile: 2 contraction halves x NV sources
  constexpr int NSTEP = NPV + DS;
  static_assert(NV == 1 || NV == 2 || NV == 4, "value sources");
  static_assert(DQK == 64 || DQK == 128, "d_qk");
  static_assert(Ly::KDMA >= 1 && Ly::VDMA >= 1 && (Ly::VDMA * NW) % 8 == 0, "DMA split");

  __shared__ __attribute__((aligned(1024))) unsigned char smem[Ly::BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;

  // ---- which positions of which group --------------------------------------
  // Causal q-block qb walks 2 qb + 2 key tiles.  The blocks go heaviest first
  // over the whole grid (every unit's last q-block, then the one before, ...),
  // so that the dispatcher's later rounds fill in behind the heavy ones.
  const int b_id = blockIdx.x;
  if (b_id >= a.n_blocks) return;
  const int n_qb = a.n_qblocks;
  const int n_units = a.n_blocks / n_qb;
  int qb = n_qb - 1 - b_id / n_units;
  int unit = b_id % n_units;
  qb = __builtin_amdgcn_readfirstlane(qb);
  unit = __builtin_amdgcn_readfirstlane(unit);
  const int grp = __builtin_amdgcn_readfirstlane(unit % a.h_kv);
  const int b = __builtin_amdgcn_readfirstlane(unit / a.h_kv);
  const int S = a.S_q;
  const int pos0 = qb * ROWS + 16 * QT * wave;    // this wave's first position

  int k_end = S, wave_kmax = S - 1;
  if (a.causal) {
    k_end = min(S, qb * ROWS + ROWS);
    wave_kmax = min(pos0 + 16 * QT - 1, S - 1);
  }
  const int n_kb = (k_end + KB - 1) / KB;

  const __bf16* qbase = (const __bf16*)a.q + (int64_t)b * a.q_sb + (int64_t)grp * a.q_sh;
  const __bf16* kbase = (const __bf16*)a.k + (int64_t)b * a.k_sb + (int64_t)grp * a.k_sh;

  // ---- resident Q^T fragments --------------------------------------------------
  u32x4 qf[QT][DS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int pos = min(pos0 + 16 * qt + li, S - 1);
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[qt][s] = ld16(qbase + (int64_t)pos * a.q_ss + 32 * s + 8 * lg);
  }

  // ---- tile DMAs ------------------------------------------------------------------
  // K: instruction j of wave w moves rows RPD (w KDMA + j) .. + RPD - 1 (lane l:
  // row l / U, unit position l % U).  V: the waves share the NV sources, each
  // wave moving 8 VDMA rows of one source (lane l: row l / 8, position l % 8).
  // Rows past the sequence end read as zeros (buffer range check).
  const uint32_t krow = (uint32_t)a.k_ss * 2u, vrow = (uint32_t)a.v_ss * 2u;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)kbase, 0, (int)((uint32_t)(S - 1) * krow + (uint32_t)Ly::KROW), kBufferFlags);
  constexpr int WPS = 8 / Ly::VDMA;               // waves per source
  const int vsrc = wave / WPS;                    // this wave's source
  const int vn0 = (wave % WPS) * Ly::VDMA;        // its first 8-row group
  const int vhead = grp * a.v_hpg + vsrc / a.v_sph, vcol = 64 * (vsrc % a.v_sph);
  const __bf16* vbase = (const __bf16*)a.v + (int64_t)b * a.v_sb + (int64_t)vhead * a.v_sh + vcol;
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)vbase, 0, (int)((uint32_t)(S - 1) * vrow + (uint32_t)VROW), kBufferFlags);
  uint32_t kofs[Ly::KDMA];
#pragma unroll
  for (int j = 0; j < Ly::KDMA; ++j) {
    const int r = (wave * Ly::KDMA + j) * Ly::RPD + lane / Ly::U;
    kofs[j] = (uint32_t)(lane / Ly::U) * krow + 16u * ((lane % Ly::U) ^ gf_k_swz(DQK, r));
  }
  const uint32_t vofs = (uint32_t)(lane >> 3) * vrow + 16u * ((lane & 7) ^ (2 * ((lane >> 4) & 3)));
  const uint32_t lds0 = lds_offset(smem);
  auto issue_k = [&](int t) __attribute__((always_inline)) {
    const uint32_t dst = lds0 + Ly::KBASE + (t & 1) * Ly::KTILE;
#pragma unroll
    for (int j = 0; j < Ly::KDMA; ++j) {
      const int n = wave * Ly::KDMA + j;
      lds_dma16(krs, dst + n * 1024, kofs[j], (uint32_t)(t * KB + n * Ly::RPD) * krow);
    }
  };
  auto issue_v = [&](int t) __attribute__((always_inline)) {
    const uint32_t dst = lds0 + Ly::VBASE + (t & 1) * Ly::VTILE + vsrc * VSRC;
#pragma unroll
    for (int j = 0; j < Ly::VDMA; ++j) {
      const int n = vn0 + j;
      lds_dma16(vrs, dst + n * 1024, vofs, (uint32_t)(t * KB + 8 * n) * vrow);
    }
  };

  // ---- fragment addresses (bytes in smem) -------------------------------------------
  // score A operand: K row 16 kt + li, unit 4 s + lg: (kfrag ^ 64 s) + 16 KROW kt
  const uint32_t kfrag = DQK == 64 ? li * 128 + 16 * (lg ^ ((li >> 1) & 7)) : li * 256 + 16 * (lg ^ li);
  // value A operand (transposing read), source lane li of group lg: V row
  // 32 k2 + 16 h + 4 lg + li / 4 of a source, columns 16 ct + 4 (li % 4) .. + 3:
  // unit 2 ct + (li / 2) % 2, byte 8 (li % 2) of it:
  // (vfrag ^ 32 ct) + 4096 k2 + 2048 h + 8192 source
  uint32_t vfrag;
  {
    const int vr = 4 * lg + (li >> 2);
    vfrag = Ly::VBASE + vr * VROW + 32 * ((vr >> 1) & 3) + 16 * ((li >> 1) & 1) + 8 * (li & 1);
  }

  // ---- running state ------------------------------------------------------------------
  f32x4 oacc[NCT][QT], lacc[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    lacc[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) oacc[ct][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float m2[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) m2[qt] = kNegInf;
  const float c2 = a.scale * kLog2e;
  const u32x4 ones = {kBf16OnePair, kBf16OnePair, kBf16OnePair, kBf16OnePair};

  // Steps of the MFMA phase: value step p < NPV is contraction half k2 = p / NV
  // of source p % NV (its four column tiles, both q-tiles; the first source of
  // each half also adds 1^T P^T to the normaliser); score step s reads K of
  // the next tile.  The score steps sit evenly among the value steps.
  auto step_kind = [](int j) -> int {  // >= 0: value step index; < 0: score step -1 - s
    constexpr int per = NSTEP / DS;    // one score step every `per` steps
    return (j % per == per - 1 && j / per < DS) ? -1 - j / per : j - min(DS, (j + 1) / per);
  };
  f32x4 sacc[4][QT];
  u32x4 fr[2][4];
  auto load_step = [&](int j, int t, u32x4 (&f)[4]) __attribute__((always_inline)) {
    const int kind = step_kind(j);
    if (kind >= 0) {
      const int k2 = kind / NV, src = kind % NV;
      const uint32_t vb = vfrag + (t & 1) * Ly::VTILE + src * VSRC + 4096 * k2;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const unsigned char* p = smem + (vb ^ (32u * ct));
        const u32x2 h0 = ld_tr(p);
        const u32x2 h1 = ld_tr(p + 2048);
        f[ct] = u32x4{h0[0], h0[1], h1[0], h1[1]};
      }
    } else {
      const int s = -1 - kind;
      const uint32_t kb = Ly::KBASE + ((t + 1) & 1) * Ly::KTILE;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) f[kt] = ld16(smem + kb + (kfrag ^ (64u * s)) + kt * 16 * Ly::KROW);
    }
  };
  auto mfma_step = [&](int j, const u32x4 (&f)[4], const u32x4 (&pf)[QT][2]) __attribute__((always_inline)) {
    const int kind = step_kind(j);
    if (kind >= 0) {
      const int k2 = kind / NV, src = kind % NV;
      if (src == 0) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) lacc[qt] = mfma_bf16(ones, pf[qt][k2], lacc[qt]);
      }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) oacc[4 * src + ct][qt] = mfma_bf16(f[ct], pf[qt][k2], oacc[4 * src + ct][qt]);
    } else {
      const int s = -1 - kind;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          sacc[kt][qt] = mfma_bf16(f[kt], qf[qt][s], s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sacc[kt][qt]);
    }
  };
  // scores of tile 0 (prologue), from K buffer 0
  auto score0 = [&]() __attribute__((always_inline)) {
    const u32x4 nopf[QT][2] = {};
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      u32x4 f[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) f[kt] = ld16(smem + Ly::KBASE + (kfrag ^ (64u * s)) + kt * 16 * Ly::KROW);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          sacc[kt][qt] = mfma_bf16(f[kt], qf[qt][s], s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sacc[kt][qt]);
    }
    (void)nopf;
  };

  if (n_kb > 0) issue_k(0);
  if (n_kb > 0) issue_v(0);
  if (n_kb > 1) issue_k(1);
  wait_vmem_all();
  __syncthreads();
  if (n_kb > 0 && pos0 < S) score0();
  __syncthreads();  // every wave is done with K buffer 0 before tile 2 lands there

  // tiles before t_mask are fully visible to every row of the work-group
  int t_mask = S / KB;
  if (a.causal) t_mask = min(t_mask, (qb * ROWS + 1) / KB);
  t_mask = min(t_mask, n_kb);

  auto iteration = [&](int t, auto masked) __attribute__((always_inline)) {
    constexpr bool kMasked = decltype(masked)::value;
    // V(t + 1) replaces V(t - 1) and K(t + 2) replaces K(t): both were last
    // read before the previous barrier
    if (t + 1 < n_kb) issue_v(t + 1);
    if (t + 2 < n_kb) issue_k(t + 2);

    const int key0 = t * KB;
    if ((!kMasked || key0 <= wave_kmax) && pos0 < S) {  // wave-uniform
      load_step(0, t, fr[0]);  // in flight during the softmax
      __builtin_amdgcn_sched_barrier(0);
      u32x4 pf[QT][2];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        if (kMasked) {
          const int qpos = pos0 + 16 * qt + li;
          const int kmax = a.causal ? min(qpos, S - 1) : S - 1;
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (key0 + 16 * kt + 4 * lg + r > kmax) sacc[kt][qt][r] = kNegInf;
        }
        float mx = fmaxf(fmaxf(sacc[0][qt][0], sacc[0][qt][1]), sacc[0][qt][2]);
        mx = fmaxf(fmaxf(mx, sacc[0][qt][3]), sacc[1][qt][0]);
        mx = fmaxf(fmaxf(mx, sacc[1][qt][1]), sacc[1][qt][2]);
        mx = fmaxf(fmaxf(mx, sacc[1][qt][3]), sacc[2][qt][0]);
        mx = fmaxf(fmaxf(mx, sacc[2][qt][1]), sacc[2][qt][2]);
        mx = fmaxf(fmaxf(mx, sacc[2][qt][3]), sacc[3][qt][0]);
        mx = fmaxf(fmaxf(mx, sacc[3][qt][1]), sacc[3][qt][2]);
        mx = fmaxf(mx, sacc[3][qt][3]);
        const float mx2 = group4_max(mx) * c2;
        if (wave_any(mx2 > m2[qt] + kRescaleSlack)) {
          const float mnew = fmaxf(m2[qt], mx2);
          const float alpha = (mnew == kNegInf) ? 1.f : fast_exp2(m2[qt] - mnew);
          m2[qt] = mnew;
          lacc[qt] *= alpha;
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) oacc[ct][qt] *= alpha;
        }
        const float msub = (m2[qt] == kNegInf) ? 0.f : m2[qt];
        float p[4][4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) p[kt][r] = fast_exp2(__builtin_fmaf(sacc[kt][qt][r], c2, -msub));
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
          pf[qt][k2] = u32x4{pack_bf16(p[2 * k2][0], p[2 * k2][1]), pack_bf16(p[2 * k2][2], p[2 * k2][3]),
                             pack_bf16(p[2 * k2 + 1][0], p[2 * k2 + 1][1]),
                             pack_bf16(p[2 * k2 + 1][2], p[2 * k2 + 1][3])};
      }

      __builtin_amdgcn_s_setprio(1);
      // P(t) V(t) and the scores of tile t + 1; past the last tile those read
      // a stale K buffer and are never used
#pragma unroll
      for (int j = 0; j < NSTEP; ++j) {
        if (j + 1 < NSTEP) load_step(j + 1, t, fr[(j + 1) & 1]);
        mfma_step(j, fr[j & 1], pf);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
    }

    wait_vmem_all();
    __syncthreads();
  };
  for (int t = 0; t < t_mask; ++t) iteration(t, std::false_type{});
  for (int t = t_mask; t < n_kb; ++t) iteration(t, std::true_type{});

  // ---- epilogue: O = O^T / l per source; lse per group --------------------------------
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int pos = pos0 + 16 * qt + li;
    if (pos >= S) continue;
    const float l = lacc[qt][0];
    const float inv = 1.f / l;
    if (a.lse != nullptr && lg == 0)
      a.lse[((int64_t)b * a.lse_heads + grp) * S + pos] = (m2[qt] + fast_log2(l)) * kLn2;
#pragma unroll
    for (int src = 0; src < NV; ++src) {
      const int head = grp * a.v_hpg + src / a.v_sph;
      const int64_t obase =
          (int64_t)b * a.o_sb + (int64_t)head * a.o_sh + (int64_t)pos * a.o_ss + 64 * (src % a.v_sph) + 4 * lg;
      // oacc[4 src + ct][qt][r] is column 16 ct + 4 lg + r of the source
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const f32x4 v = oacc[4 * src + ct][qt] * inv;
        if constexpr (OUT_F32)
          *reinterpret_cast<f32x4*>((float*)a.o + obase + 16 * ct) = v;
        else
          *reinterpret_cast<u32x2*>((__bf16*)a.o + obase + 16 * ct) = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
      }
    }
  }
}

template <int DQK, int NV>
hipError_t launch_nv(const PrefillArgs& args, bool out_f32, hipStream_t st) {
  const uint32_t grid = (uint32_t)args.n_blocks;
  if (out_f32)
    hipLaunchKernelGGL((gta_fused_kernel<DQK, NV, true>), dim3(grid), dim3(64 * NW), 0, st, args);
  else
    hipLaunchKernelGGL((gta_fused_kernel<DQK, NV, false>), dim3(grid), dim3(64 * NW), 0, st, args);
  return hipGetLastError();
}

}  // namespace

static_assert(ROWS == 128, "both GTA kernels take 128 positions per work-group");

hipError_t launch_gta_fused(const PrefillArgs& a, int d_qk, int sources, bool out_f32, hipStream_t st) {
#define GHA_GF_CASE(DQ, NVV) \
  if (d_qk == DQ && sources == NVV) return launch_nv<DQ, NVV>(a, out_f32, st);
  GHA_GF_CASE(64, 4)
  GHA_GF_CASE(64, 2)
  GHA_GF_CASE(64, 1)
  GHA_GF_CASE(128, 4)
  GHA_GF_CASE(128, 2)
  GHA_GF_CASE(128, 1)
#undef GHA_GF_CASE
  return hipErrorInvalidValue;
}

}  // namespace gha
