// GTA shared-score attention prefill, bf16 in, fp32 accumulation, gfx950.
//
// "GTA: Grouped-head latenT Attention" news article, grouped shared attention
// matrix mechanism: the heads of a group share one attention matrix, computed
// once and applied to the values of every head in the group.  Per group there
// is one query and one key (d_qk wide) and one value per head (d_v wide).
// The kernel applies the scores to H value sources of 64 columns each
// (a head of d_v = 128 or 256 is two or four sources); a group with more than
// four sources is covered by several launches, each recomputing the scores.
//
// One work-group (eight waves, two per SIMD) owns 128 positions of one group
// and walks the keys in tiles of 64.  Its waves split the work by role:
//   score waves 0..3: wave w computes S^T = K Q^T for positions 32 w ..
//          32 w + 31 (K from LDS, Q^T resident in VGPRs), runs their softmax
//          and publishes the bf16 probabilities as P^T operand fragments in
//          LDS;
//   value waves 4..7: they split the value sources (with four sources, wave
//          4 + h takes source h for all 128 positions) and accumulate
//          O^T += V^T P^T: V^T fragments come from transposing LDS reads of
//          the source's V tile, P^T fragments from LDS, one tile behind.
// So the score matrix is computed once per group, every K or V tile is
// fetched once per work-group, K is read by four waves and each V tile by one.
// Wave w and wave w + 4 share a SIMD, so one's softmax runs beside the
// other's value MFMAs.
//
// Tiles reach LDS by buffer DMA (buffer_load ... lds, no VGPR staging) into
// rings of NS slots: the DMAs of an iteration fetch the K tile NS - 1 ahead of
// the one being scored and the V tile NS - 2 ahead of the one being applied.
// Rows past the sequence end read as zeros (buffer range check).
//
// Softmax against a fixed reference: each position's reference m (log2 units)
// is the maximum of its first tile (key 0 is always visible), so the
// accumulators never need rescaling and the value waves can use any
// position's probabilities without its statistics.  A tile whose maximum
// exceeds m by more than kSlack (2^96 stays far inside bf16 and fp32 range)
// makes the work-group start again with the larger reference; the result is
// the same softmax either way.
//
// Iteration it: the score waves score tile it and publish P^T(it); the value
// waves apply P^T(it - 1) to V(it - 1); one barrier.  The iteration is bound
// by LDS throughput: per iteration and CU the LDS moves about 184 KiB (K, V^T
// and P^T reads, P^T and DMA writes).  Each role runs a loop of its own with
// its epilogue inside, so that neither keeps the other's registers live and
// no accumulator outlives the loop.
//
// Unspecialised form (SPEC = false, built with GHA_GTA_SPEC=0): every wave
// scores 16 positions and applies one source to 64 positions, the softmax of
// tile it woven between its value MFMAs of tile it - 1; the LDS then moves
// about 248 KiB per iteration and CU, and the iteration takes ~12% longer.
//
// LDS rows, 16-byte units swizzled so that every fragment read touches
// distinct banks:
//   K row r (d_qk = 64: 8 units) keeps unit u at u ^ ((r / 2) % 8); score
//     reads (16 rows, one unit) then cover all 16 positions of a 256 B window;
//     (d_qk = 128: 16 units) unit u at u ^ (r % 16).
//   V row r (8 units) keeps unit u at u ^ 2 ((r / 2) % 4); a transposing read
//     of one half-wave takes 32 B from each of 8 consecutive rows, which then
//     land on 8 distinct 32 B bank groups.
#include "device_common.hpp"
#include "kernels.hpp"
#include "lds_pipe.hpp"

namespace gha {
namespace {

constexpr int KB = 64;                  // keys per tile
constexpr int ROWS = 128;               // positions per work-group
constexpr int VROW = 128;               // bytes per V row (64 bf16)
constexpr int VHEAD = KB * VROW;        // one head's V tile: 8 KiB
constexpr int PFRAG = 1024;             // one P^T operand fragment: 64 lanes x 16 B
constexpr int PBUF = 16 * PFRAG;        // P^T of 8 row tiles x 2 contraction steps
constexpr float kSlack = 96.f;
constexpr int NW = 8;                   // waves per work-group

template <int DQK, int H, bool SPEC>
struct GtaLayout {
  static constexpr int KROW = 2 * DQK;          // bytes per K row
  static constexpr int KTILE = KB * KROW;
  static constexpr int VTILE = H * VHEAD;
  // ring slots: three when they fit (two tiles in flight), else two
  static constexpr int NS = (3 * (KTILE + VTILE) + 2 * PBUF <= 152 * 1024) ? 3 : 2;
  static constexpr int KBASE = 0;
  static constexpr int VBASE = NS * KTILE;
  static constexpr int PBASE = VBASE + NS * VTILE;
  static constexpr int STATS = PBASE + 2 * PBUF;  // 128 floats, then 2 x 8 restart flags
  static constexpr int FLAGS = STATS + 4 * ROWS;
  static constexpr int BYTES = FLAGS + 16;
  // DMA instructions per wave per K tile (by the score waves) and per V
  // tile (by the value waves); every wave does both unless specialised
  static constexpr int KDMA = KTILE / 1024 / (SPEC ? NW / 2 : NW);
  static constexpr int VDMA = VTILE / 1024 / (SPEC ? NW / 2 : NW);
  static constexpr int RPD = 1024 / KROW;         // K rows per DMA instruction
};

__host__ __device__ constexpr int k_swz(int dqk, int r) { return dqk == 64 ? ((r >> 1) & 7) : (r & 15); }
// a pointer that is the same in every lane, kept in scalar registers (the
// buffer descriptors built from it are scalar operands)
template <typename P>
__device__ __forceinline__ P* uniform_ptr(P* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (P*)(((uint64_t)hi << 32) | lo);
}

template <int DQK, int H, bool OUT_F32, bool SPEC>
__global__ __launch_bounds__(64 * NW, 1) void gta_kernel(PrefillArgs a) {
  using Ly = GtaLayout<DQK, H, SPEC>;
  constexpr int DS = DQK / 32;      // score contraction steps
  constexpr int NSW = SPEC ? NW / 2 : NW;  // score waves
  constexpr int NVW = SPEC ? NW / 2 : NW;  // value waves
  constexpr int QT = ROWS / (16 * NSW);    // 16-position score tiles per score wave
  constexpr int HW = NVW / H;       // value waves per head
  constexpr int RT = 8 / HW;        // row tiles per value wave
  constexpr int NB = 8 * RT;        // value MFMAs per tile: 2 steps x 4 column tiles x RT
  constexpr int NBS = 3 * NB / 4;   // the softmax shares the first NBS of them (unspecialised)
  constexpr int U = Ly::KROW / 16;  // 16-byte units per K row
  constexpr int NS = Ly::NS;
  static_assert(H == 1 || H == 2 || H == 4, "value sources per work-group");
  static_assert(QT == 1 || QT == 2, "score tiles per wave");
  static_assert(RT == 1 || RT == 2 || RT == 4 || RT == 8, "row tiles per wave");
  static_assert(Ly::KDMA >= 1 && Ly::KDMA <= DS && Ly::VDMA >= 1 && NB % Ly::VDMA == 0, "DMA slots");
  static_assert(Ly::BYTES <= 160 * 1024, "LDS");

  __shared__ __attribute__((aligned(1024))) unsigned char smem[Ly::BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  // roles (wave-uniform): every wave scores and applies values unless specialised
  const bool scorer = !SPEC || wave < NSW;
  const bool valuer = !SPEC || wave >= NW - NVW;
  const int sw = SPEC ? min(wave, NSW - 1) : wave;         // index among the score waves
  const int vw = SPEC ? max(wave - (NW - NVW), 0) : wave;  // ... among the value waves

  // ---- which positions of which group -----------------------------------------
  // Work-groups start in blockIdx order as CUs free up, and causal q-blocks
  // differ in work (q-block qb walks 2 qb + 2 key tiles), with only about
  // two work-groups per CU: number them heaviest first (every (batch, group)
  // of the last q-block, then of the one before, ...), so that light blocks
  // fill in behind heavy ones instead of two heavy ones meeting on one CU.
  const uint32_t lid = blockIdx.x;
  if (lid >= (uint32_t)a.n_blocks) return;
  const int n_qb = a.n_qblocks;
  const int n_bg = a.B * a.h_kv;
  const int qb = __builtin_amdgcn_readfirstlane(n_qb - 1 - (int)(lid / n_bg));
  const int grp = __builtin_amdgcn_readfirstlane((int)(lid % n_bg) % a.h_kv);
  const int b = __builtin_amdgcn_readfirstlane((int)(lid % n_bg) / a.h_kv);
  const int S = a.S_q;
  const int pos_wg = qb * ROWS;
  const int hv = vw / HW;          // value phase: head hv of the group
  const int rt0 = (vw % HW) * RT;  //   and its first row tile

  // tiles to visit; tiles from t_mask on need the mask (diagonal or ragged)
  int n_kb, t_mask;
  if (a.causal) {
    n_kb = (min(S, pos_wg + ROWS) + KB - 1) / KB;
    t_mask = min((pos_wg + 1) / KB, S / KB);
  } else {
    n_kb = (S + KB - 1) / KB;
    t_mask = S / KB;
  }
  n_kb = __builtin_amdgcn_readfirstlane(n_kb);
  t_mask = __builtin_amdgcn_readfirstlane(min(t_mask, n_kb));

  const __bf16* qbase = (const __bf16*)a.q + (int64_t)b * a.q_sb + (int64_t)grp * a.q_sh;
  const __bf16* kbase = uniform_ptr((const __bf16*)a.k + (int64_t)b * a.k_sb + (int64_t)grp * a.k_sh);
  // value source hv: columns 64 (hv % v_sph) .. + 63 of head grp v_hpg + hv / v_sph
  const int vhead = grp * a.v_hpg + hv / a.v_sph, vcol = 64 * (hv % a.v_sph);
  const __bf16* vbase = uniform_ptr((const __bf16*)a.v + (int64_t)b * a.v_sb + (int64_t)vhead * a.v_sh + vcol);

  // ---- Q^T fragments of this wave's score rows ----------------------------------
  u32x4 qf[QT][DS];
  int kmax[QT];  // last key each lane's row sees
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int pos = pos_wg + 16 * (QT * sw + qt) + li;
    const int pc = min(pos, S - 1);
    kmax[qt] = a.causal ? pc : S - 1;
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[qt][s] = ld16(qbase + (int64_t)pc * a.q_ss + 32 * s + 8 * lg);
  }
  wait_vmem_all();
  const float c2 = a.scale * kLog2e;

  // ---- tile DMAs -----------------------------------------------------------------
  // K: score wave w moves rows RPD (w KDMA + j) .. + RPD - 1 with its j-th
  // instruction (lane l: row l / U, unit position l % U).  V: value wave w
  // moves rows 8 n .. 8 n + 7 of its value head with instruction j,
  // n = (w VDMA + j) mod 8 (lane l: row l / 8, position l % 8).  Offsets of
  // tiles past the last read as zeros.
  const uint32_t krow = (uint32_t)a.k_ss * 2u, vrow = (uint32_t)a.v_ss * 2u;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)kbase, 0, (int)((uint32_t)(S - 1) * krow + (uint32_t)Ly::KROW), kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)vbase, 0, (int)((uint32_t)(S - 1) * vrow + (uint32_t)VROW), kBufferFlags);
  uint32_t kofs[Ly::KDMA];
#pragma unroll
  for (int j = 0; j < Ly::KDMA; ++j) {
    const int r = (sw * Ly::KDMA + j) * Ly::RPD + lane / U;
    kofs[j] = (uint32_t)(lane / U) * krow + 16u * ((lane % U) ^ k_swz(DQK, r));
  }
  const uint32_t vofs = (uint32_t)(lane >> 3) * vrow + 16u * ((lane & 7) ^ (2 * ((lane >> 4) & 3)));
  const uint32_t lds0 = lds_offset(smem);
  auto issue_k = [&](int t, int j) __attribute__((always_inline)) {
    const int n = sw * Ly::KDMA + j;
    const uint32_t so = t < n_kb ? (uint32_t)(t * KB + n * Ly::RPD) * krow : kOutOfRange;
    lds_dma16(krs, lds0 + Ly::KBASE + (t % NS) * Ly::KTILE + n * 1024, kofs[j], so);
  };
  auto issue_v = [&](int t, int j) __attribute__((always_inline)) {
    const int n = (vw * Ly::VDMA + j) & 7;
    const uint32_t so = t < n_kb ? (uint32_t)(t * KB + 8 * n) * vrow : kOutOfRange;
    lds_dma16(vrs, lds0 + Ly::VBASE + (t % NS) * Ly::VTILE + hv * VHEAD + n * 1024, vofs, so);
  };

  // ---- fragment addresses (bytes in smem) -------------------------------------------
  // score A operand: K row 16 kt + li, unit 4 s + lg:
  //   (kfrag ^ 64 s) + 16 KROW kt
  const uint32_t kfrag = DQK == 64 ? li * 128 + 16 * (lg ^ ((li >> 1) & 7)) : li * 256 + 16 * (lg ^ li);
  // value A operand (transposing read), source lane li of group lg: V row
  // 32 ks + 16 h + 4 lg + li / 4, columns 16 ct + 4 (li % 4) .. + 3, i.e. unit
  // 2 ct + (li / 2) % 2, byte 8 (li % 2) of it: (vfrag ^ 32 ct) + 4096 ks + 2048 h
  uint32_t vfrag;
  {
    const int vr = 4 * lg + (li >> 2);
    vfrag = vr * VROW + 32 * ((vr >> 1) & 3) + 16 * ((li >> 1) & 1) + 8 * (li & 1);
  }
  const uint32_t plane = 16 * lane;  // P^T fragments are lane-linear
  uint32_t vfr[4];                   // transposing-read lane offsets of the 4 column tiles
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) vfr[ct] = vfrag ^ (32u * ct);

  // ---- running state ----------------------------------------------------------------
  f32x4 oacc[4][RT];  // O^T: [column tile][row tile] (AGPRs)
  f32x4 lacc[QT];     // normaliser of this wave's score rows
  float m2[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) m2[qt] = kNegInf;
  // P^T fragments [contraction step][row tile]; with d_qk = 128 (more score
  // registers) one set is reloaded between the steps instead
  constexpr int NPB = DS == 4 ? 1 : 2;
  u32x4 pall[NPB][RT];
  u32x4 vf[2];        // V^T fragment, double-buffered across value steps
  uint64_t flags = 0; // restart requests (one byte per wave) read after the last barrier
  unsigned char* const flag_s = smem + Ly::FLAGS;

  // The accumulators are written by inline-asm MFMAs, which the compiler's
  // hazard checks do not see: before any other instruction may touch the
  // last value steps' accumulators (the compiler may insert copies at the end
  // of an iteration), those MFMAs must retire.  The nops are tied to them.
  auto value_retire = [&]() __attribute__((always_inline)) {
#define GHA_RETIRE "s_nop 7\n\ts_nop 7\n\ts_nop 3"
    if constexpr (SPEC) {
      // accumulators in VGPRs (see the value MFMAs of the specialised form)
      if constexpr (RT == 2)
        asm volatile(GHA_RETIRE : "+v"(oacc[3][0]), "+v"(oacc[3][RT - 1]), "+v"(oacc[2][0]), "+v"(oacc[2][RT - 1]));
      if constexpr (RT == 4)
        asm volatile(GHA_RETIRE : "+v"(oacc[3][0]), "+v"(oacc[3][1]), "+v"(oacc[3][2]), "+v"(oacc[3][RT - 1]));
      if constexpr (RT == 8)
        asm volatile(GHA_RETIRE : "+v"(oacc[3][0]), "+v"(oacc[3][1]), "+v"(oacc[3][2]), "+v"(oacc[3][3]),
                     "+v"(oacc[3][4]), "+v"(oacc[3][5]), "+v"(oacc[3][6]), "+v"(oacc[3][RT - 1]));
      return;
    }
    if constexpr (RT == 1) asm volatile(GHA_RETIRE : "+a"(oacc[3][0]), "+a"(oacc[2][0]), "+a"(oacc[1][0]));
    if constexpr (RT == 2)
      asm volatile(GHA_RETIRE : "+a"(oacc[3][0]), "+a"(oacc[3][RT - 1]), "+a"(oacc[2][0]), "+a"(oacc[2][RT - 1]));
    if constexpr (RT == 4)
      asm volatile(GHA_RETIRE : "+a"(oacc[3][0]), "+a"(oacc[3][1]), "+a"(oacc[3][2]), "+a"(oacc[3][RT - 1]));
#undef GHA_RETIRE
  };

  // Roles as compile-time constants: 0 every wave does both (unspecialised),
  // 1 score waves, 2 value waves.  The specialised roles run loops of their
  // own, so that neither keeps the other's registers live.
  using Both = std::integral_constant<int, 0>;
  using Scorer = std::integral_constant<int, 1>;
  using Valuer = std::integral_constant<int, 2>;
  // wait until at most one iteration's DMAs of this wave (NS - 2 tiles of them) are in flight
  auto wait_this_iteration_dmas = [&](auto role) __attribute__((always_inline)) {
    constexpr int kRole = decltype(role)::value;
    if constexpr (kRole == 0) wait_vmem_at_most<(Ly::KDMA + Ly::VDMA) * (NS - 2)>();
    if constexpr (kRole == 1) wait_vmem_at_most<Ly::KDMA * (NS - 2)>();
    if constexpr (kRole == 2) wait_vmem_at_most<Ly::VDMA * (NS - 2)>();
  };

  auto iter = [&](int it, auto masked, auto has_score, auto has_pv, auto role) __attribute__((always_inline)) -> bool {
    constexpr bool kMasked = decltype(masked)::value;
    constexpr bool kS = decltype(has_score)::value;
    constexpr bool kP = decltype(has_pv)::value;
    constexpr int kRole = decltype(role)::value;
    const int k0 = it * KB;
    // slot bases of this iteration, kept opaque so that each fragment address
    // is one add of a scalar to a loop-invariant lane offset
    uint32_t kb_ = Ly::KBASE + (uint32_t)(it % NS) * Ly::KTILE;
    uint32_t vb_ = Ly::VBASE + (uint32_t)((it + NS - 1) % NS) * Ly::VTILE + hv * VHEAD;
    uint32_t pr_ = Ly::PBASE + (uint32_t)((it + 1) & 1) * PBUF;  // P^T of tile it - 1
    asm volatile("" : "+s"(kb_), "+s"(vb_), "+s"(pr_));
    const int dk = it + NS - 1, dv = it + NS - 2;  // tiles whose DMAs this iteration issues

    auto load_v = [&](int step, u32x4& v) __attribute__((always_inline)) {
      const unsigned char* p = smem + vb_ + vfr[step & 3] + 4096 * (step >> 2);
      const u32x2 h0 = ld_tr(p);
      const u32x2 h1 = ld_tr(p + 2048);
      v = u32x4{h0[0], h0[1], h1[0], h1[1]};
    };
    auto load_p = [&](int ks) __attribute__((always_inline)) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) pall[ks % NPB][rt] = ld16(smem + pr_ + plane + (2 * (rt0 + rt) + ks) * PFRAG);
    };

    // ---- phase A: S^T of tile it for this wave's rows ----
    f32x4 sacc[4][QT];
    auto phase_a = [&]() __attribute__((always_inline)) {
    if constexpr (kS) {
      u32x4 kf[2][4];
      auto load_k = [&](int s, u32x4 (&f)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) f[kt] = ld16(smem + kb_ + kt * 16 * Ly::KROW + (kfrag ^ (64u * s)));
      };
      load_k(0, kf[0]);
      static_for<0, DS>([&](auto S_) __attribute__((always_inline)) {
        constexpr int s = decltype(S_)::value;
        if (s + 1 < DS) load_k(s + 1, kf[(s + 1) & 1]);
        if (s < Ly::KDMA) issue_k(dk, s);
        if (!SPEC && kP && s == DS - 1) {
          load_p(0);
          load_v(0, vf[0]);
        }
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) {
            if (s == 0) mfma_v0(sacc[kt][qt], kf[s & 1][kt], qf[qt][s]);
            else mfma_v(sacc[kt][qt], kf[s & 1][kt], qf[qt][s]);
          }
        __builtin_amdgcn_sched_barrier(0);
      });
    } else {
#pragma unroll
      for (int j = 0; j < Ly::KDMA; ++j) issue_k(dk, j);
      load_p(0);
      load_v(0, vf[0]);
    }
    };

    // ---- phase B: softmax of tile it in 23 small stages per score row (=
    // lane and q-tile); sacc[kt][qt][r] is key k0 + 16 kt + 4 lg + r and
    // becomes its probability in place ----
    float mx[QT], msub[QT];
    u32x4 pf[QT][2];
    bool restart_row = false;
    constexpr int NSQ = 23, NST = QT * NSQ;
    auto stage = [&](auto K_) __attribute__((always_inline)) {
      constexpr int k = decltype(K_)::value;
      constexpr int qt = k / NSQ, st = k % NSQ;
      if constexpr (st < 4) {
        if constexpr (kMasked) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (k0 + 16 * st + 4 * lg + r > kmax[qt]) sacc[st][qt][r] = kNegInf;
        }
      } else if constexpr (st == 4 || st == 5) {
        constexpr int kt = 2 * (st - 4);
        float x = fmaxf(fmaxf(sacc[kt][qt][0], sacc[kt][qt][1]), fmaxf(sacc[kt][qt][2], sacc[kt][qt][3]));
        x = fmaxf(x, fmaxf(fmaxf(sacc[kt + 1][qt][0], sacc[kt + 1][qt][1]), fmaxf(sacc[kt + 1][qt][2], sacc[kt + 1][qt][3])));
        mx[qt] = st == 4 ? x : fmaxf(mx[qt], x);
      } else if constexpr (st == 6) {
        mx[qt] = xor16_max(mx[qt]);
      } else if constexpr (st == 7) {
        mx[qt] = xor32_max(mx[qt]) * c2;
      } else if constexpr (st == 8) {
        // the first tile fixes a row's reference; a tile that outgrows it by
        // more than the slack asks for a restart
        const bool first = m2[qt] == kNegInf;
        const bool grow = !first && mx[qt] > m2[qt] + kSlack;
        restart_row = restart_row || grow;
        m2[qt] = (first || grow) ? mx[qt] : m2[qt];
        msub[qt] = (m2[qt] == kNegInf) ? 0.f : m2[qt];
      } else if constexpr (st >= 9 && st <= 12) {
        constexpr int kt = st - 9;
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[kt][qt][r] = __builtin_fmaf(sacc[kt][qt][r], c2, -msub[qt]);
      } else if constexpr (st >= 13 && st <= 20) {
        constexpr int kt = (st - 13) / 2, r0 = 2 * ((st - 13) % 2);
        sacc[kt][qt][r0] = fast_exp2(sacc[kt][qt][r0]);
        sacc[kt][qt][r0 + 1] = fast_exp2(sacc[kt][qt][r0 + 1]);
      } else {
        constexpr int ks = st - 21;
        pf[qt][ks] = u32x4{pack_bf16(sacc[2 * ks][qt][0], sacc[2 * ks][qt][1]),
                           pack_bf16(sacc[2 * ks][qt][2], sacc[2 * ks][qt][3]),
                           pack_bf16(sacc[2 * ks + 1][qt][0], sacc[2 * ks + 1][qt][1]),
                           pack_bf16(sacc[2 * ks + 1][qt][2], sacc[2 * ks + 1][qt][3])};
      }
    };
    // the score MFMAs must retire before the softmax reads their results
    // (the nops are tied to every score register so that no read moves above them)
    auto scores_retire = [&]() __attribute__((always_inline)) {
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
                   : "+v"(sacc[0][0]), "+v"(sacc[1][0]), "+v"(sacc[2][0]), "+v"(sacc[3][0]));
      if constexpr (QT == 2)
        asm volatile("" : "+v"(sacc[0][QT - 1]), "+v"(sacc[1][QT - 1]), "+v"(sacc[2][QT - 1]), "+v"(sacc[3][QT - 1]));
    };
    // P^T of this wave's rows to LDS with their normaliser (two wait states
    // after the VALU writes of the MFMA operands, accumulator included), and
    // the restart request
    auto publish = [&]() __attribute__((always_inline)) {
      u32x4 ones = {kBf16OnePair, kBf16OnePair, kBf16OnePair, kBf16OnePair};
      if constexpr (QT == 1) asm volatile("s_nop 1" : "+v"(pf[0][0]), "+v"(pf[0][1]), "+v"(lacc[0]), "+v"(ones));
      if constexpr (QT == 2)
        asm volatile("s_nop 1" : "+v"(pf[0][0]), "+v"(pf[0][1]), "+v"(pf[QT - 1][0]), "+v"(pf[QT - 1][1]),
                     "+v"(lacc[0]), "+v"(lacc[QT - 1]), "+v"(ones));
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) mfma_v(lacc[qt], ones, pf[qt][ks]);
      unsigned char* pw = smem + Ly::PBASE + (it & 1) * PBUF + 16 * lane;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) st16(pw + (2 * (QT * sw + qt) + ks) * PFRAG, pf[qt][ks]);
      // a wave whose rows outgrew their reference asks the whole work-group to
      // start again (every wave must run the same tiles and barriers)
      const bool any_restart = wave_any(restart_row);  // all lanes vote, outside the lane-0 branch
      if (lane == 0) flag_s[NW * (it & 1) + wave] = any_restart ? 1 : 0;
    };
    // the same per score tile (specialised form): tile qt's P^T goes to LDS as
    // soon as its softmax is done, so that its writes drain while the next
    // tile's softmax runs (the value waves' reads keep the LDS busy)
    auto publish_qt = [&](auto Q_) __attribute__((always_inline)) {
      constexpr int qt = decltype(Q_)::value;
      u32x4 ones = {kBf16OnePair, kBf16OnePair, kBf16OnePair, kBf16OnePair};
      asm volatile("s_nop 1" : "+v"(pf[qt][0]), "+v"(pf[qt][1]), "+v"(lacc[qt]), "+v"(ones));
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) mfma_v(lacc[qt], ones, pf[qt][ks]);
      unsigned char* pw = smem + Ly::PBASE + (it & 1) * PBUF + 16 * lane;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) st16(pw + (2 * (QT * sw + qt) + ks) * PFRAG, pf[qt][ks]);
      if constexpr (qt == QT - 1) {
        const bool any_restart = wave_any(restart_row);  // all lanes vote, outside the lane-0 branch
        if (lane == 0) flag_s[NW * (it & 1) + wave] = any_restart ? 1 : 0;
      }
    };

    if constexpr (kRole != 0) {
      if constexpr (kRole == 1) {
        if constexpr (kS) {
          phase_a();
          scores_retire();
          static_for<0, NST>([&](auto K_) __attribute__((always_inline)) {
            constexpr int k = decltype(K_)::value;
            stage(K_);
            if constexpr (k % NSQ == NSQ - 1) publish_qt(std::integral_constant<int, k / NSQ>{});
          });
        } else {
#pragma unroll
          for (int j = 0; j < Ly::KDMA; ++j) issue_k(dk, j);
        }
      }
      if constexpr (kRole == 2) {
        if constexpr (kP) {
          load_p(0);
          load_v(0, vf[0]);
          // O^T += V^T P^T of tile it - 1 (as below, without the softmax)
          static_for<0, NB>([&](auto M_) __attribute__((always_inline)) {
            constexpr int m = decltype(M_)::value;
            constexpr int step = m / RT, rt = m % RT, ks = step / 4, ct = step % 4;
            if (rt == 0 && step + 1 < 8) load_v(step + 1, vf[(step + 1) & 1]);
            if (NPB == 2 && m == 1) load_p(1);
            if (m % (NB / Ly::VDMA) == NB / Ly::VDMA / 2) issue_v(dv, m / (NB / Ly::VDMA));
            // accumulators in VGPRs: without AGPRs in use the compiler can give
            // either role up to 256 registers (with 128 AGPRs of accumulators it
            // splits them 128 / 128 and the score role spills)
            mfma_v(oacc[ct][rt], vf[step & 1], pall[ks % NPB][rt]);
            if (NPB == 1 && m == 4 * RT - 1) load_p(1);
            __builtin_amdgcn_sched_barrier(0);
          });
          value_retire();
        } else {
#pragma unroll
          for (int j = 0; j < Ly::VDMA; ++j) issue_v(dv, j);
        }
      }
    } else {
      phase_a();
      if constexpr (kP) {
        // O^T += V^T P^T of tile it - 1: step = 4 ks + ct, RT MFMAs per step
        static_for<0, NB>([&](auto M_) __attribute__((always_inline)) {
          constexpr int m = decltype(M_)::value;
          constexpr int step = m / RT, rt = m % RT, ks = step / 4, ct = step % 4;
          if (rt == 0 && step + 1 < 8) load_v(step + 1, vf[(step + 1) & 1]);
          if (NPB == 2 && m == 1) load_p(1);
          if (m % (NB / Ly::VDMA) == NB / Ly::VDMA / 2) issue_v(dv, m / (NB / Ly::VDMA));
          mfma_acc(oacc[ct][rt], vf[step & 1], pall[ks % NPB][rt]);
          // a single set of P^T fragments is refilled once its last reader has issued
          if (NPB == 1 && m == 4 * RT - 1) load_p(1);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (kS) {
            if (m == 0) scores_retire();
            if constexpr (m < NBS) static_for<m * NST / NBS, (m + 1) * NST / NBS>(stage);
            if (m == NBS) publish();
          }
          __builtin_amdgcn_sched_barrier(0);
        });
        value_retire();
      } else {
        scores_retire();
        static_for<0, NST>(stage);
  #pragma unroll
        for (int j = 0; j < Ly::VDMA; ++j) issue_v(dv, j);
        publish();
      }
    }

    // a restart raised at the previous barrier: nothing since is kept
    if (__builtin_amdgcn_readfirstlane((uint32_t)(flags | (flags >> 32))) != 0) return true;
    // the tiles of the next iteration have landed (this one's DMAs may fly on)
    wait_this_iteration_dmas(role);
    __syncthreads();
    if constexpr (kS) flags = *reinterpret_cast<const uint64_t*>(flag_s + NW * (it & 1));
    return false;
  };

  // run(role, done): the tile loop of a role, restarted until no wave asks for
  // it, then done() (the role's epilogue) inside the loop, so that no
  // accumulator lives on past the loop's exit
  auto run = [&](auto role, auto&& done) __attribute__((always_inline)) {
    constexpr int kRole = decltype(role)::value;
    for (;;) {
      if constexpr (kRole != 2) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) lacc[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      if constexpr (kRole != 1) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) oacc[ct][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      flags = 0;
      // K of tiles 0 .. NS - 2 and V of tiles 0 .. NS - 3, in that order
      if constexpr (kRole != 2) {
#pragma unroll
        for (int t = 0; t < NS - 1; ++t)
#pragma unroll
          for (int j = 0; j < Ly::KDMA; ++j) issue_k(t, j);
      }
      if constexpr (kRole != 1) {
#pragma unroll
        for (int t = 0; t < NS - 2; ++t)
#pragma unroll
          for (int j = 0; j < Ly::VDMA; ++j) issue_v(t, j);
      }
      // a value wave never publishes a restart request: its flag bytes stay zero
      if (lane == 0) {
        flag_s[wave] = 0;
        flag_s[NW + wave] = 0;
      }
      wait_this_iteration_dmas(role);
      __syncthreads();
      bool restart = t_mask > 0 ? iter(0, std::false_type{}, std::true_type{}, std::false_type{}, role)
                                : iter(0, std::true_type{}, std::true_type{}, std::false_type{}, role);
      int it = 1;
      for (; it < t_mask && !restart; ++it)
        restart = iter(it, std::false_type{}, std::true_type{}, std::true_type{}, role);
      for (; it < n_kb && !restart; ++it)
        restart = iter(it, std::true_type{}, std::true_type{}, std::true_type{}, role);
      if (!restart) restart = iter(n_kb, std::false_type{}, std::false_type{}, std::true_type{}, role);
      // no DMA may still target a slot that is about to be reused
      wait_vmem_all();
      if (!restart) {
        done();
        return;
      }
      __syncthreads();
    }
  };

  // ---- epilogue: 1 / l of every row through LDS, then O = O^T / l ------------------
  float* stats = reinterpret_cast<float*>(smem + Ly::STATS);
  auto write_stats = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float l = lacc[qt][0];
      const int row = 16 * (QT * sw + qt) + li;
      const int pos = pos_wg + row;
      if (lg == 0) {
        stats[row] = 1.f / l;
        if (a.lse != nullptr && pos < S)
          a.lse[((int64_t)b * a.lse_heads + grp) * S + pos] = (m2[qt] + fast_log2(l)) * kLn2;
      }
    }
  };
  auto write_outputs = [&]() __attribute__((always_inline)) {
  #pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row = 16 * (rt0 + rt) + li;
      const int pos = pos_wg + row;
      if (pos >= S) continue;
      const float inv = stats[row];
      const int64_t obase = (int64_t)b * a.o_sb + (int64_t)vhead * a.o_sh + (int64_t)pos * a.o_ss + vcol + 4 * lg;
      // oacc[ct][rt][r] is feature 16 ct + 4 lg + r of this row
  #pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const f32x4 v = oacc[ct][rt] * inv;
        if constexpr (OUT_F32)
          *reinterpret_cast<f32x4*>((float*)a.o + obase + 16 * ct) = v;
        else
          *reinterpret_cast<u32x2*>((__bf16*)a.o + obase + 16 * ct) = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
      }
    }
  };
  if constexpr (SPEC) {
    if (scorer) {
      run(Scorer{}, [&]() __attribute__((always_inline)) {
        write_stats();
        __syncthreads();
      });
    } else {
      run(Valuer{}, [&]() __attribute__((always_inline)) {
        __syncthreads();
        write_outputs();
      });
    }
  } else {
    run(Both{}, [&]() __attribute__((always_inline)) {
      write_stats();
      __syncthreads();
      write_outputs();
    });
  }
}

#ifndef GHA_GTA_SPEC
#define GHA_GTA_SPEC 1  // score and value waves specialised
#endif

template <int DQK, int H>
hipError_t launch_h(const PrefillArgs& a, bool out_f32, hipStream_t st) {
  const uint32_t padded = (uint32_t)((a.n_blocks + 7) / 8 * 8);
  constexpr bool kSpec = GHA_GTA_SPEC != 0;
  if (out_f32)
    hipLaunchKernelGGL((gta_kernel<DQK, H, true, kSpec>), dim3(padded), dim3(64 * NW), 0, st, a);
  else
    hipLaunchKernelGGL((gta_kernel<DQK, H, false, kSpec>), dim3(padded), dim3(64 * NW), 0, st, a);
  return hipGetLastError();
}

}  // namespace

int gta_positions_per_wg() { return ROWS; }

bool gta_layout_supported(const PrefillArgs& a, int d_qk, int d_v) {
  // one (batch, group) K or (batch, head) V sequence must span less than 2^31
  // bytes (32-bit buffer offsets and range) and rows must not overlap, so that
  // the range check cuts exactly at the last position
  return a.k_ss >= d_qk && a.v_ss >= d_v && span_below((int64_t)a.S_q + 2 * KB, a.k_ss, 2, (int64_t)1 << 31) &&
         span_below((int64_t)a.S_q + 2 * KB, a.v_ss, 2, (int64_t)1 << 31);
}

hipError_t launch_gta(const PrefillArgs& a, int d_qk, int sources, bool out_f32, hipStream_t st) {
#define GHA_GTA_CASE(DQ, HH) \
  if (d_qk == DQ && sources == HH) return launch_h<DQ, HH>(a, out_f32, st);
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
