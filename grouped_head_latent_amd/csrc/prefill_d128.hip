// Causal grouped-query attention prefill for head dim 128, bf16 in, fp32
// accumulation ("Grouped Query Attention (GQA)", Ultralytics glossary, "How
// GQA works": a group of query heads shares one key/value head).  Same work
// split and math as the generic bf16 kernel; what differs is how K/V tiles
// reach the MFMAs:
//
//  * Tiles go from global memory straight into LDS (buffer_load_dwordx4 ...
//    lds: lane l of a wave writes 16 bytes at LDS base + 16 l).  No VGPR staging,
//    no LDS stores, no transposition work on the VALU.  Each lane picks the
//    16-byte unit of global memory that belongs at its LDS slot, so the LDS
//    layout can be swizzled freely: rows are 256 bytes (16 units); K row r
//    keeps unit u at slot u ^ (r & 15), V row r keeps unit u at slot
//    u ^ 2(r & 7).
//  * S^T = K Q^T reads K fragments with ds_read_b128 (16 lanes, 16 rows, one
//    logical unit: 16 distinct slots, no bank conflict).
//  * O^T += V^T P^T reads V^T fragments from the row-major V tile with
//    ds_read_b64_tr_b16.  Within each 16-lane group that instruction hands
//    destination lane d, element j, the element d % 4 of source lane
//    4 j + d / 4.  Source lane s of group g points at key row
//    K0 + s / 4 (K0 = 32 k2 + 16 h + 4 g), columns 16 dt + 4 (s % 4) .. + 3,
//    so lane d receives V[K0 + j][16 dt + d], j = 0..3: the four keys that
//    the score accumulator of lane group g holds in rows 4 g .. 4 g + 3.  Two
//    such reads (h = 0, 1) give the eight contraction slots of the group.
//    The 32 bytes a row contributes sit in slots 2(dt ^ (r & 7)) + {0, 1}, so
//    the eight rows read by one half-wave cover all 16 slots.
#include "device_common.hpp"
#include "kernels.hpp"
#include "lds_pipe.hpp"

#include <atomic>
#include <type_traits>

namespace gha {

namespace {

constexpr int KB = 64;     // keys per tile
constexpr int ROWB = 256;  // bytes per K or V row in LDS (128 bf16)
constexpr int TILEB = KB * ROWB;

#ifndef GHA_PF_QT
#define GHA_PF_QT 2
#endif
#ifndef GHA_PF_MIN_WG
#define GHA_PF_MIN_WG 2
#endif
#ifndef GHA_PF_SETPRIO
#define GHA_PF_SETPRIO 1
#endif
#ifndef GHA_PF_PFD
#define GHA_PF_PFD 1
#endif
#ifndef GHA_PF_ORDER
#define GHA_PF_ORDER 1
#endif

// DK2 = 0: keys of width 128.  DK2 = 64: keys of width 192 made of a
// per-head part k (128) and a part k2 (64) with its own strides (GQLA's
// decoupled RoPE key, shared by all groups when its head stride is 0), and
// queries [q; q2] to match; values stay 128 wide.  The second key part sits
// in LDS rows of 128 bytes (8 units, unit u at u ^ ((r / 2) % 8)), two tile
// buffers above the K and V buffers.
template <int QT, bool OUT_F32, int DK2>
__global__ __launch_bounds__(256, GHA_PF_MIN_WG) void prefill_d128_kernel(PrefillArgs a) {
  constexpr int D = 128;
  constexpr int DS1 = D / 32;             // score contraction steps over k
  constexpr int DS = DS1 + DK2 / 32;      // ... over [k; k2]
  constexpr int DT = D / 16;              // 16-wide output column tiles
  constexpr int NSTEP = 4 + DS;           // MFMA steps per tile: 4 value, DS score
  constexpr int K2ROWB = 2 * DK2;         // bytes per k2 row in LDS
  constexpr int K2TILEB = KB * K2ROWB;
  constexpr int K2BASE = 4 * TILEB;
  static_assert(DK2 == 0 || DK2 == 64, "second key part");

  __shared__ __attribute__((aligned(1024))) unsigned char smem[4 * TILEB + 2 * K2TILEB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15;
  const int lg = lane >> 4;

  // ---- which work this work-group does -------------------------------------
  // Under the causal mask q-block qb costs about qb + 1 key tiles.  With
  // paired blocks a work-group takes q-block n_qb - 1 - i and then q-block i,
  // so every work-group does the same work and the grid has no tail of heavy
  // blocks; otherwise it takes one block, heavy (late) blocks first.
  // Consecutive work-groups share (batch, KV head), so their K/V tiles meet
  // in one XCD's L2.
  const uint32_t lid = xcd_logical_id(blockIdx.x, gridDim.x);
  if (lid >= (uint32_t)a.n_blocks) return;
  const int n_qb = a.n_qblocks;
  const int n_slot = a.pair_qblocks ? (n_qb + 1) / 2 : n_qb;
  const int qi = (int)(lid % n_slot);
  int rest = (int)(lid / n_slot);
  const int sg = rest % a.n_subgroups;  rest /= a.n_subgroups;
  const int kvh = rest % a.h_kv;
  const int b = rest / a.h_kv;
  const int n_pass = (a.pair_qblocks && qi != n_qb - 1 - qi) ? 2 : 1;

  const int wph = 4 / a.heads_per_wg;
  const int pos_per_wg = wph * QT * 16;
  const int qhead = kvh * a.group + sg * a.heads_per_wg + wave / wph;
  const int off = a.S_k - a.S_q;  // bottom-right causal offset

  const __bf16* qbase = (const __bf16*)a.q + (int64_t)b * a.q_sb + (int64_t)qhead * a.q_sh;
  const __bf16* kbase = (const __bf16*)a.k + (int64_t)b * a.k_sb + (int64_t)kvh * a.k_sh;
  const __bf16* vbase = (const __bf16*)a.v + (int64_t)b * a.v_sb + (int64_t)kvh * a.v_sh;

  // A second pass reuses the LDS tile buffers: its first DMAs are issued
  // after the first pass's last tile iteration, whose closing barrier every
  // wave has passed once done reading them (its epilogue reads registers).
  for (int pass = 0; pass < n_pass; ++pass) {
  const int qb = pass == 0 ? n_qb - 1 - qi : qi;
  const int pos0 = qb * pos_per_wg + (wave % wph) * QT * 16;

  int k_end = a.S_k;
  int wave_kmax = a.S_k - 1;
  if (a.causal) {
    const int last_pos = min(qb * pos_per_wg + pos_per_wg - 1, a.S_q - 1);
    k_end = min(a.S_k, last_pos + off + 1);
    wave_kmax = min(a.S_k - 1, min(pos0 + QT * 16 - 1, a.S_q - 1) + off);
  }
  const int n_kb = (k_end + KB - 1) / KB;

  // ---- resident Q^T fragments ---------------------------------------------
  u32x4 qf[QT][DS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int pos = min(pos0 + qt * 16 + li, a.S_q - 1);
#pragma unroll
    for (int s = 0; s < DS1; ++s) qf[qt][s] = ld16_stream(qbase + (int64_t)pos * a.q_ss + 32 * s + 8 * lg);
    if constexpr (DK2 > 0) {
      const __bf16* q2p = (const __bf16*)a.q2 + (int64_t)b * a.q2_sb + (int64_t)qhead * a.q2_sh + (int64_t)pos * a.q2_ss;
#pragma unroll
      for (int s = DS1; s < DS; ++s) qf[qt][s] = ld16_stream(q2p + 32 * (s - DS1) + 8 * lg);
    }
  }

  // ---- tile loads: wave w fills rows 16 w .. 16 w + 15 of both tiles -------
  // Load i of a wave covers rows 16 w + 4 i + lane / 16, LDS slot lane % 16.
  // Buffer loads with the range set to the last key's row: rows past the
  // sequence end come back as zeros (their scores are masked anyway), so the
  // tail tile needs no address clamping.
  const int lrow = lane >> 4, lslot = lane & 15;
  uint32_t kofs[4], vofs[4];  // byte offsets from the tile's first key
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = 4 * i + lrow;  // row within the wave's 16 (= r & 15)
    const int r = 16 * wave + rr;
    kofs[i] = (uint32_t)(r * a.k_ss + 8 * (lslot ^ rr)) * 2u;
    vofs[i] = (uint32_t)(r * a.v_ss + 8 * (lslot ^ (2 * (rr & 7)))) * 2u;
  }
  const uint32_t k_step = (uint32_t)a.k_ss * (2u * KB), v_step = (uint32_t)a.v_ss * (2u * KB);
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)kbase, 0, (int)((uint32_t)(a.S_k - 1) * (uint32_t)a.k_ss * 2u + 2u * D), kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)vbase, 0, (int)((uint32_t)(a.S_k - 1) * (uint32_t)a.v_ss * 2u + 2u * D), kBufferFlags);
  // second key part: 8 rows per DMA instruction, lane l taking row l / 8 and
  // LDS unit l % 8, so wave w fills rows 16 w .. 16 w + 15 with two
  __amdgpu_buffer_rsrc_t k2rs = krs;
  uint32_t k2ofs[2] = {0u, 0u};
  if constexpr (DK2 > 0) {
    const __bf16* k2base = (const __bf16*)a.k2 + (int64_t)b * a.k2_sb + (int64_t)kvh * a.k2_sh;
    k2rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)k2base, 0, (int)((uint32_t)(a.S_k - 1) * (uint32_t)a.k2_ss * 2u + 2u * DK2), kBufferFlags);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int rr = 8 * i + (lane >> 3);  // row within the wave's 16
      const int r = 16 * wave + rr;
      k2ofs[i] = (uint32_t)(r * a.k2_ss + 8 * ((lane & 7) ^ ((rr >> 1) & 7))) * 2u;
    }
  }
  const uint32_t k2_step = (uint32_t)a.k2_ss * (2u * KB);
  // LDS: K tiles in buffers 0/1 at 0 and 16 KiB, V tiles in buffers 0/1 at
  // 32 and 48 KiB; tile t goes to buffer t % 2.
  auto issue_k = [&](int t) {
    const uint32_t dst = lds_offset(smem) + (t & 1) * TILEB + wave * 16 * ROWB;
    const uint32_t so = (uint32_t)t * k_step;
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_dma16(krs, dst + 1024 * i, kofs[i], so);
    if constexpr (DK2 > 0) {
      const uint32_t dst2 = lds_offset(smem) + K2BASE + (t & 1) * K2TILEB + wave * 16 * K2ROWB;
#pragma unroll
      for (int i = 0; i < 2; ++i) lds_dma16(k2rs, dst2 + 1024 * i, k2ofs[i], (uint32_t)t * k2_step);
    }
  };
  auto issue_v = [&](int t) {
    const uint32_t dst = lds_offset(smem) + 2 * TILEB + (t & 1) * TILEB + wave * 16 * ROWB;
    const uint32_t so = (uint32_t)t * v_step;
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_dma16(vrs, dst + 1024 * i, vofs[i], so);
  };

  // ---- fragment addresses inside a stage (bytes) ----------------------------
  // K: row 16 kt + li, logical unit 4 s + lg -> slot (4 s + lg) ^ li.  Since
  // 4 s and lg occupy different bits, the byte address is
  // (li * 256 + 16 (lg ^ li)) ^ 64 s, plus 4096 kt.
  const uint32_t kfrag = li * ROWB + 16 * (lg ^ li);
  // second key part: row 16 kt + li, unit 4 (s - DS1) + lg at
  // (kfrag2 ^ 64 (s - DS1)) + 2048 kt
  const uint32_t kfrag2 = K2BASE + li * K2ROWB + 16 * (lg ^ ((li >> 1) & 7));
  // V: source lane li of group lg reads row vr = 4 lg + li / 4 (+ 32 k2 + 16 h),
  // columns 16 dt + 4 (li % 4): logical unit 2 dt + (li / 2) % 2, byte 8 (li % 2)
  // of it, at slot 2 (dt ^ (vr & 7)) + (li / 2) % 2.  Bits 5..7 of the
  // remaining terms are zero, so the address is vfrag ^ 32 dt.
  uint32_t vfrag;
  {
    const int vr = 4 * lg + (li >> 2);
    vfrag = (2 * TILEB + vr * ROWB + 16 * ((li >> 1) & 1) + 8 * (li & 1)) ^ (32 * (vr & 7));
  }
  // buffer 1 of either tile sits 16 KiB above buffer 0, and no fragment
  // offset reaches bit 14
  static_assert(TILEB == 16384, "buffer bit");

  // ---- running state -------------------------------------------------------
  f32x4 oacc[DT][QT], lacc[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    lacc[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float m2[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) m2[qt] = kNegInf;
  const float c2 = a.scale * kLog2e;
  const u32x4 ones = {kBf16OnePair, kBf16OnePair, kBf16OnePair, kBf16OnePair};

  // The MFMA phase of iteration t runs in NSTEP steps (8, or 10 with a
  // second key part), each issuing the LDS reads of a later step (GHA_PF_PFD
  // steps ahead) before its own MFMAs:
  //   steps 0..3: O^T += V^T P^T for k2 = step / 2, column tiles 4 (step % 2) ..
  //               + 3 (V from buffer t % 2; step 0 also adds 1^T P^T to the
  //               normaliser, step 2 likewise for k2 = 1)
  //   steps 4..:  S^T += K Q^T for contraction step s = step - 4 (K of tile
  //               t + 1 from buffer (t + 1) % 2; steps past 7 read the second
  //               key part)
  f32x4 sacc[4][QT];
  constexpr int NFR = GHA_PF_PFD + 1;  // fragment buffers (LDS reads run PFD steps ahead)
  // Order of the steps in the MFMA phase: PV and score steps alternate, so
  // that the transposing V reads (slow per wave) of one step overlap the
  // MFMAs of a score step, whose own K reads are few.
  auto step_at = [](int j) { return (GHA_PF_ORDER && j < 8) ? ((j & 1) ? 4 + (j >> 1) : (j >> 1)) : j; };
  u32x4 fr[NFR][4];
  auto load_step = [&](int j, int t, u32x4 (&f)[4]) __attribute__((always_inline)) {
    if (j < 4) {
      const uint32_t vst = vfrag ^ ((t & 1) << 14);
      const int k2 = j >> 1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t va = vst ^ ((4 * (j & 1) + i) << 5);
        const u32x2 h0 = ld_tr(smem + va + k2 * 32 * ROWB);
        const u32x2 h1 = ld_tr(smem + va + k2 * 32 * ROWB + 16 * ROWB);
        f[i] = u32x4{h0[0], h0[1], h1[0], h1[1]};
      }
    } else if (j - 4 < DS1) {
      const uint32_t kst = kfrag ^ (((t + 1) & 1) << 14);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) f[kt] = ld16(smem + (kst ^ ((j - 4) << 6)) + kt * 16 * ROWB);
    } else {
      const uint32_t kst = (kfrag2 ^ ((j - 4 - DS1) << 6)) + ((t + 1) & 1) * K2TILEB;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) f[kt] = ld16(smem + kst + kt * 16 * K2ROWB);
    }
  };
  auto mfma_step = [&](int j, const u32x4 (&f)[4], const u32x4 (&pf)[QT][2]) __attribute__((always_inline)) {
    if (j < 4) {
      const int k2 = j >> 1;
      if ((j & 1) == 0) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) lacc[qt] = mfma_bf16(ones, pf[qt][k2], lacc[qt]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          const int dt = 4 * (j & 1) + i;
          oacc[dt][qt] = mfma_bf16(f[i], pf[qt][k2], oacc[dt][qt]);
        }
    } else {
      const int st = j - 4;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          sacc[kt][qt] = mfma_bf16(f[kt], qf[qt][st], st == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sacc[kt][qt]);
    }
  };
  // scores of tile 0 (prologue): steps 4 .. NSTEP - 1 of a phantom iteration -1
  auto score0 = [&]() __attribute__((always_inline)) {
    const u32x4 nopf[QT][2] = {};
#pragma unroll
    for (int j = 4; j < 4 + GHA_PF_PFD; ++j) load_step(j, -1, fr[j % NFR]);
#pragma unroll
    for (int j = 4; j < NSTEP; ++j) {
      if (j + GHA_PF_PFD < NSTEP) load_step(j + GHA_PF_PFD, -1, fr[(j + GHA_PF_PFD) % NFR]);
      mfma_step(j, fr[j % NFR], nopf);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Software pipeline: iteration t runs the softmax of tile t (VALU), then
  // P(t) V(t) and the scores of tile t + 1 back to back (MFMA), so each wave
  // alternates one VALU phase and one MFMA phase per tile and the two waves
  // sharing a SIMD can overlap them.  K runs one tile ahead of V.
  if (n_kb > 0) issue_k(0);
  if (n_kb > 0) issue_v(0);
  if (n_kb > 1) issue_k(1);
  wait_vmem_all();
  __syncthreads();
  if (n_kb > 0 && wave_kmax >= 0) score0();
  __syncthreads();  // every wave is done with K buffer 0 before tile 2 lands there

  // Tiles before t_mask are fully visible to every wave of the work-group
  // (no key past the sequence end or past any row's diagonal); from t_mask
  // on, the softmax applies the mask.  Two copies of the loop keep the mask
  // test out of the main one.
  int t_mask = a.S_k / KB;
  if (a.causal) t_mask = min(t_mask, max(0, (qb * pos_per_wg + off + 1) / KB));
  t_mask = min(t_mask, n_kb);

  auto iteration = [&](int t, auto masked) __attribute__((always_inline)) {
    constexpr bool kMasked = decltype(masked)::value;
    // V(t+1) replaces V(t-1) and K(t+2) replaces K(t): both were last read
    // before the previous barrier
    if (t + 1 < n_kb) issue_v(t + 1);
    if (t + 2 < n_kb) issue_k(t + 2);

    const int key0 = t * KB;
    if (!kMasked || key0 <= wave_kmax) {  // wave-uniform: skip tiles wholly above the diagonal
#pragma unroll
      for (int j = 0; j < GHA_PF_PFD; ++j) load_step(step_at(j), t, fr[j]);  // in flight during the softmax
      __builtin_amdgcn_sched_barrier(0);
      u32x4 pf[QT][2];
      // Each lane scales the largest of its own scores of a row; only when
      // some lane exceeds its row's reference by more than the slack does the
      // wave form the row maxima across the four lane groups and move the
      // reference (the decisions of a full reduction, without it most tiles).
      float mxl[QT];
      bool grow = false;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        if (kMasked) {
          const int qpos = pos0 + qt * 16 + li;
          const int kmax = a.causal ? min(qpos + off, a.S_k - 1) : a.S_k - 1;
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (key0 + 16 * kt + 4 * lg + r > kmax) sacc[kt][qt][r] = kNegInf;
        }
        float mx = max3f(sacc[0][qt][0], sacc[0][qt][1], sacc[0][qt][2]);
        mx = max3f(mx, sacc[0][qt][3], sacc[1][qt][0]);
        mx = max3f(mx, sacc[1][qt][1], sacc[1][qt][2]);
        mx = max3f(mx, sacc[1][qt][3], sacc[2][qt][0]);
        mx = max3f(mx, sacc[2][qt][1], sacc[2][qt][2]);
        mx = max3f(mx, sacc[2][qt][3], sacc[3][qt][0]);
        mx = max3f(mx, sacc[3][qt][1], sacc[3][qt][2]);
        mxl[qt] = max2f(mx, sacc[3][qt][3]) * c2;  // = the largest scaled score (scaling is monotone)
        grow = grow || mxl[qt] > m2[qt] + kRescaleSlack;
      }
      if (wave_any(grow)) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          const float mx2 = group4_max(mxl[qt]);
          if (wave_any(mx2 > m2[qt] + kRescaleSlack)) {
            const float mnew = fmaxf(m2[qt], mx2);
            const float alpha = (mnew == kNegInf) ? 1.f : fast_exp2(m2[qt] - mnew);
            m2[qt] = mnew;
            lacc[qt] *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oacc[dt][qt] *= alpha;
          }
        }
      }
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const float msub = (m2[qt] == kNegInf) ? 0.f : m2[qt];
        float p[4][4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) p[kt][r] = fast_exp2(__builtin_fmaf(sacc[kt][qt][r], c2, -msub));
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          pf[qt][k2] = u32x4{pack_bf16(p[2 * k2][0], p[2 * k2][1]), pack_bf16(p[2 * k2][2], p[2 * k2][3]),
                             pack_bf16(p[2 * k2 + 1][0], p[2 * k2 + 1][1]),
                             pack_bf16(p[2 * k2 + 1][2], p[2 * k2 + 1][3])};
        }
      }

      if (GHA_PF_SETPRIO) __builtin_amdgcn_s_setprio(1);
      // P(t) V(t), then the scores of tile t + 1; past this wave's last tile
      // (or the last tile) those read a stale buffer and are never used
#pragma unroll
      for (int j = 0; j < NSTEP; ++j) {
        if (j + GHA_PF_PFD < NSTEP) load_step(step_at(j + GHA_PF_PFD), t, fr[(j + GHA_PF_PFD) % NFR]);
        mfma_step(step_at(j), fr[j % NFR], pf);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (GHA_PF_SETPRIO) __builtin_amdgcn_s_setprio(0);
    }

    wait_vmem_all();
    __syncthreads();
  };
  for (int t = 0; t < t_mask; ++t) iteration(t, std::false_type{});
  for (int t = t_mask; t < n_kb; ++t) iteration(t, std::true_type{});

  // ---- epilogue --------------------------------------------------------------
  // bf16 rows go out through LDS: this wave's slice of K buffer qt (rows
  // 16 w .. 16 w + 15, written only by this wave's DMAs, idle after the last
  // barrier) holds q-tile qt as 16 rows of 256 B (16-byte unit u of row r at
  // u ^ r, so that neither the 8-byte writes nor the row reads conflict in
  // the banks), and each 16 lanes then store one whole row.  The output is never read again, so the stores (like
  // the query loads) are non-temporal: they stream past L2 instead of
  // evicting the K/V tiles that other work-groups of the head still read.
  static_assert(QT <= 2, "q-tile qt is staged in K buffer qt");
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int qpos = pos0 + qt * 16 + li;
    const float l = lacc[qt][0];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (qpos < a.S_q && a.lse != nullptr && lg == 0) {
      a.lse[((int64_t)b * a.lse_heads + qhead) * a.S_q + qpos] = (m2[qt] + fast_log2(l)) * kLn2;
    }
    if constexpr (OUT_F32) {
      if (qpos < a.S_q) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int64_t obase = (int64_t)b * a.o_sb + (int64_t)qhead * a.o_sh + (int64_t)qpos * a.o_ss + 16 * dt + 4 * lg;
          *reinterpret_cast<f32x4*>((float*)a.o + obase) = oacc[dt][qt] * inv;
        }
      }
    } else {
      unsigned char* stage = smem + qt * TILEB + wave * 16 * ROWB + li * ROWB;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f32x4 v = oacc[dt][qt] * inv;
        *reinterpret_cast<u32x2*>(stage + 16 * ((2 * dt + (lg >> 1)) ^ li) + 8 * (lg & 1)) =
            u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
      }
    }
  }
  if constexpr (!OUT_F32) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * i + (lane >> 4);  // row of the q-tile
        const int qpos = pos0 + qt * 16 + r;
        const u32x4 v = ld16(smem + qt * TILEB + wave * 16 * ROWB + r * ROWB + 16 * ((lane & 15) ^ r));
        if (qpos < a.S_q) {
          const int64_t obase = (int64_t)b * a.o_sb + (int64_t)qhead * a.o_sh + (int64_t)qpos * a.o_ss + 8 * (lane & 15);
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>((__bf16*)a.o + obase));
        }
      }
    }
    // every staging read has returned before a second pass's DMAs refill the slice
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  }  // pass
}

}  // namespace

bool prefill_d128_supported(const PrefillArgs& a) {
  // one (batch, head) sequence of K or V must span less than 2^31 bytes
  // (buffer offsets and range are 32-bit), and rows must not overlap, so
  // that the range check cuts exactly at the last key
  int64_t ss = a.k_ss > a.v_ss ? a.k_ss : a.v_ss;
  if (a.dk2 > 0) ss = ss > a.k2_ss ? ss : a.k2_ss;
  return a.k_ss >= 128 && a.v_ss >= 128 && (a.dk2 == 0 || a.k2_ss >= a.dk2) &&
         span_below((int64_t)a.S_k + 4 * KB, ss, 2, (int64_t)1 << 31);
}

int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = -1;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n > 0 ? n : 0;
}

namespace {
// Work-groups of this kernel resident at once on the current device, or 0 if
// the device cannot be queried.
int resident_wgs() { return device_cus() * GHA_PF_MIN_WG; }
}  // namespace

hipError_t launch_prefill_d128(const PrefillArgs& args, bool out_f32, hipStream_t st) {
  // Pair heavy and light causal q-blocks once the grid outgrows one round of
  // resident work-groups: every work-group then does the same work.  Within
  // one round, single blocks finish sooner.
  PrefillArgs a = args;
  a.pair_qblocks = 0;
  if (a.causal && a.n_qblocks > 1) {
    const int slots = resident_wgs();
    if (slots > 0 && a.n_blocks > slots) {
      a.pair_qblocks = 1;
      a.n_blocks = a.n_blocks / a.n_qblocks * ((a.n_qblocks + 1) / 2);
    }
  }
  const uint32_t padded = (uint32_t)((a.n_blocks + 7) / 8 * 8);
  if (a.dk2 == 64) {
    if (out_f32)
      hipLaunchKernelGGL((prefill_d128_kernel<GHA_PF_QT, true, 64>), dim3(padded), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((prefill_d128_kernel<GHA_PF_QT, false, 64>), dim3(padded), dim3(256), 0, st, a);
  } else if (a.dk2 == 0) {
    if (out_f32)
      hipLaunchKernelGGL((prefill_d128_kernel<GHA_PF_QT, true, 0>), dim3(padded), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((prefill_d128_kernel<GHA_PF_QT, false, 0>), dim3(padded), dim3(256), 0, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gha
