// Causal grouped-query attention prefill, bf16 inputs, fp32 accumulation, on
// gfx950 MFMA ("Grouped Query Attention (GQA)", Ultralytics glossary, "How
// GQA works": a group of query heads shares one key/value head).  A
// work-group takes up to four query heads of one group and one block of
// positions, so every K/V tile staged in LDS is used by all of those heads.
//
// Per wave: QT tiles of 16 query rows.  Per iteration: 64 keys.
//   S^T (keys x queries) = K Q^T on MFMA, K from LDS, Q^T resident in VGPRs.
//   Online softmax on S^T: each lane holds one query column, so the running
//   max and the rescale factor are per-lane scalars.
//   O^T (dv x queries) += V^T P^T on MFMA: P^T is the S^T accumulator itself,
//   converted to bf16 in place; V^T comes from LDS, where the tile was stored
//   transposed (and its keys permuted to match the accumulator's key order)
//   when it was staged.
// K/V tiles are double-buffered in LDS: global loads for tile t+1 are issued
// before tile t is computed.
#include "device_common.hpp"
#include "kernels.hpp"

namespace gha {

namespace {

constexpr int KB = 64;  // keys per iteration

// Tuning knobs (compile-time): 16-row query tiles per wave for the GQA
// kernels, minimum resident work-groups per CU, and whether waves raise
// their issue priority while in the score-MFMA phase.
#ifndef GHA_PF_QT
#define GHA_PF_QT 2
#endif
#ifndef GHA_PF_MIN_WG
#define GHA_PF_MIN_WG 2
#endif
#ifndef GHA_PF_SETPRIO
#define GHA_PF_SETPRIO 1
#endif

// Position of key u (0..63) of a tile inside a V^T row.  The S^T accumulator
// of lane group g holds keys 16*kt + 4*g + r; the PV contraction step ks takes
// tiles 2ks and 2ks+1, so group g's eight slots are keys
// 32ks + {4g..4g+3, 16+4g..16+4g+3}, stored contiguously here.
__device__ __forceinline__ int vt_pos(int u) {
  int ks = u >> 5, w = u & 31, half = w >> 4, g = (w & 15) >> 2, r = w & 3;
  return 32 * ks + 8 * g + 4 * half + r;
}

template <int DQK, int DV, int QT, bool OUT_F32>
__global__ __launch_bounds__(256, GHA_PF_MIN_WG) void prefill_bf16_kernel(PrefillArgs a) {
  constexpr int KP = DQK + 8;   // K row pitch in LDS (elements): 16 B pad
  constexpr int VP = KB + 8;    // V^T row pitch in LDS (elements): 16 B pad
  constexpr int K_ELEMS = KB * KP;
  constexpr int V_ELEMS = DV * VP;
  constexpr int DS = DQK / 32;  // contraction steps of the score MFMA
  constexpr int DT = DV / 16;   // 16-wide output column tiles
  constexpr int KCH = DQK / 8;  // 16-byte chunks per K row
  constexpr int K_LOADS = KB * KCH / 256;       // 16-byte K loads per thread
  constexpr int K_ROWSTEP = 256 / KCH;          // rows between a thread's K loads
  constexpr int VCH = DV / 8;                   // 8-column chunks per V row
  constexpr int V_UNITS = (KB / 4) * VCH;       // (4 keys x 8 columns) units
  constexpr int V_PER_THREAD = (V_UNITS + 255) / 256;
  static_assert(K_LOADS >= 1 && KB * KCH % 256 == 0, "tile staging");

  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * (K_ELEMS + V_ELEMS)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 15;  // MFMA row / column index
  const int lg = lane >> 4;  // MFMA lane group

  // ---- which work this work-group does -----------------------------------
  const uint32_t lid = xcd_logical_id(blockIdx.x, gridDim.x);
  if (lid >= (uint32_t)a.n_blocks) return;
  const int n_qb = a.n_qblocks;
  const int qb = n_qb - 1 - (int)(lid % n_qb);  // heavy (late) blocks first
  int rest = (int)(lid / n_qb);
  const int sg = rest % a.n_subgroups;  rest /= a.n_subgroups;
  const int kvh = rest % a.h_kv;        // KV head
  const int b = rest / a.h_kv;

  const int wph = 4 / a.heads_per_wg;   // waves per head
  const int pos_per_wg = wph * QT * 16;
  const int qhead = kvh * a.group + sg * a.heads_per_wg + wave / wph;
  const int pos0 = qb * pos_per_wg + (wave % wph) * QT * 16;  // this wave's first row
  const int off = a.S_k - a.S_q;  // bottom-right causal offset

  // keys this work-group must visit, and this wave's own last visible key
  int k_end = a.S_k;
  int wave_kmax = a.S_k - 1;
  if (a.causal) {
    int last_pos = min(qb * pos_per_wg + pos_per_wg - 1, a.S_q - 1);
    k_end = min(a.S_k, last_pos + off + 1);
    wave_kmax = min(a.S_k - 1, min(pos0 + QT * 16 - 1, a.S_q - 1) + off);
  }
  const int n_kb = (k_end + KB - 1) / KB;

  const __bf16* qbase = (const __bf16*)a.q + (int64_t)b * a.q_sb + (int64_t)qhead * a.q_sh;
  const __bf16* kbase = (const __bf16*)a.k + (int64_t)b * a.k_sb + (int64_t)kvh * a.k_sh;
  const __bf16* vbase = (const __bf16*)a.v + (int64_t)b * a.v_sb + (int64_t)kvh * a.v_sh;

  // ---- resident Q^T fragments (B operand of the score MFMA) ---------------
  u32x4 qf[QT][DS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int pos = min(pos0 + qt * 16 + li, a.S_q - 1);  // rows past S_q are never written
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[qt][s] = ld16(qbase + (int64_t)pos * a.q_ss + 32 * s + 8 * lg);
  }

  // ---- staging: global -> registers -> LDS --------------------------------
  // Each thread loads K rows k_row + K_ROWSTEP*i (16 bytes each) and, per V
  // unit, 4 consecutive keys x 8 columns of V, which it transposes into V^T.
  // Tiles wholly inside the sequence use plain strided addresses; the tail
  // tile clamps rows to the last key (their scores are masked to -inf).
  const int k_row = tid / KCH, k_col = (tid % KCH) * 8;
  const __bf16* kthr = kbase + (int64_t)k_row * a.k_ss + k_col;
  const int64_t k_rowstep = (int64_t)K_ROWSTEP * a.k_ss;
  const __bf16* vthr[V_PER_THREAD];
  int v_dchunk[V_PER_THREAD], v_kgrp[V_PER_THREAD];
#pragma unroll
  for (int i = 0; i < V_PER_THREAD; ++i) {
    const int u = min(tid + 256 * i, V_UNITS - 1);
    v_dchunk[i] = u % VCH;
    v_kgrp[i] = u / VCH;
    const int d = v_dchunk[i] * 8;
    vthr[i] = vbase + d + (int64_t)(4 * v_kgrp[i]) * a.v_ss;
  }

  u32x4 kreg[K_LOADS];
  u32x4 vreg[V_PER_THREAD][4];

  auto load_tile = [&](int kb) {
    const int key0 = kb * KB;
    const int64_t koff = (int64_t)key0 * a.k_ss, voff = (int64_t)key0 * a.v_ss;
    if (key0 + KB <= a.S_k) {
#pragma unroll
      for (int i = 0; i < K_LOADS; ++i) kreg[i] = ld16(kthr + koff + i * k_rowstep);
#pragma unroll
      for (int i = 0; i < V_PER_THREAD; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) vreg[i][r] = ld16(vthr[i] + voff + r * a.v_ss);
    } else {
#pragma unroll
      for (int i = 0; i < K_LOADS; ++i) {
        const int kk = min(key0 + k_row + K_ROWSTEP * i, a.S_k - 1);
        kreg[i] = ld16(kbase + (int64_t)kk * a.k_ss + k_col);
      }
#pragma unroll
      for (int i = 0; i < V_PER_THREAD; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kk = min(key0 + 4 * v_kgrp[i] + r, a.S_k - 1);
          vreg[i][r] = ld16(vthr[i] + (int64_t)(kk - 4 * v_kgrp[i]) * a.v_ss);
        }
    }
  };

  // V^T rows are 64 keys (128 B) + 16 B pad; the 16-byte column unit of row d
  // is XOR-swizzled by (d >> 4) & 7, so that the 16 lanes writing one key
  // group to 16 different rows land in distinct banks while the MFMA-side
  // reads (16 consecutive rows, one unit) stay conflict-free.
  auto store_tile = [&](int buf) {
    __bf16* ks = smem + buf * (K_ELEMS + V_ELEMS);
    __bf16* vs = ks + K_ELEMS;
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) st16(ks + (k_row + K_ROWSTEP * i) * KP + k_col, kreg[i]);
#pragma unroll
    for (int i = 0; i < V_PER_THREAD; ++i) {
      if (tid + 256 * i < V_UNITS) {
        const int p = vt_pos(4 * v_kgrp[i]);
        const int sw = (v_dchunk[i] >> 1) & 7;
        const int pp = (((p >> 3) ^ sw) << 3) | (p & 7);
        __bf16* vrow = vs + (v_dchunk[i] * 8) * VP + pp;
        // 4 keys x 8 columns -> 8 rows (columns) x 4 keys
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          u32x2 lo = {lo_pair(vreg[i][0][w], vreg[i][1][w]), lo_pair(vreg[i][2][w], vreg[i][3][w])};
          u32x2 hi = {hi_pair(vreg[i][0][w], vreg[i][1][w]), hi_pair(vreg[i][2][w], vreg[i][3][w])};
          *reinterpret_cast<u32x2*>(vrow + (2 * w) * VP) = lo;
          *reinterpret_cast<u32x2*>(vrow + (2 * w + 1) * VP) = hi;
        }
      }
    }
  };

  // ---- running state -------------------------------------------------------
  // oacc[dt][qt]: O^T tile; lacc[qt]: the normaliser, from the ones-MFMA
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

  if (n_kb > 0) {
    load_tile(0);
    store_tile(0);
  }
  wait_vmem_all();
  __syncthreads();

  for (int kb = 0; kb < n_kb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < n_kb) load_tile(kb + 1);

    const int key0 = kb * KB;
    if (key0 <= wave_kmax) {  // wave-uniform: skip tiles wholly above the diagonal
      const __bf16* ks = smem + buf * (K_ELEMS + V_ELEMS);
      const __bf16* vs = ks + K_ELEMS;

      // S^T = K Q^T: per contraction step, read the four key tiles' fragments
      // first so several LDS reads are in flight per MFMA chain
      f32x4 sacc[4][QT];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) sacc[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (GHA_PF_SETPRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        u32x4 kf[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) kf[kt] = ld16(ks + (16 * kt + li) * KP + 32 * s + 8 * lg);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) sacc[kt][qt] = mfma_bf16(kf[kt], qf[qt][s], sacc[kt][qt]);
      }

      if (GHA_PF_SETPRIO) __builtin_amdgcn_s_setprio(0);
      // mask + online softmax (per query column = per lane)
      const bool need_mask = (key0 + KB > a.S_k) ||
                             (a.causal && key0 + KB - 1 > pos0 + off);
      u32x4 pf[QT][2];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        if (need_mask) {
          const int qpos = pos0 + qt * 16 + li;
          const int kmax = a.causal ? min(qpos + off, a.S_k - 1) : a.S_k - 1;
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
          for (int dt = 0; dt < DT; ++dt) oacc[dt][qt] *= alpha;
        }
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

      // O^T += V^T P^T, and the normaliser += 1^T P^T
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) lacc[qt] = mfma_bf16(ones, pf[qt][k2], lacc[qt]);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int unit = (4 * k2 + lg) ^ (dt & 7);
          u32x4 vf = ld16(vs + (16 * dt + li) * VP + 8 * unit);
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) oacc[dt][qt] = mfma_bf16(vf, pf[qt][k2], oacc[dt][qt]);
        }
      }
    }

    if (kb + 1 < n_kb) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise and write --------------------------------------
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int qpos = pos0 + qt * 16 + li;
    const float l = lacc[qt][0];
    if (qpos >= a.S_q) continue;
    const float inv = 1.f / l;
    if (a.lse != nullptr && lg == 0) {
      a.lse[((int64_t)b * a.lse_heads + qhead) * a.S_q + qpos] = (m2[qt] + fast_log2(l)) * kLn2;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = 16 * dt + 4 * lg;
      const int64_t obase = (int64_t)b * a.o_sb + (int64_t)qhead * a.o_sh + (int64_t)qpos * a.o_ss + d;
      const f32x4 v = oacc[dt][qt] * inv;
      if constexpr (OUT_F32) {
        *reinterpret_cast<f32x4*>((float*)a.o + obase) = v;
      } else {
        *reinterpret_cast<u32x2*>((__bf16*)a.o + obase) = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
      }
    }
  }
}

template <int D, int QT, bool OUT_F32>
hipError_t launch_one(const PrefillArgs& a, hipStream_t st) {
  const uint32_t padded = (uint32_t)((a.n_blocks + 7) / 8 * 8);
  hipLaunchKernelGGL((prefill_bf16_kernel<D, D, QT, OUT_F32>), dim3(padded), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

int prefill_rows_per_wave() { return GHA_PF_QT * 16; }

#ifndef GHA_PF_DIRECT
#define GHA_PF_DIRECT 1
#endif

static bool use_d128(const PrefillArgs& a, int d) { return d == 128 && GHA_PF_DIRECT && prefill_d128_supported(a); }

int prefill_bf16_waves(const PrefillArgs&, int) { return 4; }

hipError_t launch_prefill_bf16(const PrefillArgs& a, int d, bool out_f32, hipStream_t st) {
  if (use_d128(a, d)) return launch_prefill_d128(a, out_f32, st);
  if (d == 128) return out_f32 ? launch_one<128, GHA_PF_QT, true>(a, st) : launch_one<128, GHA_PF_QT, false>(a, st);
  if (d == 64) return out_f32 ? launch_one<64, GHA_PF_QT, true>(a, st) : launch_one<64, GHA_PF_QT, false>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace gha
