// Absorbed latent decode (MLA / GQLA MQA-absorb path), bf16, split-KV with a
// log-sum-exp merge.
//
// "GQLA: Group-Query Latent Attention ...", section 1 and Figure 2 (right):
// with W^UK folded into the query and W^UV into the output, every query head
// attends directly over the cached latent.  Each cached token is one row of
// r_kv + d_r = 576 bf16 (the latent c^KV followed by the shared RoPE key k^R).
// For head i and token u the score is q_lat_i . c_u + q_rope_i . k^R_u (a
// 576-long dot product) and the value is c_u (the first 512 features).
//
// One work-group takes 128 query rows (all heads of one token at s_q = 1),
// one wave per SIMD, and walks a split of the cache in tiles of 32 tokens.
// Every tile goes from HBM straight into LDS (buffer DMA, no VGPR staging)
// once and serves all 128 rows:
//   S^T (tokens x rows) = C Q^T over 576 features: wave w scores rows
//   32 w .. 32 w + 31; K-side fragments are 16 B LDS reads, Q^T stays in
//   VGPRs.  The wave runs the softmax of its rows and publishes P^T in LDS.
//   O^T (512 x rows) += C^T P^T: wave w owns output columns
//   128 w .. 128 w + 127 for all 128 rows; C^T fragments come from
//   transposing LDS reads (ds_read_b64_tr_b16) and P^T of all rows from LDS.
// The O^T accumulator (128 x 128 fp32 per wave) lives in AGPRs.  The scores
// of tile t and the values of tile t - 1 are contracted in one interleaved
// MFMA stream, so LDS latency hides behind the other half's matrix work.
//
// LDS tile layout, token-major: token k's latent row (64 chunks of 16 B) at
// 1024 k with chunk c at position c ^ sw(k), sw a 4-bit permutation of
// k mod 16; its RoPE row (8 chunks) at 128 k in a separate ring with chunk c
// at position c ^ ((k / 2) mod 8).  One DMA instruction moves one token's
// 1 KiB latent row (or the RoPE rows of 8 tokens) from contiguous HBM.
// The transposing value reads (4 tokens x 32 B per 16 lanes) are free of
// bank conflicts.  The score reads (16 tokens, one chunk) are not: gfx950's
// LDS maps rows 1 KiB apart onto its banks so that every 4-bit permutation
// of k mod 16 leaves them two-way conflicted (an LDS probe of this pattern
// counts 3.9 conflict cycles per read; the kernel's counters show about two
// per LDS instruction).  Swizzles that the probe measured conflict-free for
// both kinds of read (e.g. sw(k) = 2 (k2 + 2 k0 + 4 (k1 ^ k2)) from the bits
// of k) made this kernel 1-3% slower at s_q = 1 and 2, so this one is kept.
#include "device_common.hpp"
#include "kernels.hpp"
#include "lds_pipe.hpp"

#include <algorithm>
#include <type_traits>

namespace gha {
namespace {

constexpr int RKV = 512, DR = 64, DL = RKV + DR;  // 576
constexpr int T = 32;                             // tokens per tile
constexpr int LROW = RKV * 2;                     // 1 KiB latent row of a token in LDS
constexpr int RROW = DR * 2;                      // 128 B RoPE row
constexpr int LTILE = T * LROW;                   // 32 KiB
constexpr int RTILE = T * RROW;                   // 4 KiB
constexpr int NLS = 4, NRS = 3;                   // latent and RoPE ring slots
constexpr int ROWS = 128;                         // query rows per work-group
constexpr int DS = DL / 32;                       // 18 score contraction steps
constexpr int PQT = 1024;                         // P^T fragments of one q-tile (64 lanes x 16 B)
constexpr int PBUF = 8 * PQT;                     // P^T of the work-group's 8 q-tiles
constexpr int RBASE = NLS * LTILE;
constexpr int PBASE = RBASE + NRS * RTILE;
constexpr int LDS_BYTES = PBASE + 2 * PBUF;       // 156 KiB
constexpr float kLatentSlack = 96.f;              // see the running state below
// the cost of starting a segment (loading 128 query rows, writing a 256 KiB
// partial: some 400 KiB of traffic at a work-group's share of the bandwidth,
// plus latency), in tiles of 36 KiB; measured at about 30 us against 1.9 us
// per tile on the 128-head workload
constexpr int kSegStartTiles = 16;
// the value MFMA after which P^T is published (after the last softmax step,
// with value MFMAs left to cover the LDS writes before the barrier)
constexpr int kPublishSlot = 44;

// chunk swizzles of the LDS rows (see the layout above)
__host__ __device__ constexpr int lat_sw(int k) { return ((k & 7) << 1) | ((k >> 3) & 1); }
__host__ __device__ constexpr int rope_sw(int k) { return (k >> 1) & 7; }

// tiles of sequence b (0 past the batch); lengths are clamped to [0, L_cap]
__device__ __forceinline__ int latent_tiles(const LatentArgs& a, int b) {
  return b < a.B ? (min(max(a.seqlens[b], 0), a.L_cap) + T - 1) / T : 0;
}
// wait until at most one tile's DMAs (9 per wave) are in flight
__device__ __forceinline__ void wait_vmem_but_one_tile() { asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); }

// The cache tiles load non-temporal: with one row block a tile is read once;
// with two (s_q = 2 at 128 heads) the neighbouring work-groups of a tile range
// run close together, and the non-temporal stream measured 1.5% faster than
// the default policy there too.
__global__ __launch_bounds__(256, 1) void latent_split_kernel(LatentArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[LDS_BYTES];
  __shared__ __attribute__((aligned(4))) unsigned char restart_flag[2][4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;

  const uint32_t lid = xcd_logical_id(blockIdx.x, gridDim.x);
  if (lid >= (uint32_t)(a.n_wg * a.n_rb)) return;
  // work-group-uniform indices, kept in scalar registers; the two row
  // blocks of one tile range are neighbours (same XCD, shared L2)
  const int rb = __builtin_amdgcn_readfirstlane(lid % a.n_rb);
  const int w = __builtin_amdgcn_readfirstlane(lid / a.n_rb);

  // ---- this work-group's share of the tiles of all sequences ----------------
  // The tiles of sequences 0 .. B - 1 (NT in all) are numbered one after
  // another, each sequence's preceded by X placeholder positions that stand
  // for the cost of starting a segment there (loading the queries, writing a
  // partial): X = kSegStartTiles, at most the mean share NT / n_wg.
  // Work-group w takes the positions [w NV / n_wg, (w + 1) NV / n_wg) of
  // the NV = NT + X B, i.e. the tiles among them: equal costs whatever the
  // length mix, a share that opens a second sequence holding X tiles fewer.
  // Each sequence it touches is a segment with its own partial, in slot
  // w + b (unique: along the segments either w or b grows).
  int NT = 0;
  for (int c0 = 0; c0 < a.B; c0 += 64)
    NT += __builtin_amdgcn_readlane(wave_incl_scan(latent_tiles(a, c0 + lane)), 63);
  const int X = __builtin_amdgcn_readfirstlane(min(kSegStartTiles, NT / a.n_wg));
  // positions of sequence b: X placeholders, then its tiles (none past the batch)
  auto positions = [&](int b) __attribute__((always_inline)) { return b < a.B ? latent_tiles(a, b) + X : 0; };
  const int NV = NT + X * a.B;  // below 2^31: checked on the host
  const int lo = (int)((int64_t)w * NV / a.n_wg), hi = (int)((int64_t)(w + 1) * NV / a.n_wg);
  // one work-group publishes the prefix sums of the positions for the merge
  if (lid == 0 && wave == 0) {
    int run = 0;
    for (int c0 = 0; c0 < a.B; c0 += 64) {
      const int t = positions(c0 + lane);
      const int incl = wave_incl_scan(t) + run;
      if (c0 + lane < a.B) a.ws_tiles[c0 + lane] = incl - t;
      run = __builtin_amdgcn_readlane(incl, 63);
    }
    if (lane == 0) a.ws_tiles[a.B] = run;
  }

  if (lo >= hi) return;
  // first sequence with positions at or after lo, and the positions before it
  int b0 = 0, P = 0;
  for (int c0 = 0;; c0 += 64) {
    const int t = positions(c0 + lane);
    const int incl = wave_incl_scan(t) + P;
    const uint64_t m = __builtin_amdgcn_ballot_w64(incl > lo);
    if (m != 0) {
      const int j = __builtin_ctzll(m);
      b0 = c0 + j;
      P = __builtin_amdgcn_readlane(incl - t, j);
      break;
    }
    P = __builtin_amdgcn_readlane(incl, 63);
  }
  b0 = __builtin_amdgcn_readfirstlane(b0);
  P = __builtin_amdgcn_readfirstlane(P);
  // ---- one segment: sequence b, tokens [start, end), partial slot ----------
  auto segment = [&](int b, int L, int start, int end, int slot) __attribute__((always_inline)) {

  // ---- rows: wave w scores rows 32 w .. 32 w + 31 (two q-tiles) and owns
  // their softmax; it accumulates output columns 128 w .. 128 w + 127 for all
  // 128 rows of the work-group.  Row R = t * h_q + head. --------------------
  const int n_rows = a.s_q * a.h_q;
  int kvis[2];
  bool row_ok[2];
  u32x4 qf[2][DS];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int R = rb * ROWS + 32 * wave + 16 * qt + li;
    row_ok[qt] = R < n_rows;
    const int tq = R / a.h_q, head = R % a.h_q;
    kvis[qt] = L - a.s_q + tq;  // last visible token (bottom-right causal)
    const __bf16* qp = (const __bf16*)a.q + (int64_t)b * a.q_sb + (int64_t)head * a.q_sh + (int64_t)tq * a.q_ss;
    const __bf16* qrp = (const __bf16*)a.qr + (int64_t)b * a.qr_sb + (int64_t)head * a.qr_sh + (int64_t)tq * a.qr_ss;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      if (!row_ok[qt]) qf[qt][s] = u32x4{0u, 0u, 0u, 0u};
      else if (s < RKV / 32) qf[qt][s] = ld16(qp + 32 * s + 8 * lg);
      else qf[qt][s] = ld16(qrp + 32 * (s - RKV / 32) + 8 * lg);
    }
  }
  wait_vmem_all();
  const float c2 = a.scale * kLog2e;

  // ---- tile loads ------------------------------------------------------------
  // Tile t: latent rows in ring slot t % 4, RoPE rows in slot t % 3.  Wave w
  // moves tokens 8 w .. 8 w + 7: one instruction per latent row (lane l
  // brings chunk l ^ sw(k) to position l) and one for their RoPE rows (lane l:
  // token 8 w + l / 8, position l % 8).  Rows at or past the sequence end,
  // and tiles past the split, read as zeros (range check).
  const uint32_t c_row = (uint32_t)a.c_ss * 2u, r_row = (uint32_t)a.kr_ss * 2u;
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const __bf16*)a.c + (int64_t)b * a.c_sb), 0, (int)((uint32_t)(L - 1) * c_row + 2u * RKV), kBufferFlags);
  const __amdgpu_buffer_rsrc_t rrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const __bf16*)a.kr + (int64_t)b * a.kr_sb), 0, (int)((uint32_t)(L - 1) * r_row + 2u * DR), kBufferFlags);
  // lat_sw(8 w + j) = 2 j + (w & 1): the chunk of lane l for row j is l ^ (2 j + (w & 1))
  const uint32_t dma_v = (16u * lane) ^ (16u * (wave & 1));
  const int rtok = 8 * wave + (lane >> 3);
  const uint32_t r_off = (uint32_t)(lane >> 3) * r_row + 16u * ((lane & 7) ^ rope_sw(rtok));
  const uint32_t lds0 = lds_offset(smem);
  const int n_t = (end - start + T - 1) / T;
  // the DMAs of tile t (offsets of a tile past the split land out of range),
  // spread over the first score steps of an iteration
  struct DmaTile { uint32_t cso, rso, ldl, ldr; };
  auto dma_tile = [&](int t) __attribute__((always_inline)) -> DmaTile {
    const bool ok = t < n_t;
    const uint32_t tok = (uint32_t)(start + t * T + 8 * wave);
    return DmaTile{ok ? tok * c_row : kOutOfRange, ok ? tok * r_row : kOutOfRange,
                   lds0 + (t & 3) * LTILE + (8 * wave) * LROW, lds0 + RBASE + (t % NRS) * RTILE + wave * 1024};
  };
  auto dma = [&](const DmaTile& d, int j) __attribute__((always_inline)) {
    if (j < 8) lds_dma16_stream(crs, d.ldl + j * LROW, dma_v ^ (32u * j), d.cso + j * c_row);
    else lds_dma16_stream(rrs, d.ldr, r_off, d.rso);
  };

  // ---- fragment addresses (byte offsets in smem) ----------------------------
  // score A operand: chunk 4 s + lg of token 16 kt + li, i.e. byte
  // 1024 (16 kt + li) + 16 ((4 s + lg) ^ sw(li)) = (sfrag ^ 64 s) + 16384 kt
  const uint32_t sfrag = li * LROW + 16 * (lg ^ lat_sw(li));
  // RoPE steps s = 16, 17: chunk 4 (s - 16) + lg: (rfrag ^ 64 (s - 16)) + 2048 kt
  const uint32_t rfrag = li * RROW + 16 * (lg ^ rope_sw(li));
  // value A operand (transposing read), source lane li of group lg: token
  // 4 lg + li / 4 (+ 16 for the second half), chunk 16 w + 2 dt + (li / 2) % 2,
  // byte 8 (li % 2) of it: (vfrag ^ 32 dt) + 16384 half
  const int vtok = 4 * lg + (li >> 2);
  const uint32_t vfrag = vtok * LROW + 256 * wave + 16 * (((li >> 1) & 1) ^ lat_sw(vtok)) + 8 * (li & 1);

  // ---- running state -----------------------------------------------------------
  // Scores are taken against a per-row reference m2 (log2 units) fixed by
  // the first visible tile: probabilities 2^(s - m2) up to 2^kLatentSlack stay
  // far inside bf16 and fp32 range, so the accumulators never need
  // rescaling, and the other waves can use a row's probabilities without its
  // statistics.  A tile whose maximum exceeds m2 + kLatentSlack restarts the
  // split with the new maximum as reference; the result is the same softmax
  // either way.
  f32x4 oacc[8][8], lacc[2];  // oacc[column tile][q-tile of the work-group] (AGPRs)
  float m2[2] = {kNegInf, kNegInf};
  float m2s[2] = {kNegInf, kNegInf};  // m2 + slack: the restart threshold
  float msub[2] = {0.f, 0.f};         // m2, or 0 while the row has seen nothing
  u32x4 pall[8];              // P^T of all 8 q-tiles of the previous tile

  // Tiles wholly before `end` and before every row's causal limit need no
  // mask; only the last one or two may.
  int t_mask = (end - start) / T;
  {
    int lim = L - a.s_q;  // smallest last-visible token over the rows (tq = 0)
    t_mask = min(t_mask, max(0, (lim + 1 - start) / T));
  }

  // O^T += C^T P^T for this wave's 8 column tiles of the tile in slot `slot`,
  // one column tile (8 MFMAs) per step, C^T fragments read one step ahead
  u32x4 vf[2];
  auto load_v = [&](uint32_t vb, int dt, u32x4& v) __attribute__((always_inline)) {
    const unsigned char* vp = smem + (vb ^ (32u * dt));
    const u32x2 h0 = ld_tr(vp);
    const u32x2 h1 = ld_tr(vp + 16384);
    v = u32x4{h0[0], h0[1], h1[0], h1[1]};
  };
  // P^T of all rows for tile t (double-buffered by tile parity)
  auto load_p = [&](int t) __attribute__((always_inline)) {
    const unsigned char* pb = smem + PBASE + (t & 1) * PBUF + 16 * lane;
#pragma unroll
    for (int qt = 0; qt < 8; ++qt) pall[qt] = ld16(pb + qt * PQT);
  };
  auto pv_step = [&](uint32_t vb, int dt) __attribute__((always_inline)) {
    if (dt + 1 < 8) load_v(vb, dt + 1, vf[(dt + 1) & 1]);
#pragma unroll
    for (int qt = 0; qt < 8; ++qt) mfma_acc(oacc[dt][qt], vf[dt & 1], pall[qt]);
  };

  // Iteration t: phase A, the scores of tile t (with the P^T reads of tile
  // t - 1), then
  // phase B, the values of tile t - 1 with the softmax of tile t spread
  // between their MFMAs (VALU and matrix core run side by side).  P^T goes
  // to LDS and one barrier follows (tile t + 1 has landed, every row's P^T
  // is visible).  The DMAs of tile t + 2 (into the slots of tile t - 2) are
  // spread over both phases: the CU moves about 1 KiB per 64 cycles into LDS,
  // and bursts stall the issuing wave.  Restart requests raised at a barrier
  // are acted on before the next one: nothing computed in between is kept.
  uint32_t flags = 0;  // restart requests (one byte per wave) read after the last barrier
  auto iter = [&](int it, auto masked, auto has_pv) __attribute__((always_inline)) -> bool {
    constexpr bool kMasked = decltype(masked)::value;
    constexpr bool kPV = decltype(has_pv)::value;
    const int k0 = start + it * T;
    const uint32_t sb = (uint32_t)(it & 3) * LTILE + sfrag;
    const uint32_t rb_ = RBASE + (uint32_t)(it % NRS) * RTILE + rfrag;
    const uint32_t vb = (uint32_t)((it + 3) & 3) * LTILE + vfrag;

    f32x4 sacc[2][2];
    u32x4 kf[3][2];
    auto load_k = [&](int s, u32x4 (&f)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        if (s < 16) f[kt] = ld16(smem + (sb ^ (64u * s)) + 16384 * kt);
        else f[kt] = ld16(smem + (rb_ ^ (64u * (s - 16))) + 2048 * kt);
      }
    };
    auto s_step = [&](int s) __attribute__((always_inline)) {
      if (s + 2 < DS) load_k(s + 2, kf[(s + 2) % 3]);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          if (s == 0) mfma_v0(sacc[kt][qt], kf[s % 3][kt], qf[qt][s]);
          else mfma_v(sacc[kt][qt], kf[s % 3][kt], qf[qt][s]);
        }
    };

    // ---- phase A ----
    const DmaTile dt2 = dma_tile(it + 2);
    load_k(0, kf[0]);
    load_k(1, kf[1]);
    static_for<0, DS>([&](auto S_) __attribute__((always_inline)) {
      constexpr int s = decltype(S_)::value;
      if (s % 4 == 0) dma(dt2, s / 4);
      if (kPV && s == DS - 2) load_p(it - 1);
      if (kPV && s == DS - 1) load_v(vb, 0, vf[0]);
      s_step(s);
      __builtin_amdgcn_sched_barrier(0);
    });

    // ---- phase B: softmax per row (= per lane and q-tile) against a fixed
    // reference, in small stages; sacc[kt][qt][r] is token k0 + 16 kt + 4 lg + r
    // and becomes its probability in place.  A lane compares the largest of
    // its own eight scores with the row's threshold m2 + slack (-inf while
    // the row has seen nothing): only when some lane of the wave exceeds it
    // (a row's first visible scores, or a restart) is the row maximum formed
    // across the four lane groups; otherwise the reference stands and no
    // lanes need to talk.  The decisions are those of the full maximum. ----
    float lm[2], lm2[2];
    u32x4 pf[2];
    bool restart_row = false;
    // stages of q-tile qt: 0, 1 mask key tiles 0, 1 (masked tiles only);
    // 2 .. 5 lane maximum, scaled; 6 .. 9 shift by the reference (two scores
    // each); 10 .. 17 exp2 (one score each); 18, 19 bf16 packing
    auto stage = [&](auto QT_, auto ST_) __attribute__((always_inline)) {
      constexpr int qt = decltype(QT_)::value, st = decltype(ST_)::value;
      if constexpr (st <= 1) {
        if constexpr (kMasked) {
          const int kmax = min(end - 1, kvis[qt]);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (k0 + 16 * st + 4 * lg + r > kmax) sacc[st][qt][r] = kNegInf;
        }
      } else if constexpr (st == 2) {
        lm[qt] = max3f(sacc[0][qt][0], sacc[0][qt][1], sacc[0][qt][2]);
        lm2[qt] = max3f(sacc[0][qt][3], sacc[1][qt][0], sacc[1][qt][1]);
      } else if constexpr (st == 3) {
        lm[qt] = max3f(sacc[1][qt][2], sacc[1][qt][3], lm[qt]);
      } else if constexpr (st == 4) {
        lm[qt] = max2f(lm[qt], lm2[qt]);
      } else if constexpr (st == 5) {
        lm[qt] = lm[qt] * c2;  // = the largest scaled score (scaling is monotone)
      } else if constexpr (st >= 6 && st <= 9) {
        constexpr int kt = (st - 6) / 2, r0 = 2 * ((st - 6) % 2);
        sacc[kt][qt][r0] = __builtin_fmaf(sacc[kt][qt][r0], c2, -msub[qt]);
        sacc[kt][qt][r0 + 1] = __builtin_fmaf(sacc[kt][qt][r0 + 1], c2, -msub[qt]);
      } else if constexpr (st >= 10 && st <= 17) {
        constexpr int kt = (st - 10) / 4, r = (st - 10) % 4;
        sacc[kt][qt][r] = fast_exp2(sacc[kt][qt][r]);
      } else if constexpr (st == 18) {
        pf[qt][0] = pack_bf16(sacc[0][qt][0], sacc[0][qt][1]);
        pf[qt][1] = pack_bf16(sacc[0][qt][2], sacc[0][qt][3]);
      } else if constexpr (st == 19) {
        pf[qt][2] = pack_bf16(sacc[1][qt][0], sacc[1][qt][1]);
        pf[qt][3] = pack_bf16(sacc[1][qt][2], sacc[1][qt][3]);
      }
    };
    // after stage 5 of both q-tiles: the wave-uniform check, and the row
    // maxima when some lane asks for them.  A row's first visible scores fix
    // its reference; a tile that outgrows it by more than the slack asks for
    // a restart.
    auto check = [&]() __attribute__((always_inline)) {
      if (wave_any(lm[0] > m2s[0] || lm[1] > m2s[1])) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          const float mx = group4_max(lm[qt]);
          const bool first = m2[qt] == kNegInf;
          const bool grow = !first && mx > m2s[qt];
          restart_row = restart_row || grow;
          m2[qt] = (first || grow) ? mx : m2[qt];
          m2s[qt] = m2[qt] + kLatentSlack;
          msub[qt] = (m2[qt] == kNegInf) ? 0.f : m2[qt];
        }
      }
    };
    // the softmax as a list of steps: stages 0 .. 5 of both q-tiles
    // alternating, the check, stages 6 .. 19 alternating
    constexpr int NSTEP = 2 * 6 + 1 + 2 * 14;
    static_assert(NSTEP < kPublishSlot && kPublishSlot < 64, "P^T is published after the last softmax step");
    auto step = [&](auto J_) __attribute__((always_inline)) {
      constexpr int j = decltype(J_)::value;
      if constexpr (j < 12) stage(std::integral_constant<int, j % 2>{}, std::integral_constant<int, j / 2>{});
      else if constexpr (j == 12) check();
      else stage(std::integral_constant<int, (j - 13) % 2>{}, std::integral_constant<int, 6 + (j - 13) / 2>{});
    };
    // the scores must retire before the softmax reads them
    auto scores_retire = [&]() __attribute__((always_inline)) {
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(sacc[0][0]), "+v"(sacc[0][1]), "+v"(sacc[1][0]), "+v"(sacc[1][1]));
    };
    // P^T of this wave's rows to LDS, with their normaliser (two wait states
    // after the VALU writes of the MFMA operands, accumulator included), and
    // the restart request; issued well before the barrier so that the LDS
    // writes drain behind matrix work
    unsigned char* pb = smem + PBASE + (it & 1) * PBUF;
    auto publish = [&]() __attribute__((always_inline)) {
      u32x4 ones = {kBf16OnePair, kBf16OnePair, kBf16OnePair, kBf16OnePair};
      asm volatile("s_nop 1" : "+v"(pf[0]), "+v"(pf[1]), "+v"(ones), "+v"(lacc[0]), "+v"(lacc[1]));
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) mfma_v(lacc[qt], ones, pf[qt]);
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) st16(pb + (2 * wave + qt) * PQT + 16 * lane, pf[qt]);
      // a wave whose rows outgrew their reference asks the whole work-group
      // to start the split again (every wave must run the same tiles and
      // barriers)
      const bool any_restart = wave_any(restart_row);  // all lanes vote, outside the lane-0 branch
      if (lane == 0) restart_flag[it & 1][wave] = any_restart ? 1 : 0;
    };
    if constexpr (kPV) {
      constexpr int NB = 64;  // value MFMAs; step j of the softmax follows MFMA j + 1
      static_for<0, NB>([&](auto M_) __attribute__((always_inline)) {
        constexpr int m = decltype(M_)::value;
        constexpr int dt = m / 8, qt = m % 8;
        if (qt == 0 && dt + 1 < 8) load_v(vb, dt + 1, vf[(dt + 1) & 1]);
        if (m % 16 == 8) dma(dt2, 5 + m / 16);
        mfma_acc(oacc[dt][qt], vf[dt & 1], pall[qt]);
        __builtin_amdgcn_sched_barrier(0);
        if (m == 0) scores_retire();
        if constexpr (m >= 1 && m <= NSTEP) step(std::integral_constant<int, m - 1>{});
        if (m == kPublishSlot) publish();
        __builtin_amdgcn_sched_barrier(0);
      });
    } else {
      scores_retire();
      static_for<0, NSTEP>(step);
#pragma unroll
      for (int j = 5; j < 9; ++j) dma(dt2, j);
      publish();
    }

    if (__builtin_amdgcn_readfirstlane(flags) != 0) return true;
    wait_vmem_but_one_tile();
    __syncthreads();
    flags = *reinterpret_cast<const uint32_t*>(restart_flag[it & 1]);
    return false;
  };

  int it = 0;
  for (;;) {
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) lacc[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int qt = 0; qt < 8; ++qt) oacc[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
    flags = 0;
    {
      const DmaTile d0 = dma_tile(0), d1 = dma_tile(1);
#pragma unroll
      for (int j = 0; j < 9; ++j) dma(d0, j);
#pragma unroll
      for (int j = 0; j < 9; ++j) dma(d1, j);
    }
    wait_vmem_but_one_tile();
    __syncthreads();
    bool restart = iter(0, std::true_type{}, std::false_type{});
    for (it = 1; it < t_mask && !restart; ++it) restart = iter(it, std::false_type{}, std::true_type{});
    for (; it < n_t && !restart; ++it) restart = iter(it, std::true_type{}, std::true_type{});
    if (!restart) restart = __builtin_amdgcn_readfirstlane(flags) != 0;
    // no DMA may still target a slot that is about to be reused, and no wave
    // may still read one
    wait_vmem_all();
    if (!restart) break;
    __syncthreads();
  }
  // values of the last tile
  {
    const uint32_t vb = (uint32_t)((n_t - 1) & 3) * LTILE + vfrag;
    load_p(n_t - 1);
    load_v(vb, 0, vf[0]);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      pv_step(vb, dt);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- partial of this split: normalised output and log2-sum-exp ---------
  // the last accumulator MFMAs must retire before the VALU reads them
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(oacc[7][7]), "+a"(oacc[7][6]), "+v"(lacc[0]), "+v"(lacc[1]));
  // 1 / l of all 128 rows, in the RoPE ring (idle now)
  float* stats = reinterpret_cast<float*>(smem + RBASE);
  const int64_t pbase = ((int64_t)rb * (a.n_wg + a.B) + slot) * ROWS;
  __syncthreads();
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float l = lacc[qt][0];
    const int row = 32 * wave + 16 * qt + li;
    if (lg == 0) {
      stats[row] = l > 0.f ? 1.f / l : 0.f;
      if (row_ok[qt]) a.ws_lse[pbase + row] = l > 0.f ? m2[qt] + fast_log2(l) : kNegInf;
    }
  }
  __syncthreads();
#pragma unroll
  for (int qt = 0; qt < 8; ++qt) {
    const int row = 16 * qt + li;
    if (rb * ROWS + row >= n_rows) continue;
    const float inv = stats[row];
    float* wo = a.ws_o + (pbase + row) * RKV + 128 * wave + 4 * lg;
    // oacc[dt][qt][r] is feature 128 w + 16 dt + 4 lg + r
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      *reinterpret_cast<f32x4*>(wo + 16 * dt) = oacc[dt][qt] * inv;
      if ((dt & 3) == 3) __builtin_amdgcn_sched_barrier(0);
    }
  }
  // the next segment's first DMAs overwrite the statistics
  __syncthreads();
  };

  for (int b = b0; b < a.B && P < hi; ++b) {
    const int L = __builtin_amdgcn_readfirstlane(min(max(a.seqlens[b], 0), a.L_cap));
    const int nt = (L + T - 1) / T;
    const int first = P + X;  // position of the sequence's tile 0
    const int t0 = max(lo, first) - first, t1 = min(hi, first + nt) - first;
    if (t0 < t1) segment(b, L, t0 * T, min(L, t1 * T), w + b);
    P = first + nt;
  }
}

// Merge the segments of a sequence, 4 query rows per work-group (64 threads
// per row, 8 features per thread): each segment s holds its normalised output
// O_s and its log2-sum-exp l_s; the result is
// sum_s 2^(l_s - M) O_s / sum_s 2^(l_s - M).
template <bool OUT_F32>
__global__ __launch_bounds__(256) void latent_merge_kernel(LatentArgs a) {
  const int unit = blockIdx.x / (ROWS / 4);  // b * n_rb + rb
  const int rb = unit % a.n_rb, b = unit / a.n_rb;
  const int tid = threadIdx.x;
  const int row = (blockIdx.x % (ROWS / 4)) * 4 + (tid >> 6);
  const int f = (tid & 63) * 8;
  const int R = rb * ROWS + row;
  if (R >= a.s_q * a.h_q) return;
  // the work-groups whose share of the positions meets this sequence's
  // tiles [p0, p1) (its last positions: the split kernel numbers each
  // sequence's placeholders, then its tiles)
  const int p1 = a.ws_tiles[b + 1], p0 = p1 - latent_tiles(a, b), NV = a.ws_tiles[a.B];
  const int64_t n = a.n_wg;
  int w_first = 0, w_last = -1;
  if (p0 < p1) {
    w_first = (int)(((int64_t)(p0 + 1) * n - 1) / NV);  // last w with w NV / n <= p0
    w_last = (int)(((int64_t)p1 * n - 1) / NV);         // last w with w NV / n < p1
  }
  auto meets = [&](int w) {
    const int lo = (int)(w * (int64_t)NV / n), hi = (int)((w + 1) * (int64_t)NV / n);
    return max(lo, p0) < min(hi, p1);
  };
  const int64_t base = (int64_t)rb * (a.n_wg + a.B) * ROWS + row;
  float M = kNegInf;
  for (int w = w_first; w <= w_last; ++w)
    if (meets(w)) M = fmaxf(M, a.ws_lse[base + (int64_t)(w + b) * ROWS]);
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int w = w_first; w <= w_last; ++w) {
    if (!meets(w)) continue;
    const float ls = a.ws_lse[base + (int64_t)(w + b) * ROWS];
    const float wt = (ls == kNegInf) ? 0.f : fast_exp2(ls - M);
    den += wt;
    const float* src = a.ws_o + (base + (int64_t)(w + b) * ROWS) * RKV + f;
    acc0 += wt * *reinterpret_cast<const f32x4*>(src);
    acc1 += wt * *reinterpret_cast<const f32x4*>(src + 4);
  }
  // a row with no visible token gets zeros (and lse = -inf)
  const float inv = den > 0.f ? 1.f / den : 0.f;
  acc0 *= inv;
  acc1 *= inv;
  const int tq = R / a.h_q, head = R % a.h_q;
  const int64_t obase = (int64_t)b * a.o_sb + (int64_t)head * a.o_sh + (int64_t)tq * a.o_ss + f;
  if constexpr (OUT_F32) {
    *reinterpret_cast<f32x4*>((float*)a.o + obase) = acc0;
    *reinterpret_cast<f32x4*>((float*)a.o + obase + 4) = acc1;
  } else {
    *reinterpret_cast<u32x4*>((__bf16*)a.o + obase) =
        u32x4{pack_bf16(acc0[0], acc0[1]), pack_bf16(acc0[2], acc0[3]), pack_bf16(acc1[0], acc1[1]),
              pack_bf16(acc1[2], acc1[3])};
  }
  if (a.lse != nullptr && (tid & 63) == 0)
    a.lse[((int64_t)b * a.s_q + tq) * a.h_q + head] = den > 0.f ? (M + fast_log2(den)) * kLn2 : kNegInf;
}

}  // namespace

int latent_rows_per_wg() { return ROWS; }
int latent_tile_tokens() { return T; }
int latent_segment_start_tiles() { return kSegStartTiles; }

int latent_plan_wgs(int n_rb, int64_t max_tiles) {
  // one work-group per CU in a single round: equal tile shares then finish
  // together
  int64_t n = std::max<int64_t>(1, 256 / n_rb);
  return (int)std::max<int64_t>(1, std::min<int64_t>(n, max_tiles));
}

hipError_t launch_latent_decode(const LatentArgs& a, bool out_f32, hipStream_t st) {
  const int n_units = a.n_wg * a.n_rb;
  const int padded = (n_units + 7) / 8 * 8;
  hipLaunchKernelGGL(latent_split_kernel, dim3(padded), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (out_f32)
    hipLaunchKernelGGL(latent_merge_kernel<true>, dim3(a.B * a.n_rb * (ROWS / 4)), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(latent_merge_kernel<false>, dim3(a.B * a.n_rb * (ROWS / 4)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace gha
