// Streaming decode over contiguous caches, bf16, split-KV with a
// log-sum-exp merge, for the decode forms that differ only in where a
// group's key and value come from:
//   * GTA shared-score decode ("GTA: Grouped-head latenT Attention" news
//     article, grouped shared attention matrix): per group one query and one
//     cached key (d_qk wide) per token, so one score vector per new token, and
//     the cached values of the group's heads that all use it (value sources
//     of 64 or 128 columns of a head; a group wider than one launch's sources
//     is covered by several launches);
//   * GQLA's GQA-path decode ("GQLA: Group-Query Latent Attention ...",
//     section 1 and section 3.1, Eq. (1)): per group a cached key k^C and a
//     cached value, plus one decoupled RoPE key k^R per token that every group
//     shares (2 g d_h + d^R cached elements per token); each head's key is
//     [k^C_j; k^R];
//   * plain grouped-query decode, with no shared key part.
//
// Decode reads the whole cache once per step, so the kernel streams, with one
// work-group (four waves, one per SIMD) per CU in a single round: the keys of
// every unit are cut into 128-key chunks, all units' chunks are numbered one
// after another, and teams of Z work-groups take equal shares of them whatever
// the length mix.  Without a shared key part Z = 1 and a unit is one
// (sequence, group); with one, Z = G, a unit is a sequence, and member j of a
// team serves group j, so a team's members walk the same keys together on one
// XCD and the shared key rows meet in its L2.  Each unit a share touches is a
// segment with its own partial; inside a segment every wave walks its own
// tiles (tiles w, w + 4, ...).
// A wave moves its tiles from HBM into a private LDS ring by buffer DMA
// (buffer_load ... lds; no VGPR staging; non-temporal, as every tile of a
// group's key and value is read once per step), keeps NSLOT - 1 tiles in flight
// while it computes on the oldest, and never waits for another wave until the
// end.  Per tile, with all query rows of the group (the query heads times the
// s_q new tokens, padded to 16 or 32) in one wave:
//   S^T = K Q^T from 16-byte LDS reads of the key rows (group part, then shared
//   part), online softmax with a lazily moved running maximum, and
//   O^T += V^T P^T with V^T fragments from transposing LDS reads; the score
//   accumulator is the P^T operand, no data movement.
// The waves combine through LDS at the end and write one normalised partial
// plus its log2-sum-exp per segment; a second kernel merges the segments of
// each unit.
//
// LDS rows keep their 16-byte units swizzled so that fragment reads touch
// distinct banks: key rows of 128 B keep unit u at u ^ ((r / 2) % 8) and of
// 256 B at u ^ (r % 16) (16 rows of one unit per read); value rows of 128 B
// keep u at u ^ 2 ((r / 2) % 4) and of 256 B at u ^ 2 (r % 8) (a transposing
// read takes 32 B from each of 8 consecutive rows per half-wave).
#include "device_common.hpp"
#include "kernels.hpp"
#include "lds_pipe.hpp"

namespace gha {
namespace {

// T keys per tile: 32 (one 16x16x32 value MFMA step) or 16 (one 16x16x16
// step), whichever lets a wave keep more tiles in flight.  EB is the bytes
// per cached element: 2 (bf16 tiles feed the MFMAs straight from the ring)
// or 1 (8-bit tiles land in the ring and are converted to bf16 in registers
// as the MFMAs read them: keys by plain reads, values by 8-bit transposing
// reads).
template <int DK1, int DK2, int DVW, int NVS, int T, int EB = 2>
struct SdLayout {
  // the bf16 tile the MFMAs read (swizzled rows)
  static constexpr int K1ROW = 2 * DK1, K2ROW = 2 * DK2, VROW = 2 * DVW;
  static constexpr int K1B = T * K1ROW, K2B = T * K2ROW, VB = T * VROW;
  static constexpr int TILE = K1B + K2B + NVS * VB;
  // the tile as it arrives from HBM
  static constexpr int RK1ROW = EB * DK1, RK2ROW = EB * DK2, RVROW = EB * DVW;
  static constexpr int RK1B = T * RK1ROW, RK2B = T * RK2ROW, RVB = T * RVROW;
  static constexpr int SLOT = RK1B + RK2B + NVS * RVB;          // one ring slot
  static constexpr int STAGE = 0;  // (no staging: every tile is read where it lands)
  // LDS per work-group: all of a CU's for 16-bit tiles (one work-group per
  // CU); half for 8-bit ones, so that two work-groups share a CU and one's
  // conversions and softmax run beside the other's MFMAs
  static constexpr int BUDGET = EB == 1 ? 80 * 1024 : 160 * 1024;
  // four waves per work-group when each can keep two tiles, else two
  static constexpr int NW = 4 * (2 * SLOT + STAGE) <= BUDGET ? 4 : 2;
  static constexpr int NSLOT_FIT = (BUDGET / NW - STAGE) / SLOT;
  static constexpr int NSLOT = NSLOT_FIT > 6 ? 6 : NSLOT_FIT;  // ring slots per wave
  static constexpr int WAVE = NSLOT * SLOT + STAGE;
  static constexpr int BYTES = NW * WAVE;
  static constexpr int NK1 = RK1B / 1024, NK2 = RK2B / 1024, NV = RVB / 1024;
  static constexpr int NDMA = NK1 + NK2 + NVS * NV;            // DMA instructions per tile
  static constexpr int DV = NVS * DVW;                         // output width of a row
};

constexpr int CH = 128;  // keys per scheduling chunk

// first key any query row of a length-L sequence sees (sliding window), and
// the chunk-aligned key the chunks of that sequence start from
__device__ __forceinline__ int sd_first_key(const StreamDecodeArgs& a, int L) {
  return a.window > 0 ? max(0, L - a.s_q + 1 - a.window) : 0;
}
__device__ __forceinline__ int sd_chunk0(const StreamDecodeArgs& a, int L) { return sd_first_key(a, L) / CH * CH; }
// chunks of sequence b (0 past the batch); lengths are clamped to [0, L_cap]
__device__ __forceinline__ int sd_chunks(const StreamDecodeArgs& a, int b) {
  if (b >= a.B) return 0;
  const int L = min(max(a.seqlens[b], 0), a.L_cap);
  return (L - sd_chunk0(a, L) + CH - 1) / CH;
}

template <int DK1, int DK2, int DVW, int NVS, int EB = 2>
constexpr int sd_tile_keys() {
  return EB == 1 ? 16 : (SdLayout<DK1, DK2, DVW, NVS, 32, EB>::NSLOT >= 3 ? 32 : 16);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
// v_mfma_f32_16x16x16_bf16: lane (i, g) supplies A[i][4g .. 4g + 3] and
// B[4g .. 4g + 3][i], and receives D[4g + r][i] as the 16x16x32 form does
__device__ __forceinline__ f32x4 mfma_k16(const u32x2& a, const u32x2& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// One int32 through the scalar cache, waited for in the same asm block.  A
// plain load of the block table becomes a vector load here (the compiler
// cannot prove the table unwritten), and waiting for it would wait for every
// tile DMA in flight.
__device__ __forceinline__ int scalar_load_i32(const int32_t* p) {
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}

// unit swizzles (see above)
__device__ __forceinline__ int key_swz(int row_bytes, int r) { return row_bytes == 128 ? ((r >> 1) & 7) : (r & 15); }
__device__ __forceinline__ int val_swz(int row_bytes, int r) { return row_bytes == 128 ? 2 * ((r >> 1) & 3) : 2 * (r & 7); }
// 8-bit key rows (128 or 64 B): 16-byte unit u of row r at u ^ k8_swz; an
// 8-byte fragment read of 16 rows then covers distinct banks
__device__ __forceinline__ int k8_swz(int row_bytes, int r) { return row_bytes == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
// 8-bit value rows: unit u of row r at u ^ v8_swz; a transposing read takes
// 32 B (two units) from each of 8 rows per half-wave, in distinct banks
__device__ __forceinline__ int v8_swz(int row_bytes, int r) { return row_bytes == 128 ? 2 * ((r >> 1) & 3) : 2 * ((r >> 2) & 1); }

template <int DK1, int DK2, int DVW, int NVS, int T, int QT, int EB>
__global__ __launch_bounds__((64 * SdLayout<DK1, DK2, DVW, NVS, T, EB>::NW), 1)
void stream_decode_split_kernel(StreamDecodeArgs a) {
  using Ly = SdLayout<DK1, DK2, DVW, NVS, T, EB>;
  static_assert(EB == 2 || (EB == 1 && DK2 == 0 && NVS == 1 && DK1 == DVW), "8-bit caches: one key part, one value");
  constexpr int NWAVE = Ly::NW;
  constexpr int KT = T / 16;  // 16-key score tiles per tile
  static_assert(T == 16 || T == 32, "tile keys");
  constexpr int DS1 = DK1 / 32, DS = (DK1 + DK2) / 32;  // score contraction steps
  constexpr int NCT = DVW / 16;                         // 16-wide column tiles per value source
  constexpr int NSLOT = Ly::NSLOT;
  static_assert(NSLOT >= 2, "LDS ring");
  static_assert(DK1 == 64 || DK1 == 128, "group key width");
  static_assert(DK2 == 0 || DK2 == 64, "shared key width");
  static_assert(DVW == 64 || DVW == 128, "value width");
  static_assert(Ly::NDMA * (NSLOT - 1) < 64, "vmcnt range");

  __shared__ __attribute__((aligned(1024))) unsigned char smem[Ly::BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;

  // ---- this team's equal share of all chunks -----------------------------------
  // Unit (b, jb), jb < G / Z, has ceil(L_b / 128) chunks; team t (work-groups
  // t Z .. t Z + Z - 1; member m serves group jb Z + m) takes chunks
  // [t NT / n_teams, (t + 1) NT / n_teams) of the NT in all.
  const int G = a.n_groups, Z = a.team, GZ = G / Z;
  const int wid = (int)xcd_logical_id(blockIdx.x, gridDim.x);
  if (wid >= a.n_wg) return;
  const int n_teams = a.n_wg / Z;
  const int team = wid / Z, m = wid % Z;
  int NT = 0;
  for (int c0 = 0; c0 < a.B; c0 += 64)
    NT += __builtin_amdgcn_readlane(wave_incl_scan(sd_chunks(a, c0 + lane) * GZ), 63);
  NT = __builtin_amdgcn_readfirstlane(NT);
  const int lo = (int)((int64_t)team * NT / n_teams), hi = (int)((int64_t)(team + 1) * NT / n_teams);
  // one work-group publishes the per-sequence prefix sums for the merge
  if (wid == 0 && wave == 0) {
    int run = 0;
    for (int c0 = 0; c0 < a.B; c0 += 64) {
      const int t = sd_chunks(a, c0 + lane) * GZ;
      const int incl = wave_incl_scan(t) + run;
      if (c0 + lane < a.B) a.ws_pref[c0 + lane] = incl - t;
      run = __builtin_amdgcn_readlane(incl, 63);
    }
    if (lane == 0) a.ws_pref[a.B] = run;
  }
  if (lo >= hi) return;
  // first sequence whose chunks reach past lo, and the chunks before it
  int b0 = 0, P0 = 0;
  for (int c0 = 0;; c0 += 64) {
    const int t = sd_chunks(a, c0 + lane) * GZ;
    const int incl = wave_incl_scan(t) + P0;
    const uint64_t m = __builtin_amdgcn_ballot_w64(incl > lo);
    if (m != 0) {
      const int f = __builtin_ctzll(m);
      b0 = c0 + f;
      P0 = __builtin_amdgcn_readlane(incl - t, f);
      break;
    }
    P0 = __builtin_amdgcn_readlane(incl, 63);
  }
  b0 = __builtin_amdgcn_readfirstlane(b0);
  P0 = __builtin_amdgcn_readfirstlane(P0);

  // ---- one segment: unit (b, j), keys [start, end), partial slot ----------------
  auto segment = [&](int b, int j, int L, int start, int end, int slot) __attribute__((always_inline)) {
  const int n_tiles = (end - start + T - 1) / T;
  const int n_my = (n_tiles - wave + NWAVE - 1) / NWAVE;  // tiles w, w + 4, ... of the segment

  // ---- query rows: R = hh * s_q + t, head j * qpg + hh -----------------------
  u32x4 qf[QT][DS];
  int kvis[QT], kmin[QT];  // last and first key each lane's row sees (bottom-right causal, window)
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int R = 16 * qt + li;
    const bool ok = R < a.rows;
    const int hh = ok ? R / a.s_q : 0, tq = ok ? R % a.s_q : 0;
    kvis[qt] = L - a.s_q + tq;
    kmin[qt] = a.window > 0 ? kvis[qt] - a.window + 1 : 0;
    const int head = j * a.qpg + hh;
    const __bf16* qp = (const __bf16*)a.q + (int64_t)b * a.q_sb + (int64_t)head * a.q_sh + (int64_t)tq * a.q_ss;
#pragma unroll
    for (int s = 0; s < DS1; ++s) qf[qt][s] = ok ? ld16(qp + 32 * s + 8 * lg) : u32x4{0u, 0u, 0u, 0u};
    if constexpr (DK2 > 0) {
      const __bf16* qp2 = (const __bf16*)a.q2 + (int64_t)b * a.q2_sb + (int64_t)head * a.q2_sh + (int64_t)tq * a.q2_ss;
#pragma unroll
      for (int s = DS1; s < DS; ++s) qf[qt][s] = ok ? ld16(qp2 + 32 * (s - DS1) + 8 * lg) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  wait_vmem_all();
  const float c2 = a.scale * kLog2e;

  // ---- tile DMAs into this wave's ring -------------------------------------------
  // Each source is a buffer whose range ends at this sequence's last token:
  // rows past it read as zeros.  One instruction moves 1 KiB: 1024 / row_bytes
  // rows, lane l taking row l / (row_bytes / 16), unit position
  // l % (row_bytes / 16) and fetching the global unit that belongs there.
  const uint32_t k1row = (uint32_t)a.k_ss * EB, k2row = (uint32_t)a.k2_ss * EB, vrow = (uint32_t)a.v_ss * EB;
  const uint32_t lastk = (uint32_t)(L - 1);
  // (strides count elements of EB bytes)
  const __amdgpu_buffer_rsrc_t k1rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const unsigned char*)a.k + ((int64_t)b * a.k_sb + (int64_t)j * a.k_sh) * EB), 0,
      (int)(lastk * k1row + (uint32_t)Ly::RK1ROW), kBufferFlags);
  __amdgpu_buffer_rsrc_t k2rs = k1rs;
  if constexpr (DK2 > 0)
    k2rs = __builtin_amdgcn_make_buffer_rsrc((void*)((const __bf16*)a.k2 + (int64_t)b * a.k2_sb), 0,
                                             (int)(lastk * k2row + (uint32_t)Ly::RK2ROW), kBufferFlags);
  __amdgpu_buffer_rsrc_t vrs[NVS];
#pragma unroll
  for (int vs = 0; vs < NVS; ++vs)
    vrs[vs] = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const unsigned char*)a.v +
                ((int64_t)b * a.v_sb + (int64_t)(j * a.v_hpg + vs / a.v_sph) * a.v_sh + (vs % a.v_sph) * DVW) * EB),
        0,
        (int)(lastk * vrow + (uint32_t)Ly::RVROW), kBufferFlags);
  // per-lane offsets of the instructions of one tile (they repeat every tile)
  auto lane_ofs = [&](int row_bytes, uint32_t gl_row, int n, bool is_key) -> uint32_t {
    const int upr = row_bytes / 16, rpi = 1024 / row_bytes;
    const int r = n * rpi + lane / upr;  // row in the tile
    const int sw = EB == 1 ? (is_key ? k8_swz(row_bytes, r) : v8_swz(row_bytes, r))
                           : (is_key ? key_swz(row_bytes, r) : val_swz(row_bytes, r));
    return (uint32_t)r * gl_row + 16u * (uint32_t)((lane % upr) ^ sw);
  };
  uint32_t k1o[Ly::NK1], k2o[Ly::NK2 > 0 ? Ly::NK2 : 1], vo[Ly::NV];
#pragma unroll
  for (int n = 0; n < Ly::NK1; ++n) k1o[n] = lane_ofs(Ly::RK1ROW, k1row, n, true);
#pragma unroll
  for (int n = 0; n < Ly::NK2; ++n) k2o[n] = lane_ofs(Ly::RK2ROW, k2row, n, true);
#pragma unroll
  for (int n = 0; n < Ly::NV; ++n) vo[n] = lane_ofs(Ly::RVROW, vrow, n, false);
  const uint32_t ring = lds_offset(smem) + wave * Ly::WAVE;
  const int klo = sd_first_key(a, L);
  // tile i of this wave (global tile i * 4 + w of the split) into slot i % NSLOT;
  // tiles past the split or wholly before the window read out of range
  // (zeros), keeping DMA counts uniform
  auto issue_tile = [&](int i) __attribute__((always_inline)) {
    const int key0 = start + (i * NWAVE + wave) * T;
    const bool ok = i < n_my && key0 + T > klo;
    const uint32_t dst = ring + (uint32_t)(i % NSLOT) * Ly::SLOT;
    if constexpr (DK2 == 0 && NVS == 1) {
      if (a.block_table != nullptr) {
        // the tile lies in one page (page_size is a multiple of 32 and tiles
        // start at multiples of T); each tile gets buffers whose range ends at
        // the page's last token of the sequence
        int pidx = 0, rows = 0, u = 0;
        if (ok) {
          const int pg = key0 / a.page_size;
          pidx = scalar_load_i32(a.block_table + __builtin_amdgcn_readfirstlane(b * a.bt_stride + pg));
          rows = min(a.page_size, L - pg * a.page_size);
          u = key0 - pg * a.page_size;
        }
        const __amdgpu_buffer_rsrc_t kp = __builtin_amdgcn_make_buffer_rsrc(
            (void*)((const unsigned char*)a.k + ((int64_t)pidx * a.k_sb + (int64_t)j * a.k_sh) * EB), 0,
            rows > 0 ? (int)((uint32_t)(rows - 1) * k1row + (uint32_t)Ly::RK1ROW) : 0, kBufferFlags);
        const __amdgpu_buffer_rsrc_t vp = __builtin_amdgcn_make_buffer_rsrc(
            (void*)((const unsigned char*)a.v + ((int64_t)pidx * a.v_sb + (int64_t)j * a.v_sh) * EB), 0,
            rows > 0 ? (int)((uint32_t)(rows - 1) * vrow + (uint32_t)Ly::RVROW) : 0, kBufferFlags);
#pragma unroll
        for (int n = 0; n < Ly::NK1; ++n)
          lds_dma16_stream(kp, dst + 1024 * n, k1o[n], ok ? (uint32_t)u * k1row : kOutOfRange);
#pragma unroll
        for (int n = 0; n < Ly::NV; ++n)
          lds_dma16_stream(vp, dst + Ly::RK1B + 1024 * n, vo[n], ok ? (uint32_t)u * vrow : kOutOfRange);
        return;
      }
    }
#pragma unroll
    for (int n = 0; n < Ly::NK1; ++n)
      lds_dma16_stream(k1rs, dst + 1024 * n, k1o[n], ok ? (uint32_t)key0 * k1row : kOutOfRange);
    // the shared key part is read by every group of the team through L2
#pragma unroll
    for (int n = 0; n < Ly::NK2; ++n)
      lds_dma16(k2rs, dst + Ly::RK1B + 1024 * n, k2o[n], ok ? (uint32_t)key0 * k2row : kOutOfRange);
#pragma unroll
    for (int vs = 0; vs < NVS; ++vs)
#pragma unroll
      for (int n = 0; n < Ly::NV; ++n)
        lds_dma16_stream(vrs[vs], dst + Ly::RK1B + Ly::RK2B + vs * Ly::RVB + 1024 * n, vo[n], ok ? (uint32_t)key0 * vrow : kOutOfRange);
  };

  // ---- fragment addresses ----------------------------------------------------------
  // score A operand, key row 16 kt + li, unit 4 s + lg of a part with
  // row_bytes: (frag ^ 64 s) + 16 row_bytes kt
  auto key_frag = [&](int row_bytes) -> uint32_t {
    return row_bytes == 128 ? li * 128 + 16 * (lg ^ ((li >> 1) & 7)) : li * 256 + 16 * (lg ^ li);
  };
  const uint32_t kf1 = key_frag(Ly::K1ROW);
  const uint32_t kf2 = DK2 > 0 ? key_frag(Ly::K2ROW) : 0u;
  // value A operand (transposing read), source lane li of group lg: row
  // 16 h + 4 lg + li / 4, columns 16 ct + 4 (li % 4) .. + 3:
  // (vfrag ^ 32 ct) + 16 row_bytes h
  uint32_t vfrag;
  {
    const int vr = 4 * lg + (li >> 2);
    const uint32_t in_row = 16 * ((li >> 1) & 1) + 8 * (li & 1);
    vfrag = Ly::VROW == 128 ? vr * 128 + 32 * ((vr >> 1) & 3) + in_row
                            : (vr * 256 + in_row) ^ (32 * (vr & 7));
  }

  // ---- running state (per lane: one row per q-tile) ------------------------------
  f32x4 oacc[NVS][NCT][QT], lacc[QT];
  float m2[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    lacc[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m2[qt] = kNegInf;
#pragma unroll
    for (int vs = 0; vs < NVS; ++vs)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) oacc[vs][ct][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const u32x4 ones = {kBf16OnePair, kBf16OnePair, kBf16OnePair, kBf16OnePair};

#pragma unroll
  for (int i = 0; i < NSLOT - 1; ++i) issue_tile(i);
  // tile i of this wave: keys start + (i NWAVE + wave) T ..; the mask is
  // applied only where some row may not see a key of the tile
  auto tile = [&](int i, auto masked_) __attribute__((always_inline)) {
    constexpr bool kMasked = decltype(masked_)::value;
    issue_tile(i + NSLOT - 1);                       // into the slot of tile i - 1
    wait_vmem_at_most<Ly::NDMA * (NSLOT - 1)>();     // tile i has landed
    const unsigned char* sl = smem + wave * Ly::WAVE + (i % NSLOT) * Ly::SLOT;
    auto cvt_lo = [](uint32_t w) -> uint32_t {  // E4M3 codes 0, 1 of the word as two bf16
      return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
    };
    auto cvt_hi = [](uint32_t w) -> uint32_t {  // codes 2, 3
      return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
    };
    const int key0 = start + (i * NWAVE + wave) * T;

    // S^T = K Q^T: keys key0 + 16 kt + 4 lg + r in sacc[kt][qt][r]
    f32x4 sacc[KT][QT];
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      u32x4 kf[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        if constexpr (EB == 1) {
          // 8 codes of key row 16 kt + li (dims 32 s + 8 lg ..): unit
          // 2 s + lg / 2 of the 8-bit row, half lg % 2, converted in registers
          const int r = 16 * kt + li;
          const u32x2 w = *reinterpret_cast<const u32x2*>(
              sl + r * Ly::RK1ROW + 16 * ((2 * s + (lg >> 1)) ^ k8_swz(Ly::RK1ROW, r)) + 8 * (lg & 1));
          kf[kt] = u32x4{cvt_lo(w[0]), cvt_hi(w[0]), cvt_lo(w[1]), cvt_hi(w[1])};
        } else if (s < DS1) {
          kf[kt] = ld16(sl + kt * 16 * Ly::K1ROW + (kf1 ^ (64u * s)));
        } else {
          kf[kt] = ld16(sl + Ly::K1B + kt * 16 * Ly::K2ROW + (kf2 ^ (64u * (s - DS1))));
        }
      }
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          sacc[kt][qt] = mfma_bf16(kf[kt], qf[qt][s], s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sacc[kt][qt]);
    }


    // online softmax per row, running maximum moved lazily (log2 units); the
    // bf16 probabilities of a row are the value MFMA's P^T operand as they lie
    std::conditional_t<T == 32, u32x4, u32x2> pf[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float mx = kNegInf;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = key0 + 16 * kt + 4 * lg + r;
          if (kMasked && (key >= end || key > kvis[qt] || key < kmin[qt])) sacc[kt][qt][r] = kNegInf;
          mx = fmaxf(mx, sacc[kt][qt][r]);
        }
      const float mx2 = group4_max(mx) * c2;
      if (wave_any(mx2 > m2[qt] + kRescaleSlack)) {
        const float mnew = fmaxf(m2[qt], mx2);
        const float alpha = (mnew == kNegInf) ? 1.f : fast_exp2(m2[qt] - mnew);
        m2[qt] = mnew;
        lacc[qt] *= alpha;
#pragma unroll
        for (int vs = 0; vs < NVS; ++vs)
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) oacc[vs][ct][qt] *= alpha;
      }
      const float msub = (m2[qt] == kNegInf) ? 0.f : m2[qt];
      float p[KT][4];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) p[kt][r] = fast_exp2(__builtin_fmaf(sacc[kt][qt][r], c2, -msub));
      if constexpr (T == 32) {
        pf[qt] = u32x4{pack_bf16(p[0][0], p[0][1]), pack_bf16(p[0][2], p[0][3]),
                       pack_bf16(p[KT - 1][0], p[KT - 1][1]), pack_bf16(p[KT - 1][2], p[KT - 1][3])};
        lacc[qt] = mfma_bf16(ones, pf[qt], lacc[qt]);
      } else {
        pf[qt] = u32x2{pack_bf16(p[0][0], p[0][1]), pack_bf16(p[0][2], p[0][3])};
        lacc[qt] = mfma_k16(u32x2{kBf16OnePair, kBf16OnePair}, pf[qt], lacc[qt]);
      }
    }

    // O^T += V^T P^T for every value source and column tile
    if constexpr (EB == 1) {
      // 8-bit values (one source, 16-key tiles): one transposing read per
      // pair of column tiles.  Within each 16-lane group g, ds_read_b64_tr_b8
      // hands destination lane t, as byte j, byte t % 8 of the 8 bytes that
      // source lane 2 j + t / 8 points at.  Source lane 2 j + p of group g
      // points at key row 4 g + j % 4, dims c + 8 p, c = 16 ct for j < 4 and
      // 16 (ct + 1) for j >= 4; lane t so receives keys 4 g .. 4 g + 3 of dim
      // 16 ct + t (bytes 0..3) and of dim 16 (ct + 1) + t (bytes 4..7): the
      // A operands of both tiles, converted in registers.
      static_assert(T == 16 && NVS == 1 && NCT % 2 == 0, "8-bit values");
      const int j = li >> 1;
      const int vrow = 4 * lg + (j & 3);
      const unsigned char* vbase = sl + Ly::RK1B + vrow * Ly::RVROW + 8 * (li & 1);
      const int vsw = v8_swz(Ly::RVROW, vrow);
#pragma unroll
      for (int ct = 0; ct < NCT; ct += 2) {
        const u32x2 w = ld_tr8(vbase + 16 * ((ct + (j >> 2)) ^ vsw));
        const u32x2 a0 = {cvt_lo(w[0]), cvt_hi(w[0])}, a1 = {cvt_lo(w[1]), cvt_hi(w[1])};
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          oacc[0][ct][qt] = mfma_k16(a0, pf[qt], oacc[0][ct][qt]);
          oacc[0][ct + 1][qt] = mfma_k16(a1, pf[qt], oacc[0][ct + 1][qt]);
        }
      }
    } else {
#pragma unroll
      for (int vs = 0; vs < NVS; ++vs)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const unsigned char* vp = sl + Ly::K1B + Ly::K2B + vs * Ly::VB + (vfrag ^ (32u * ct));
          const u32x2 h0 = ld_tr(vp);
          if constexpr (T == 32) {
            const u32x2 h1 = ld_tr(vp + 16 * Ly::VROW);
            const u32x4 vt = {h0[0], h0[1], h1[0], h1[1]};
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) oacc[vs][ct][qt] = mfma_bf16(vt, pf[qt], oacc[vs][ct][qt]);
          } else {
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) oacc[vs][ct][qt] = mfma_k16(h0, pf[qt], oacc[vs][ct][qt]);
          }
        }
    }
  };
  // Keys below safe_end are visible to every row (s_q new tokens: row t sees
  // up to L - s_q + t) and inside the segment; keys from kmin_top on are
  // inside every row's window.  The tiles wholly in [kmin_top, safe_end) are
  // consecutive for each wave and skip the mask.
  {
    const int safe_end = min(end, L - a.s_q + 1);
    const int kmin_top = a.window > 0 ? L - a.window : 0;
    const int step = NWAVE * T, first = start + wave * T;  // key0 of tile i: first + i step
    int i_lo = kmin_top > first ? (kmin_top - first + step - 1) / step : 0;
    int i_hi = safe_end - first - T >= 0 ? (safe_end - first - T) / step + 1 : 0;
    i_lo = __builtin_amdgcn_readfirstlane(min(i_lo, n_my));
    i_hi = __builtin_amdgcn_readfirstlane(max(i_lo, min(i_hi, n_my)));
    int i = 0;
    for (; i < i_lo; ++i) tile(i, std::true_type{});
    for (; i < i_hi; ++i) tile(i, std::false_type{});
    for (; i < n_my; ++i) tile(i, std::true_type{});
  }
  // no DMA of this wave may still land in the ring, which now holds the
  // combination buffers
  wait_vmem_all();
  __syncthreads();

  // ---- combine the four waves: per row M = max m_w, weights 2^(m_w - M) ----------
  constexpr int RP = 16 * QT;               // padded rows
  constexpr int DV = Ly::DV;
  constexpr int OP = DV + 4;                // row pitch in floats (spreads banks)
  float* s_o = reinterpret_cast<float*>(smem);                 // [4][RP][OP]
  float* s_m = s_o + NWAVE * RP * OP;                          // [4][RP]
  float* s_l = s_m + NWAVE * RP;                               // [4][RP]
  static_assert((NWAVE * RP * OP + 2 * NWAVE * RP) * 4 <= Ly::BYTES, "combine buffers");
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int row = 16 * qt + li;
    if (lg == 0) {
      s_m[wave * RP + row] = m2[qt];
      s_l[wave * RP + row] = lacc[qt][0];
    }
    // oacc[vs][ct][qt][r] is feature vs * DVW + 16 ct + 4 lg + r of the row
#pragma unroll
    for (int vs = 0; vs < NVS; ++vs)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        *reinterpret_cast<f32x4*>(&s_o[(wave * RP + row) * OP + vs * DVW + 16 * ct + 4 * lg]) = oacc[vs][ct][qt];
  }
  __syncthreads();
  constexpr int TPR = 64 * NWAVE / RP, FPT = DV / TPR;  // threads per row, features per thread
  static_assert(FPT % 4 == 0, "features per thread");
  const int row = tid / TPR, f0 = (tid % TPR) * FPT;
  if (row < a.rows) {
    float M = kNegInf;
#pragma unroll
    for (int v = 0; v < NWAVE; ++v) M = fmaxf(M, s_m[v * RP + row]);
    float wt[NWAVE], Lsum = 0.f;
#pragma unroll
    for (int v = 0; v < NWAVE; ++v) {
      const float mw = s_m[v * RP + row];
      wt[v] = (mw == kNegInf) ? 0.f : fast_exp2(mw - M);
      Lsum += wt[v] * s_l[v * RP + row];
    }
    // (8-bit values carry their tensor scale, applied here)
    const float inv = (Lsum > 0.f ? 1.f / Lsum : 0.f) * (EB == 1 ? a.v_scale : 1.f);
    const int64_t pidx = (int64_t)slot * RP + row;
    float* wo = a.ws_o + pidx * DV + f0;
#pragma unroll
    for (int f = 0; f < FPT; f += 4) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < NWAVE; ++v) acc += wt[v] * *reinterpret_cast<const f32x4*>(&s_o[(v * RP + row) * OP + f0 + f]);
      *reinterpret_cast<f32x4*>(wo + f) = acc * inv;
    }
    if (tid % TPR == 0) a.ws_lse[pidx] = Lsum > 0.f ? M + fast_log2(Lsum) : kNegInf;
  }
  // the next segment's DMAs overwrite the combination buffers
  __syncthreads();
  };

  // partial slot (t + b GZ + jb) Z + m: unique, since along a team's segments
  // the unit index b GZ + jb grows and across teams t grows with it never
  // falling
  for (int b = b0, P = P0; b < a.B && P < hi; ++b) {
    const int L = __builtin_amdgcn_readfirstlane(min(max(a.seqlens[b], 0), a.L_cap));
    const int kc = sd_chunk0(a, L);
    const int c = (L - kc + CH - 1) / CH;
    for (int jb = 0; jb < GZ; ++jb) {
      const int U0 = P + jb * c;
      const int s0 = max(lo, U0), s1 = min(hi, U0 + c);
      if (s0 < s1)
        segment(b, jb * Z + m, L, kc + (s0 - U0) * CH, min(L, kc + (s1 - U0) * CH), (team + b * GZ + jb) * Z + m);
    }
    P += c * GZ;
  }
}

// Merge the segments of one (sequence, group): the teams whose chunk share
// meets the unit's chunks each left a normalised output O_s and log2-sum-exp
// l_s in slot (t + u) Z + m; the result is
// sum_s 2^(l_s - M) O_s / sum_s 2^(l_s - M), M = max_s l_s.
template <int DV, int DVW, int QT, bool OUT_F32>
__global__ __launch_bounds__(256) void stream_decode_merge_kernel(StreamDecodeArgs a) {
  constexpr int RP = 16 * QT, TPR = 256 / RP, FPT = DV / TPR;
  const int unit = blockIdx.x;
  const int j = unit % a.n_groups, b = unit / a.n_groups;
  const int tid = threadIdx.x;
  const int row = tid / TPR, f0 = (tid % TPR) * FPT;
  if (row >= a.rows) return;
  const int Z = a.team, GZ = a.n_groups / Z, jb = j / Z, m = j % Z;
  const int c = sd_chunks(a, b);
  const int p0 = a.ws_pref[b] + jb * c, p1 = p0 + c, NT = a.ws_pref[a.B];
  const int64_t u = (int64_t)b * GZ + jb;
  const int64_t n = a.n_wg / Z;
  int w_first = 0, w_last = -1;
  if (p0 < p1) {
    w_first = (int)(((int64_t)(p0 + 1) * n - 1) / NT);  // last w with w NT / n <= p0
    w_last = (int)(((int64_t)p1 * n - 1) / NT);         // last w with w NT / n < p1
  }
  auto meets = [&](int w) {
    const int lo = (int)(w * (int64_t)NT / n), hi = (int)((w + 1) * (int64_t)NT / n);
    return max(lo, p0) < min(hi, p1);
  };
  float M = kNegInf;
  for (int t = w_first; t <= w_last; ++t)
    if (meets(t)) M = fmaxf(M, a.ws_lse[((t + u) * Z + m) * RP + row]);
  float acc[FPT];
#pragma unroll
  for (int f = 0; f < FPT; ++f) acc[f] = 0.f;
  float den = 0.f;
  for (int s = w_first; s <= w_last; ++s) {
    if (!meets(s)) continue;
    const int64_t base = ((s + u) * Z + m) * RP + row;
    const float ls = a.ws_lse[base];
    const float w = (ls == kNegInf) ? 0.f : fast_exp2(ls - M);
    den += w;
    const float* src = a.ws_o + base * DV + f0;
#pragma unroll
    for (int f = 0; f < FPT; f += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(src + f);
      acc[f] += w * x[0]; acc[f + 1] += w * x[1]; acc[f + 2] += w * x[2]; acc[f + 3] += w * x[3];
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const int hh = row / a.s_q, tq = row % a.s_q;
  const int qhead = j * a.qpg + hh;
#pragma unroll
  for (int f = 0; f < FPT; f += 4) {
    // features f0 + f .. + 3 lie in one value source (DVW is a multiple of FPT)
    const int fe = f0 + f, src = fe / DVW;
    const int head = qhead * a.v_hpg + src / a.v_sph;
    const int64_t o = (int64_t)b * a.o_sb + (int64_t)head * a.o_sh + (int64_t)tq * a.o_ss +
                      (src % a.v_sph) * DVW + fe % DVW;
    if constexpr (OUT_F32)
      *reinterpret_cast<f32x4*>((float*)a.o + o) = f32x4{acc[f] * inv, acc[f + 1] * inv, acc[f + 2] * inv, acc[f + 3] * inv};
    else
      *reinterpret_cast<u32x2*>((__bf16*)a.o + o) =
          u32x2{pack_bf16(acc[f] * inv, acc[f + 1] * inv), pack_bf16(acc[f + 2] * inv, acc[f + 3] * inv)};
  }
  if (a.lse != nullptr && tid % TPR == 0)
    a.lse[((int64_t)b * a.n_groups * a.qpg + qhead) * a.s_q + tq] = den > 0.f ? (M + fast_log2(den)) * kLn2 : kNegInf;
}

template <int DK1, int DK2, int DVW, int NVS, int QT, int EB>
hipError_t launch_cfg(const StreamDecodeArgs& a, bool out_f32, hipStream_t st) {
  constexpr int DV = NVS * DVW;
  constexpr int T = sd_tile_keys<DK1, DK2, DVW, NVS, EB>();
  const uint32_t padded = (uint32_t)(a.n_wg + 7) / 8 * 8;
  hipLaunchKernelGGL((stream_decode_split_kernel<DK1, DK2, DVW, NVS, T, QT, EB>), dim3(padded),
                     dim3(64 * SdLayout<DK1, DK2, DVW, NVS, T, EB>::NW), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (out_f32)
    hipLaunchKernelGGL((stream_decode_merge_kernel<DV, DVW, QT, true>), dim3(a.B * a.n_groups), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((stream_decode_merge_kernel<DV, DVW, QT, false>), dim3(a.B * a.n_groups), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int DK1, int DK2, int DVW, int NVS, int EB = 2>
hipError_t launch_qt(const StreamDecodeArgs& a, bool out_f32, hipStream_t st) {
  if (a.rows <= 16) return launch_cfg<DK1, DK2, DVW, NVS, 1, EB>(a, out_f32, st);
  // 32 rows keep an accumulator of NVS * DVW / 16 tiles per q-tile: at most
  // 256 columns, so that it fits the accumulation registers
  if constexpr (NVS * DVW <= 256)
    if (a.rows <= 32) return launch_cfg<DK1, DK2, DVW, NVS, 2, EB>(a, out_f32, st);
  return hipErrorInvalidValue;
}

}  // namespace

int stream_decode_chunk() { return CH; }

hipError_t launch_stream_decode(const StreamDecodeArgs& a, int dk1, int dk2, int dvw, int nvs, bool out_f32,
                                hipStream_t st, bool fp8) {
  if (fp8) {
    if (dk1 == 64 && dk2 == 0 && dvw == 64 && nvs == 1) return launch_qt<64, 0, 64, 1, 1>(a, out_f32, st);
    if (dk1 == 128 && dk2 == 0 && dvw == 128 && nvs == 1) return launch_qt<128, 0, 128, 1, 1>(a, out_f32, st);
    return hipErrorInvalidValue;
  }
#define GHA_SD_CASE(K1, K2, VW, NV) \
  if (dk1 == K1 && dk2 == K2 && dvw == VW && nvs == NV) return launch_qt<K1, K2, VW, NV>(a, out_f32, st);
  GHA_SD_CASE(64, 0, 64, 1)
  GHA_SD_CASE(64, 0, 64, 2)
  GHA_SD_CASE(64, 0, 64, 4)
  GHA_SD_CASE(128, 0, 64, 1)
  GHA_SD_CASE(128, 0, 64, 2)
  GHA_SD_CASE(128, 0, 64, 4)
  GHA_SD_CASE(128, 64, 128, 1)
  GHA_SD_CASE(128, 0, 128, 1)
  GHA_SD_CASE(64, 0, 128, 1)
  GHA_SD_CASE(64, 0, 128, 2)
  GHA_SD_CASE(64, 0, 128, 4)
  GHA_SD_CASE(128, 0, 128, 2)
  GHA_SD_CASE(128, 0, 128, 4)
#undef GHA_SD_CASE
  return hipErrorInvalidValue;
}

}  // namespace gha
