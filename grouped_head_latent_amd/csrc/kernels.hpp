// Launch descriptors shared by the C-ABI layer and the kernels.  Every size
// and stride here has already been validated on the host.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gha.h"

namespace gha {

// rows * stride * elem_bytes < limit for non-negative operands, with no
// intermediate overflow (a product that overflows is not below any limit)
inline bool span_below(int64_t rows, int64_t stride, int64_t elem_bytes, int64_t limit) {
  int64_t p = 0;
  return !__builtin_mul_overflow(rows, stride, &p) && !__builtin_mul_overflow(p, elem_bytes, &p) && p < limit;
}

struct PrefillArgs {
  const void* q; int64_t q_sb, q_sh, q_ss;
  const void* k; int64_t k_sb, k_sh, k_ss;
  const void* v; int64_t v_sb, v_sh, v_ss;
  void* o;       int64_t o_sb, o_sh, o_ss;
  float* lse;         // dense (B, lse_heads, S_q) or null
  int lse_heads;      // h_q (GQA) or n_grp (GTA)
  int S_q, S_k;
  int h_kv;           // GQA: key/value heads; GTA: groups
  int group;          // GQA: query heads per KV head; GTA: heads per group
  int heads_per_wg;   // query heads sharing one work-group (1, 2 or 4)
  int n_subgroups;    // group / heads_per_wg
  int n_qblocks;      // position blocks per (batch, head set)
  int n_blocks;       // work-groups with work
  int pair_qblocks;   // d = 128 kernel: a work-group takes q-blocks n_qblocks - 1 - i and i
  int causal;
  int B;
  float scale;
  // second key part (d = 128 kernel only): keys [k; k2] of width 128 + dk2
  // against queries [q; q2]; dk2 = 0 for none
  int dk2;
  // GTA: value heads per group, and 64-wide value sources per head (d_v / 64);
  // the kernel's value source s of group j is columns 64 (s % v_sph) .. + 63
  // of head j v_hpg + s / v_sph
  int v_hpg, v_sph;
  const void* q2; int64_t q2_sb, q2_sh, q2_ss;
  const void* k2; int64_t k2_sb, k2_sh, k2_ss;
};

struct DecodeArgs {
  const void* q; int64_t q_sb, q_sh, q_ss;
  const void* k; int64_t k_sb, k_sh, k_ss;
  const void* v; int64_t v_sb, v_sh, v_ss;
  const int32_t* seqlens;
  void* o;       int64_t o_sb, o_sh, o_ss;
  float* lse;         // dense (B, h_q, s_q) or null
  float* ws_o;        // (units, n_splits, 16, d) fp32 partial outputs
  float* ws_lse;      // (units, n_splits, 16) fp32 partial log2-sum-exp
  int B, h_q, h_kv, s_q, group;
  int L_cap;          // cache capacity: lengths are clamped to [0, L_cap]
  int rows;           // group * s_q query rows per KV head
  int n_rb;           // 16-row blocks per KV head
  int split_len;      // keys per split (multiple of 256)
  int n_splits;       // splits per unit at L_max_hint
  float scale;
};

struct LatentArgs {
  const void* q; int64_t q_sb, q_sh, q_ss;     // q_lat (B, s_q, h_q, r_kv)
  const void* qr; int64_t qr_sb, qr_sh, qr_ss; // q_rope (B, s_q, h_q, d_r)
  const void* c; int64_t c_sb, c_ss;           // c_kv (B, L_cap, r_kv)
  const void* kr; int64_t kr_sb, kr_ss;        // k_rope (B, L_cap, d_r)
  const int32_t* seqlens;
  void* o;       int64_t o_sb, o_sh, o_ss;     // o_lat (B, s_q, h_q, r_kv)
  float* lse;         // dense (B, s_q, h_q) or null
  float* ws_o;        // (n_rb, n_wg + B, rows per work-group, r_kv) partials
  float* ws_lse;      // (n_rb, n_wg + B, rows per work-group)
  int32_t* ws_tiles;  // (B + 1) prefix sums of the split positions per sequence
  int B, h_q, s_q, L_cap;
  int n_rb;           // row blocks (of latent_rows_per_wg()) over s_q * h_q rows
  int n_wg;           // work-groups per row block, each takes 1/n_wg of all tiles
  float scale;
};

// Streaming split-KV decode where a group's key is a per-group part (width
// dk1) optionally followed by a part shared by all groups (width dk2), and
// its value is the concatenation of nvs value heads (width dvw each).
struct StreamDecodeArgs {
  const void* q;  int64_t q_sb, q_sh, q_ss;    // query part 1: (B, G * qpg, s_q, dk1)
  const void* q2; int64_t q2_sb, q2_sh, q2_ss; // query part 2: (B, G * qpg, s_q, dk2), if dk2 > 0
  const void* k;  int64_t k_sb, k_sh, k_ss;    // per-group key cache (B, G, L_cap, dk1)
  const void* k2; int64_t k2_sb, k2_ss;        // shared key cache (B, L_cap, dk2), if dk2 > 0
  const void* v;  int64_t v_sb, v_sh, v_ss;    // value heads (B, G * v_hpg, L_cap, v_sph * dvw)
  // value source s (of nvs, each dvw wide) of group j is columns
  // dvw (s % v_sph) .. + dvw - 1 of value head j v_hpg + s / v_sph; output
  // row (hh, t) of group j writes that source to head (j qpg + hh) v_hpg +
  // s / v_sph at the same columns
  int v_hpg, v_sph;
  const int32_t* seqlens;
  void* o;        int64_t o_sb, o_sh, o_ss;    // (B, G * qpg * v_hpg, s_q, v_sph * dvw)
  float* lse;         // dense (B, G * qpg, s_q) or null
  float* ws_o;        // (n_wg + B * G slots, rows padded to 16 or 32, nvs * dvw) partials
  float* ws_lse;      // (n_wg + B * G slots, padded rows)
  int32_t* ws_pref;   // (B + 1) prefix sums over sequences of (G / team) * (128-key chunks)
  int B, n_groups, qpg, s_q, rows;  // rows = qpg * s_q query rows per group (<= 32)
  int L_cap, n_wg;    // n_wg work-groups (teams of `team`) share all chunks equally
  int team;           // 1, or n_groups when the groups share a key part
  float scale;
  // sliding window: with window > 0 query t of sequence b sees only keys
  // L_b - s_q + t - window + 1 .. L_b - s_q + t
  int window;
  // paged cache (one key part, one value source): block_table != null means
  // k and v are pages, indexed (page, group, token in page) by the k_sb / v_sb,
  // k_sh / v_sh, k_ss / v_ss strides; key u of sequence b sits in page
  // block_table[b * bt_stride + u / page_size] at token u % page_size
  const int32_t* block_table;
  int bt_stride, page_size;
  // 8-bit caches: k and v hold E4M3 codes; the key scale is folded into
  // `scale`, the value scale multiplies the outputs
  float v_scale;
};

// The per-group absorption products of the latent decode (d_h = 128,
// r_kv = 512): rows are (batch, new token, head) with head in group
// head / (h_q / g).
struct AbsorbArgs {
  const void* in; int64_t in_sb, in_sh, in_ss;  // q^C (B, s_q, h_q, d_h) by (batch, head, token) strides
  const void* w;                                // W^UK or W^UV, (g * d_h, r_kv) row-major bf16
  void* wt;                                     // workspace for W^UK transposed, (g, r_kv, d_h) bf16
  const void* lat;                              // o_lat, dense bf16 (B, s_q, h_q, r_kv)
  void* out; int64_t o_sb, o_sh, o_ss;          // q~ dense bf16 (B, s_q, h_q, r_kv), or O by strides
  int B, s_q, h_q, g;
};
hipError_t launch_absorb_query(const AbsorbArgs& a, hipStream_t st);
hipError_t launch_absorb_output(const AbsorbArgs& a, bool out_f32, hipStream_t st);

hipError_t launch_prefill_bf16(const PrefillArgs& a, int d, bool out_f32, hipStream_t st);
bool prefill_d128_supported(const PrefillArgs& a);
hipError_t launch_prefill_d128(const PrefillArgs& a, bool out_f32, hipStream_t st);
hipError_t launch_prefill_f32(const PrefillArgs& a, int d, hipStream_t st);
int prefill_rows_per_wave();
int prefill_bf16_waves(const PrefillArgs& a, int d);  // waves per work-group of the kernel chosen for a
// compute units of the current device, 0 if it cannot be queried
int device_cus();
// sets the detail string gha_last_error() returns (defined in abi.cpp)
void set_last_error(const char* msg);
// debug checks: tests lo <= seqlens[b] <= hi for b < B on the device and
// writes out[0] = the first failing b (-1 if none) and out[1] = its length
hipError_t launch_check_lengths(const int32_t* seqlens, int B, int lo, int hi, int32_t* out, hipStream_t st);
// the workspace gqa_decode needs for these cache views (defined in abi.cpp)
size_t gqa_decode_path_workspace(const gha_tensor* k_cache, const gha_tensor* v_cache, int B, int h_q, int h_kv,
                                 int s_q, int L_cap, int L_max_hint, int d);

hipError_t launch_gta(const PrefillArgs& a, int d_qk, int sources, bool out_f32, hipStream_t st);
// the one-stream GTA prefill kernel: same arguments, also 128 positions per work-group
hipError_t launch_gta_fused(const PrefillArgs& a, int d_qk, int sources, bool out_f32, hipStream_t st);
int gta_positions_per_wg();
// K/V spans and row pitches the GTA kernel's 32-bit buffer addressing covers
bool gta_layout_supported(const PrefillArgs& a, int d_qk, int d_v);

hipError_t launch_gqa_decode(const DecodeArgs& a, int d, bool out_f32, hipStream_t st);
hipError_t launch_stream_decode(const StreamDecodeArgs& a, int dk1, int dk2, int dvw, int nvs, bool out_f32,
                                hipStream_t st, bool fp8 = false);
int stream_decode_chunk();  // keys per scheduling chunk of the streaming decode
hipError_t launch_latent_decode(const LatentArgs& a, bool out_f32, hipStream_t st);
int latent_rows_per_wg();    // query rows per work-group of the split kernel
int latent_tile_tokens();    // tokens per tile
int latent_segment_start_tiles();  // placeholder positions per sequence in the split (at most)
// work-groups per row block for n_rb row blocks and at most max_tiles tiles
int latent_plan_wgs(int n_rb, int64_t max_tiles);

}  // namespace gha
