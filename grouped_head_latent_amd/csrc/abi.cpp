// C ABI of the grouped-head attention library: argument validation, split
// planning and dispatch.  Every check runs on the host before anything is
// launched; see include/gha.h for the contract of each entry point.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/gha.h"
#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";

gha_status fail(gha_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

int elem_size(gha_dtype t) { return t == GHA_F32 ? 4 : t == GHA_FP8_E4M3 ? 1 : 2; }

// Upper limits on sizes.  Within them every size, grid and workspace formula
// in this file stays inside 64-bit arithmetic and every row count (heads per
// group times new tokens) inside 32-bit; larger arguments are refused
// (GHA_ERR_SHAPE, and 0 from the workspace queries).
constexpr int kMaxBatch = 1 << 20;
constexpr int kMaxHeads = 1 << 12;
constexpr int kMaxNewTokens = 1 << 16;
constexpr int kMaxLen = 1 << 30;
bool within_limits(int B, int heads_a, int heads_b, int s_q, int len_a, int len_b) {
  return B <= kMaxBatch && heads_a <= kMaxHeads && heads_b <= kMaxHeads && s_q <= kMaxNewTokens &&
         len_a <= kMaxLen && len_b <= kMaxLen;
}
gha_status limits_fail() {
  return fail(GHA_ERR_SHAPE, "a size exceeds the library's limits (B <= %d, heads <= %d, s_q <= %d, lengths <= %d)",
              kMaxBatch, kMaxHeads, kMaxNewTokens, kMaxLen);
}

// A view must be present, non-negative and keep every row 16-byte aligned.
// Strides above 2^48 elements cannot address real memory and are refused,
// which also keeps the offset arithmetic of the launches within 64 bits.
constexpr int64_t kMaxStride = (int64_t)1 << 48;
gha_status check_view(const char* name, const gha_tensor* t, gha_dtype dt, bool use_sb,
                      bool use_sh, bool use_ss) {
  if (t == nullptr || t->ptr == nullptr) return fail(GHA_ERR_NULL, "%s: null tensor or pointer", name);
  if (t->sb < 0 || t->sh < 0 || t->ss < 0) return fail(GHA_ERR_STRIDE, "%s: negative stride", name);
  if (t->sb > kMaxStride || t->sh > kMaxStride || t->ss > kMaxStride)
    return fail(GHA_ERR_STRIDE, "%s: a stride exceeds 2^48 elements", name);
  const int64_t es = elem_size(dt);
  if ((reinterpret_cast<uintptr_t>(t->ptr) & 15u) != 0)
    return fail(GHA_ERR_ALIGN, "%s: pointer not 16-byte aligned", name);
  if ((use_sb && (t->sb * es) % 16) || (use_sh && (t->sh * es) % 16) || (use_ss && (t->ss * es) % 16))
    return fail(GHA_ERR_ALIGN, "%s: a stride is not a multiple of 16 bytes", name);
  return GHA_OK;
}

gha_status check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GHA_ERR_HIP, "no HIP device: %s", hipGetErrorString(e));
  return GHA_OK;
}

// Debug checks: -1 until first asked for, then 0 or 1 (gha_set_debug_checks,
// else the environment variable GHA_DEBUG_CHECKS).
std::atomic<int> g_debug_checks{-1};

bool debug_checks_on() {
  int v = g_debug_checks.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* env = std::getenv("GHA_DEBUG_CHECKS");
    int expected = -1;
    g_debug_checks.compare_exchange_strong(expected, (env != nullptr && std::atoi(env) != 0) ? 1 : 0);
    v = g_debug_checks.load();
  }
  return v != 0;
}

// With debug checks on: has the device test s_q <= seqlens_k[b] <= L_cap for
// every b, answering in the first 8 bytes of `scratch` (the call's
// workspace, 16-byte aligned and larger than that), waits for the answer and
// refuses the call if a length is out of range.  Nothing else has been
// launched by then.
gha_status check_lengths_on_device(const int32_t* seqlens, int B, int s_q, int L_cap, void* scratch,
                                   void* stream, const char* what) {
  if (!debug_checks_on()) return GHA_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  int32_t* answer = reinterpret_cast<int32_t*>(scratch);
  int32_t h[2] = {-1, 0};
  hipError_t e = gha::launch_check_lengths(seqlens, B, s_q, L_cap, answer, st);
  if (e == hipSuccess) e = hipMemcpyAsync(h, answer, sizeof(h), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(GHA_ERR_HIP, "%s: debug length check failed: %s", what, hipGetErrorString(e));
  if (h[0] >= 0)
    return fail(GHA_ERR_PRECONDITION, "%s: seqlens_k[%d] = %d is outside [s_q, L_cap] = [%d, %d]", what, h[0],
                h[1], s_q, L_cap);
  return GHA_OK;
}

gha_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(GHA_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  g_err[0] = 0;
  return GHA_OK;
}

// Split plan of the GQA decode: aim for about 8192 work-groups so that short
// and long sequences spread evenly over 256 CUs; splits are whole multiples
// of 256 keys (four waves x 64 keys).
void gqa_decode_plan(int B, int h_kv, int n_rb, int L_max, int* split_len, int* n_splits) {
  const int64_t units = (int64_t)B * h_kv * n_rb;
  const int64_t want = units >= 8192 ? 1 : (8192 + units - 1) / units;
  int64_t sl = (L_max + want - 1) / want;
  sl = (sl + 255) / 256 * 256;
  if (sl < 256) sl = 256;
  *split_len = (int)sl;
  *n_splits = (int)((L_max + sl - 1) / sl);
}

int gqa_row_blocks(int h_q, int h_kv, int s_q) { return ((h_q / h_kv) * s_q + 15) / 16; }

// Plan of the streaming decode: teams of Z work-groups, about `target`
// work-groups in all (a single round: GHA_SD_WGS = one per CU for bf16
// caches, GHA_SD_WGS_8BIT = two per CU for 8-bit caches, whose kernel sizes
// its LDS for two), share all 128-key chunks of all units equally; fewer
// teams when there are fewer chunks than that.
// Z = 1 (units are (sequence, group)) unless the groups share a key part,
// then Z = G (units are sequences, member j serves group j).  Partials: one
// slot per team and per unit for each member, 16 or 32 padded rows each.
#ifndef GHA_SD_WGS
#define GHA_SD_WGS 256
#endif
#ifndef GHA_SD_WGS_8BIT
#define GHA_SD_WGS_8BIT 512
#endif
int stream_decode_wgs(int B, int G, int Z, int L_max, int target = GHA_SD_WGS) {
  const int64_t chunks = (int64_t)B * (G / Z) * ((L_max + gha::stream_decode_chunk() - 1) / gha::stream_decode_chunk());
  const int64_t teams = std::max<int64_t>(1, std::min<int64_t>(target / Z, chunks));
  return (int)(teams * Z);
}
size_t stream_decode_ws(int B, int G, int Z, int rows, int L_max, int dv, int target = GHA_SD_WGS) {
  const size_t rp = rows <= 16 ? 16 : 32;
  const size_t n = ((size_t)stream_decode_wgs(B, G, Z, L_max, target) + (size_t)B * G) * rp;
  return n * (size_t)dv * 4 + n * 4 + (size_t)(B + 1) * 4;
}
// workspace carve-up: partial outputs, their log2-sum-exp, the chunk prefix sums
void stream_decode_carve(gha::StreamDecodeArgs& a, void* workspace, int dv) {
  const size_t n = ((size_t)a.n_wg + (size_t)a.B * a.n_groups) * (a.rows <= 16 ? 16 : 32);
  a.ws_o = reinterpret_cast<float*>(workspace);
  a.ws_lse = a.ws_o + n * (size_t)dv;
  a.ws_pref = reinterpret_cast<int32_t*>(a.ws_lse + n);
}
// one (batch, head) sequence of a cache read through 32-bit buffer offsets
bool span_ok(int L_cap, int64_t ss) { return gha::span_below((int64_t)L_cap + 64, ss, 2, (int64_t)1 << 31); }
int latent_row_blocks(int h_q, int s_q) {
  const int r = gha::latent_rows_per_wg();
  return (h_q * s_q + r - 1) / r;
}

// GTA value sources: the kernels apply a group's scores to value sources of
// `dvw` columns, a head of d_v columns being d_v / dvw of them.  A launch
// takes `nvs` sources (the largest of 4, 2, 1 that divides the group's
// `nsrc`, within `max_cols` columns); `launches` launches cover the group.
struct GtaSources {
  int dvw, sph, nsrc, nvs, launches;
};
GtaSources gta_sources(int per, int d_v, int dvw, int max_cols) {
  GtaSources p{};
  p.dvw = dvw;
  p.sph = d_v / dvw;
  p.nsrc = per * p.sph;
  p.nvs = 1;
  for (int n : {4, 2})
    if (n * dvw <= max_cols && p.nsrc % n == 0) {
      p.nvs = n;
      break;
    }
  p.launches = p.nsrc / p.nvs;
  return p;
}
// prefill: 64-column sources, up to four per work-group
GtaSources gta_prefill_sources(int per, int d_v) { return gta_sources(per, d_v, 64, 256); }
// decode: 64-column sources for d_v = 64, else 128; a 16-row q-tile holds up
// to 512 accumulated columns, a 32-row one up to 256
GtaSources gta_decode_sources(int per, int d_v, int s_q) {
  return gta_sources(per, d_v, d_v == 64 ? 64 : 128, s_q <= 16 ? 512 : 256);
}
bool gta_dv_ok(int d_v) { return d_v == 64 || d_v == 128 || d_v == 256; }

}  // namespace

namespace gha {
// the thread-local detail string of gha_last_error(), for entry points
// defined in other source files
void set_last_error(const char* msg) { snprintf(g_err, sizeof(g_err), "%s", msg); }
}  // namespace gha

extern "C" {

const char* gha_status_string(gha_status s) {
  switch (s) {
    case GHA_OK: return "GHA_OK";
    case GHA_ERR_NULL: return "GHA_ERR_NULL";
    case GHA_ERR_SHAPE: return "GHA_ERR_SHAPE";
    case GHA_ERR_GROUPING: return "GHA_ERR_GROUPING";
    case GHA_ERR_STRIDE: return "GHA_ERR_STRIDE";
    case GHA_ERR_ALIGN: return "GHA_ERR_ALIGN";
    case GHA_ERR_DTYPE: return "GHA_ERR_DTYPE";
    case GHA_ERR_HEAD_DIM: return "GHA_ERR_HEAD_DIM";
    case GHA_ERR_WORKSPACE: return "GHA_ERR_WORKSPACE";
    case GHA_ERR_HIP: return "GHA_ERR_HIP";
    case GHA_ERR_PRECONDITION: return "GHA_ERR_PRECONDITION";
  }
  return "GHA_ERR_UNKNOWN";
}

const char* gha_last_error(void) { return g_err; }

void gha_set_debug_checks(int on) { g_debug_checks.store(on != 0 ? 1 : 0); }

int gha_debug_checks(void) { return debug_checks_on() ? 1 : 0; }

int gha_version(void) { return 100; }  // 0.1.0

gha_status gqa_prefill(const gha_tensor* q, const gha_tensor* k, const gha_tensor* v,
                       const gha_tensor* o, float* lse, int B, int h_q, int h_kv, int S_q,
                       int S_k, int d, gha_dtype in_dtype, gha_dtype out_dtype, float scale,
                       int causal, void* stream) {
  if (B < 1 || h_q < 1 || h_kv < 1 || S_q < 1 || S_k < 1)
    return fail(GHA_ERR_SHAPE, "sizes must be positive (B=%d h_q=%d h_kv=%d S_q=%d S_k=%d)", B, h_q, h_kv, S_q, S_k);
  if (!within_limits(B, h_q, h_kv, 1, S_q, S_k)) return limits_fail();
  if (h_q % h_kv) return fail(GHA_ERR_GROUPING, "h_q=%d is not a multiple of h_kv=%d", h_q, h_kv);
  if (causal && S_q > S_k) return fail(GHA_ERR_SHAPE, "causal needs S_q <= S_k (got %d > %d)", S_q, S_k);
  if (d != 64 && d != 128) return fail(GHA_ERR_HEAD_DIM, "head dim %d not in {64, 128}", d);
  const bool f32in = in_dtype == GHA_F32;
  if (!((in_dtype == GHA_BF16 && (out_dtype == GHA_BF16 || out_dtype == GHA_F32)) ||
        (f32in && out_dtype == GHA_F32)))
    return fail(GHA_ERR_DTYPE, "unsupported in/out dtypes (%d, %d)", (int)in_dtype, (int)out_dtype);
  gha_status s;
  if ((s = check_view("q", q, in_dtype, B > 1, h_q > 1, S_q > 1)) != GHA_OK) return s;
  if ((s = check_view("k", k, in_dtype, B > 1, h_kv > 1, S_k > 1)) != GHA_OK) return s;
  if ((s = check_view("v", v, in_dtype, B > 1, h_kv > 1, S_k > 1)) != GHA_OK) return s;
  if ((s = check_view("o", o, out_dtype, B > 1, h_q > 1, S_q > 1)) != GHA_OK) return s;
  if ((s = check_device()) != GHA_OK) return s;

  gha::PrefillArgs a{};
  a.q = q->ptr; a.q_sb = q->sb; a.q_sh = q->sh; a.q_ss = q->ss;
  a.k = k->ptr; a.k_sb = k->sb; a.k_sh = k->sh; a.k_ss = k->ss;
  a.v = v->ptr; a.v_sb = v->sb; a.v_sh = v->sh; a.v_ss = v->ss;
  a.o = o->ptr; a.o_sb = o->sb; a.o_sh = o->sh; a.o_ss = o->ss;
  a.lse = lse; a.lse_heads = h_q;
  a.S_q = S_q; a.S_k = S_k; a.h_kv = h_kv; a.group = h_q / h_kv;
  a.causal = causal ? 1 : 0;
  a.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)d);
  a.B = B;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (f32in) {
    a.n_blocks = B;
    return launched(gha::launch_prefill_f32(a, d, st), "gqa_prefill(f32)");
  }
  const int G = a.group;
  a.heads_per_wg = (G % 4 == 0) ? 4 : (G % 2 == 0 ? 2 : 1);
  a.n_subgroups = G / a.heads_per_wg;
  const int pos_per_wg = (gha::prefill_bf16_waves(a, d) / a.heads_per_wg) * gha::prefill_rows_per_wave();
  a.n_qblocks = (S_q + pos_per_wg - 1) / pos_per_wg;
  const int64_t nb = (int64_t)B * h_kv * a.n_subgroups * a.n_qblocks;
  if (nb > (1LL << 30)) return fail(GHA_ERR_SHAPE, "problem too large for one launch");
  a.n_blocks = (int)nb;
  return launched(gha::launch_prefill_bf16(a, d, out_dtype == GHA_F32, st), "gqa_prefill");
}

gha_status gqla_gqa_prefill(const gha_tensor* q_c, const gha_tensor* q_r, const gha_tensor* k_c,
                            const gha_tensor* k_r, const gha_tensor* v, const gha_tensor* o, float* lse,
                            int B, int h_q, int g, int S_q, int S_k, int d_h, int d_r,
                            gha_dtype in_dtype, gha_dtype out_dtype, float scale, int causal,
                            void* stream) {
  if (B < 1 || h_q < 1 || g < 1 || S_q < 1 || S_k < 1)
    return fail(GHA_ERR_SHAPE, "sizes must be positive (B=%d h_q=%d g=%d S_q=%d S_k=%d)", B, h_q, g, S_q, S_k);
  if (!within_limits(B, h_q, g, 1, S_q, S_k)) return limits_fail();
  if (h_q % g) return fail(GHA_ERR_GROUPING, "h_q=%d is not a multiple of g=%d", h_q, g);
  if (causal && S_q > S_k) return fail(GHA_ERR_SHAPE, "causal needs S_q <= S_k (got %d > %d)", S_q, S_k);
  if (d_h != 128 || d_r != 64) return fail(GHA_ERR_HEAD_DIM, "need d_h == 128 and d_r == 64 (got %d, %d)", d_h, d_r);
  if (!(scale > 0.f)) return fail(GHA_ERR_SHAPE, "scale must be given (> 0): 1/sqrt(d_h + d_r) for the expanded key");
  if (in_dtype != GHA_BF16 || (out_dtype != GHA_BF16 && out_dtype != GHA_F32))
    return fail(GHA_ERR_DTYPE, "takes bf16 inputs and bf16 or f32 outputs");
  gha_status s;
  if ((s = check_view("q_c", q_c, in_dtype, B > 1, h_q > 1, S_q > 1)) != GHA_OK) return s;
  if ((s = check_view("q_r", q_r, in_dtype, B > 1, h_q > 1, S_q > 1)) != GHA_OK) return s;
  if ((s = check_view("k_c", k_c, in_dtype, B > 1, g > 1, S_k > 1)) != GHA_OK) return s;
  if ((s = check_view("k_r", k_r, in_dtype, B > 1, false, S_k > 1)) != GHA_OK) return s;
  if ((s = check_view("v", v, in_dtype, B > 1, g > 1, S_k > 1)) != GHA_OK) return s;
  if ((s = check_view("o", o, out_dtype, B > 1, h_q > 1, S_q > 1)) != GHA_OK) return s;

  gha::PrefillArgs a{};
  a.q = q_c->ptr; a.q_sb = q_c->sb; a.q_sh = q_c->sh; a.q_ss = q_c->ss;
  a.k = k_c->ptr; a.k_sb = k_c->sb; a.k_sh = k_c->sh; a.k_ss = k_c->ss;
  a.v = v->ptr; a.v_sb = v->sb; a.v_sh = v->sh; a.v_ss = v->ss;
  a.o = o->ptr; a.o_sb = o->sb; a.o_sh = o->sh; a.o_ss = o->ss;
  a.dk2 = d_r;
  a.q2 = q_r->ptr; a.q2_sb = q_r->sb; a.q2_sh = q_r->sh; a.q2_ss = q_r->ss;
  a.k2 = k_r->ptr; a.k2_sb = k_r->sb; a.k2_sh = 0; a.k2_ss = k_r->ss;  // one RoPE key for every group
  a.lse = lse; a.lse_heads = h_q;
  a.S_q = S_q; a.S_k = S_k; a.h_kv = g; a.group = h_q / g;
  a.causal = causal ? 1 : 0;
  a.scale = scale;
  a.B = B;
  if (!gha::prefill_d128_supported(a))
    return fail(GHA_ERR_STRIDE, "rows overlap or one sequence spans 2 GiB or more");
  if ((s = check_device()) != GHA_OK) return s;
  const int G = a.group;
  a.heads_per_wg = (G % 4 == 0) ? 4 : (G % 2 == 0 ? 2 : 1);
  a.n_subgroups = G / a.heads_per_wg;
  const int pos_per_wg = (4 / a.heads_per_wg) * gha::prefill_rows_per_wave();
  a.n_qblocks = (S_q + pos_per_wg - 1) / pos_per_wg;
  const int64_t nb = (int64_t)B * g * a.n_subgroups * a.n_qblocks;
  if (nb > (1LL << 30)) return fail(GHA_ERR_SHAPE, "problem too large for one launch");
  a.n_blocks = (int)nb;
  return launched(gha::launch_prefill_d128(a, out_dtype == GHA_F32, reinterpret_cast<hipStream_t>(stream)),
                  "gqla_gqa_prefill");
}

}  // extern "C"

namespace {
// gqa_decode's choice of kernel: up to 32 query rows per group (heads per
// group times new tokens) and caches the 32-bit buffer addressing covers go
// to the streaming kernel (one pass over each group's cache with every row of
// the group), anything else to the register-fed kernel with 16-row blocks
bool gqa_decode_streams(const gha_tensor* k_cache, const gha_tensor* v_cache, int h_q, int h_kv, int s_q,
                        int L_cap, int d) {
  return (h_q / h_kv) * s_q <= 32 && k_cache->ss >= d && v_cache->ss >= d && span_ok(L_cap, k_cache->ss) &&
         span_ok(L_cap, v_cache->ss);
}
// workspace of the register-fed kernel's split plan
size_t gqa_decode_register_ws(int B, int h_q, int h_kv, int s_q, int L_max_hint, int d) {
  const int n_rb = gqa_row_blocks(h_q, h_kv, s_q);
  int sl, ns;
  gqa_decode_plan(B, h_kv, n_rb, L_max_hint, &sl, &ns);
  const size_t rows = (size_t)B * h_kv * n_rb * ns * 16;
  return rows * (size_t)d * 4 + rows * 4;
}
bool gqa_decode_sizes_ok(int B, int h_q, int h_kv, int s_q, int L_max_hint, int d) {
  return B >= 1 && h_q >= 1 && h_kv >= 1 && s_q >= 1 && L_max_hint >= 1 && (d == 64 || d == 128) &&
         h_q % h_kv == 0 && within_limits(B, h_q, h_kv, s_q, L_max_hint, 1);
}
}  // namespace

namespace gha {
// the workspace gqa_decode needs for these cache views (the kernel it takes
// depends on their strides); 0 for arguments it rejects
size_t gqa_decode_path_workspace(const gha_tensor* k_cache, const gha_tensor* v_cache, int B, int h_q, int h_kv,
                                 int s_q, int L_cap, int L_max_hint, int d) {
  if (!gqa_decode_sizes_ok(B, h_q, h_kv, s_q, L_max_hint, d) || k_cache == nullptr || v_cache == nullptr) return 0;
  if (gqa_decode_streams(k_cache, v_cache, h_q, h_kv, s_q, L_cap, d))
    return stream_decode_ws(B, h_kv, 1, (h_q / h_kv) * s_q, L_max_hint, d);
  return gqa_decode_register_ws(B, h_q, h_kv, s_q, L_max_hint, d);
}
}  // namespace gha

extern "C" {

size_t gqa_decode_workspace_bytes(int B, int h_q, int h_kv, int s_q, int L_max_hint, int d) {
  if (!gqa_decode_sizes_ok(B, h_q, h_kv, s_q, L_max_hint, d)) return 0;
  // enough for either kernel: which one runs depends on the cache strides
  size_t need = gqa_decode_register_ws(B, h_q, h_kv, s_q, L_max_hint, d);
  if ((h_q / h_kv) * s_q <= 32) need = std::max(need, stream_decode_ws(B, h_kv, 1, (h_q / h_kv) * s_q, L_max_hint, d));
  return need;
}

gha_status gqa_decode(const gha_tensor* q, const gha_tensor* k_cache, const gha_tensor* v_cache,
                      const int32_t* seqlens_k, const gha_tensor* o, float* lse, int B, int h_q,
                      int h_kv, int s_q, int L_cap, int L_max_hint, int d, gha_dtype in_dtype,
                      gha_dtype out_dtype, float scale, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (B < 1 || h_q < 1 || h_kv < 1 || s_q < 1 || L_cap < 1 || L_max_hint < 1)
    return fail(GHA_ERR_SHAPE, "sizes must be positive");
  if (!within_limits(B, h_q, h_kv, s_q, L_cap, L_max_hint)) return limits_fail();
  if (h_q % h_kv) return fail(GHA_ERR_GROUPING, "h_q=%d is not a multiple of h_kv=%d", h_q, h_kv);
  if (L_max_hint > L_cap || s_q > L_max_hint)
    return fail(GHA_ERR_SHAPE, "need s_q <= L_max_hint <= L_cap (s_q=%d L_max_hint=%d L_cap=%d)", s_q, L_max_hint, L_cap);
  if (d != 64 && d != 128) return fail(GHA_ERR_HEAD_DIM, "head dim %d not in {64, 128}", d);
  if (in_dtype != GHA_BF16 || (out_dtype != GHA_BF16 && out_dtype != GHA_F32))
    return fail(GHA_ERR_DTYPE, "decode takes bf16 inputs and bf16 or f32 outputs");
  if (seqlens_k == nullptr) return fail(GHA_ERR_NULL, "seqlens_k is null");
  gha_status s;
  if ((s = check_view("q", q, in_dtype, B > 1, h_q > 1, s_q > 1)) != GHA_OK) return s;
  if ((s = check_view("k_cache", k_cache, in_dtype, B > 1, h_kv > 1, true)) != GHA_OK) return s;
  if ((s = check_view("v_cache", v_cache, in_dtype, B > 1, h_kv > 1, true)) != GHA_OK) return s;
  if ((s = check_view("o", o, out_dtype, B > 1, h_q > 1, s_q > 1)) != GHA_OK) return s;
  // the workspace of the kernel these views take (at most the size that
  // gqa_decode_workspace_bytes reports)
  const size_t need = gha::gqa_decode_path_workspace(k_cache, v_cache, B, h_q, h_kv, s_q, L_cap, L_max_hint, d);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(GHA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 15u) != 0)
    return fail(GHA_ERR_ALIGN, "workspace not 16-byte aligned");
  if ((s = check_device()) != GHA_OK) return s;
  if ((s = check_lengths_on_device(seqlens_k, B, s_q, L_cap, workspace, stream, "gqa_decode")) != GHA_OK) return s;

  const int rows = (h_q / h_kv) * s_q;
  if (gqa_decode_streams(k_cache, v_cache, h_q, h_kv, s_q, L_cap, d)) {
    gha::StreamDecodeArgs sa{};
    sa.q = q->ptr; sa.q_sb = q->sb; sa.q_sh = q->sh; sa.q_ss = q->ss;
    sa.k = k_cache->ptr; sa.k_sb = k_cache->sb; sa.k_sh = k_cache->sh; sa.k_ss = k_cache->ss;
    sa.v = v_cache->ptr; sa.v_sb = v_cache->sb; sa.v_sh = v_cache->sh; sa.v_ss = v_cache->ss;
    sa.seqlens = seqlens_k;
    sa.o = o->ptr; sa.o_sb = o->sb; sa.o_sh = o->sh; sa.o_ss = o->ss;
    sa.lse = lse;
    sa.B = B; sa.n_groups = h_kv; sa.qpg = h_q / h_kv; sa.s_q = s_q; sa.rows = rows; sa.L_cap = L_cap;
    sa.v_hpg = 1; sa.v_sph = 1;
    sa.team = 1;
    sa.n_wg = stream_decode_wgs(B, h_kv, 1, L_max_hint);
    stream_decode_carve(sa, workspace, d);
    sa.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)d);
    if ((int64_t)B * ((L_cap + 127) / 128) >= (1LL << 31) || (int64_t)h_kv * 2 > (1LL << 30))
      return fail(GHA_ERR_SHAPE, "problem too large for one launch");
    return launched(gha::launch_stream_decode(sa, d, 0, d, 1, out_dtype == GHA_F32,
                                              reinterpret_cast<hipStream_t>(stream)),
                    "gqa_decode");
  }

  gha::DecodeArgs a{};
  a.q = q->ptr; a.q_sb = q->sb; a.q_sh = q->sh; a.q_ss = q->ss;
  a.k = k_cache->ptr; a.k_sb = k_cache->sb; a.k_sh = k_cache->sh; a.k_ss = k_cache->ss;
  a.v = v_cache->ptr; a.v_sb = v_cache->sb; a.v_sh = v_cache->sh; a.v_ss = v_cache->ss;
  a.seqlens = seqlens_k;
  a.o = o->ptr; a.o_sb = o->sb; a.o_sh = o->sh; a.o_ss = o->ss;
  a.lse = lse;
  a.B = B; a.h_q = h_q; a.h_kv = h_kv; a.s_q = s_q; a.group = h_q / h_kv; a.L_cap = L_cap;
  a.rows = a.group * s_q;
  a.n_rb = gqa_row_blocks(h_q, h_kv, s_q);
  gqa_decode_plan(B, h_kv, a.n_rb, L_max_hint, &a.split_len, &a.n_splits);
  const size_t n_part = (size_t)B * h_kv * a.n_rb * a.n_splits * 16;
  a.ws_o = reinterpret_cast<float*>(workspace);
  a.ws_lse = a.ws_o + n_part * d;
  a.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)d);
  if ((int64_t)B * h_kv * a.n_rb * a.n_splits > (1LL << 30))
    return fail(GHA_ERR_SHAPE, "problem too large for one launch");
  return launched(gha::launch_gqa_decode(a, d, out_dtype == GHA_F32, reinterpret_cast<hipStream_t>(stream)),
                  "gqa_decode");
}

// Keys a windowed sequence can touch, for the streaming plan: the window,
// the new tokens and up to two chunks of alignment.
static int window_keys(int L_max_hint, int s_q, int window) {
  if (window <= 0) return L_max_hint;
  const int64_t k = (int64_t)window + s_q + 2 * gha::stream_decode_chunk();
  return (int)std::min<int64_t>(L_max_hint, k);
}

size_t gqa_decode_paged_workspace_bytes(int B, int h_q, int h_kv, int s_q, int L_max_hint, int window, int d) {
  if (B < 1 || h_q < 1 || h_kv < 1 || s_q < 1 || L_max_hint < 1 || window < 0 || h_q % h_kv || (d != 64 && d != 128))
    return 0;
  if (!within_limits(B, h_q, h_kv, s_q, L_max_hint, window)) return 0;
  if ((h_q / h_kv) * s_q > 32) return 0;
  // enough for either cache type (the 8-bit plan has more work-groups)
  return stream_decode_ws(B, h_kv, 1, (h_q / h_kv) * s_q, window_keys(L_max_hint, s_q, window), d, GHA_SD_WGS_8BIT);
}

}  // extern "C"

namespace {
// GQA decode on the streaming kernel over a contiguous or paged cache of
// bf16 or E4M3 elements, with an optional sliding window
gha_status stream_gqa_decode(const gha_tensor* q, const gha_tensor* k_cache, const gha_tensor* v_cache,
                             const int32_t* block_table, int bt_stride, int page_size,
                             const int32_t* seqlens_k, const gha_tensor* o, float* lse, int B, int h_q,
                             int h_kv, int s_q, int L_cap, int L_max_hint, int window, int d,
                             gha_dtype in_dtype, gha_dtype cache_dtype, gha_dtype out_dtype, float scale,
                             float k_scale, float v_scale, void* workspace, size_t workspace_bytes,
                             void* stream, const char* name) {
  if (B < 1 || h_q < 1 || h_kv < 1 || s_q < 1 || L_cap < 1 || L_max_hint < 1)
    return fail(GHA_ERR_SHAPE, "sizes must be positive");
  if (!within_limits(B, h_q, h_kv, s_q, L_cap, L_max_hint)) return limits_fail();
  if (h_q % h_kv) return fail(GHA_ERR_GROUPING, "h_q=%d is not a multiple of h_kv=%d", h_q, h_kv);
  if (L_max_hint > L_cap || s_q > L_max_hint)
    return fail(GHA_ERR_SHAPE, "need s_q <= L_max_hint <= L_cap (s_q=%d L_max_hint=%d L_cap=%d)", s_q, L_max_hint, L_cap);
  if (window < 0) return fail(GHA_ERR_SHAPE, "window must be >= 0 (0: no window), got %d", window);
  if ((h_q / h_kv) * s_q > 32)
    return fail(GHA_ERR_SHAPE, "at most 32 query rows per KV head ((h_q / h_kv) * s_q = %d)", (h_q / h_kv) * s_q);
  if (d != 64 && d != 128) return fail(GHA_ERR_HEAD_DIM, "head dim %d not in {64, 128}", d);
  if (in_dtype != GHA_BF16 || (out_dtype != GHA_BF16 && out_dtype != GHA_F32))
    return fail(GHA_ERR_DTYPE, "decode takes bf16 inputs and bf16 or f32 outputs");
  if (seqlens_k == nullptr) return fail(GHA_ERR_NULL, "seqlens_k is null");
  const bool paged = block_table != nullptr;
  if (paged) {
    if (page_size < 32 || page_size % 32 != 0)
      return fail(GHA_ERR_SHAPE, "page_size must be a positive multiple of 32 (got %d)", page_size);
    if (bt_stride < 1 || (int64_t)bt_stride * page_size < L_cap)
      return fail(GHA_ERR_SHAPE, "block table rows of %d pages of %d tokens do not cover L_cap=%d", bt_stride, page_size, L_cap);
  }
  gha_status s;
  if ((s = check_view("q", q, in_dtype, B > 1, h_q > 1, s_q > 1)) != GHA_OK) return s;
  if ((s = check_view("k_cache", k_cache, cache_dtype, true, h_kv > 1, true)) != GHA_OK) return s;
  if ((s = check_view("v_cache", v_cache, cache_dtype, true, h_kv > 1, true)) != GHA_OK) return s;
  if ((s = check_view("o", o, out_dtype, B > 1, h_q > 1, s_q > 1)) != GHA_OK) return s;
  if (k_cache->ss < d || v_cache->ss < d) return fail(GHA_ERR_STRIDE, "cache rows overlap (token stride < d)");
  const int span_rows = paged ? page_size : L_cap;
  const int64_t eb = elem_size(cache_dtype);
  if (!gha::span_below((int64_t)span_rows + 64, std::max(k_cache->ss, v_cache->ss), eb, (int64_t)1 << 31))
    return fail(GHA_ERR_STRIDE, "one %s spans 2 GiB or more", paged ? "page" : "sequence");
  const int rows = (h_q / h_kv) * s_q;
  const int L_plan = window_keys(L_max_hint, s_q, window);
  const int target = cache_dtype == GHA_FP8_E4M3 ? GHA_SD_WGS_8BIT : GHA_SD_WGS;
  const size_t need = stream_decode_ws(B, h_kv, 1, rows, L_plan, d, target);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(GHA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 15u) != 0)
    return fail(GHA_ERR_ALIGN, "workspace not 16-byte aligned");
  if ((int64_t)B * ((L_cap + 127) / 128) >= (1LL << 31))
    return fail(GHA_ERR_SHAPE, "problem too large for one launch");
  if ((s = check_device()) != GHA_OK) return s;
  if ((s = check_lengths_on_device(seqlens_k, B, s_q, L_cap, workspace, stream, name)) != GHA_OK) return s;

  gha::StreamDecodeArgs sa{};
  sa.q = q->ptr; sa.q_sb = q->sb; sa.q_sh = q->sh; sa.q_ss = q->ss;
  sa.k = k_cache->ptr; sa.k_sb = k_cache->sb; sa.k_sh = k_cache->sh; sa.k_ss = k_cache->ss;
  sa.v = v_cache->ptr; sa.v_sb = v_cache->sb; sa.v_sh = v_cache->sh; sa.v_ss = v_cache->ss;
  sa.seqlens = seqlens_k;
  sa.o = o->ptr; sa.o_sb = o->sb; sa.o_sh = o->sh; sa.o_ss = o->ss;
  sa.lse = lse;
  sa.B = B; sa.n_groups = h_kv; sa.qpg = h_q / h_kv; sa.s_q = s_q; sa.rows = rows; sa.L_cap = L_cap;
  sa.v_hpg = 1; sa.v_sph = 1;
  sa.team = 1;
  sa.n_wg = stream_decode_wgs(B, h_kv, 1, L_plan, target);
  stream_decode_carve(sa, workspace, d);
  sa.scale = (scale > 0.f ? scale : 1.0f / std::sqrt((float)d)) * k_scale;
  sa.v_scale = v_scale;
  sa.window = window;
  sa.block_table = block_table;
  sa.bt_stride = paged ? bt_stride : 0;
  sa.page_size = paged ? page_size : 0;
  return launched(gha::launch_stream_decode(sa, d, 0, d, 1, out_dtype == GHA_F32,
                                            reinterpret_cast<hipStream_t>(stream), cache_dtype == GHA_FP8_E4M3),
                  name);
}
}  // namespace

extern "C" {

gha_status gqa_decode_paged(const gha_tensor* q, const gha_tensor* k_cache, const gha_tensor* v_cache,
                            const int32_t* block_table, int bt_stride, int page_size,
                            const int32_t* seqlens_k, const gha_tensor* o, float* lse, int B, int h_q,
                            int h_kv, int s_q, int L_cap, int L_max_hint, int window, int d,
                            gha_dtype in_dtype, gha_dtype out_dtype, float scale, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return stream_gqa_decode(q, k_cache, v_cache, block_table, bt_stride, page_size, seqlens_k, o, lse, B, h_q,
                           h_kv, s_q, L_cap, L_max_hint, window, d, in_dtype, in_dtype, out_dtype, scale, 1.f, 1.f,
                           workspace, workspace_bytes, stream, "gqa_decode_paged");
}

gha_status gqa_decode_fp8(const gha_tensor* q, const gha_tensor* k_cache, const gha_tensor* v_cache,
                          float k_scale, float v_scale, const int32_t* block_table, int bt_stride, int page_size,
                          const int32_t* seqlens_k, const gha_tensor* o, float* lse, int B, int h_q, int h_kv,
                          int s_q, int L_cap, int L_max_hint, int window, int d, gha_dtype out_dtype, float scale,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(GHA_ERR_SHAPE, "k_scale and v_scale must be positive and finite");
  return stream_gqa_decode(q, k_cache, v_cache, block_table, bt_stride, page_size, seqlens_k, o, lse, B, h_q,
                           h_kv, s_q, L_cap, L_max_hint, window, d, GHA_BF16, GHA_FP8_E4M3, out_dtype, scale,
                           k_scale, v_scale, workspace, workspace_bytes, stream, "gqa_decode_fp8");
}

gha_status gta_shared_score_prefill(const gha_tensor* q, const gha_tensor* k, const gha_tensor* v,
                                    const gha_tensor* o, float* lse, int B, int h, int n_grp, int S,
                                    int d_qk, int d_v, gha_dtype in_dtype, gha_dtype out_dtype,
                                    float scale, int causal, void* stream) {
  if (B < 1 || h < 1 || n_grp < 1 || S < 1) return fail(GHA_ERR_SHAPE, "sizes must be positive");
  if (!within_limits(B, h, n_grp, 1, S, 1)) return limits_fail();
  if (h % n_grp) return fail(GHA_ERR_GROUPING, "h=%d is not a multiple of n_grp=%d", h, n_grp);
  const int per = h / n_grp;
  if ((d_qk != 64 && d_qk != 128) || !gta_dv_ok(d_v))
    return fail(GHA_ERR_HEAD_DIM, "need d_qk in {64,128} and d_v in {64,128,256} (d_qk=%d d_v=%d)", d_qk, d_v);
  if (in_dtype != GHA_BF16 || (out_dtype != GHA_BF16 && out_dtype != GHA_F32))
    return fail(GHA_ERR_DTYPE, "GTA takes bf16 inputs and bf16 or f32 outputs");
  gha_status s;
  if ((s = check_view("q", q, in_dtype, B > 1, n_grp > 1, S > 1)) != GHA_OK) return s;
  if ((s = check_view("k", k, in_dtype, B > 1, n_grp > 1, S > 1)) != GHA_OK) return s;
  if ((s = check_view("v", v, in_dtype, B > 1, h > 1, S > 1)) != GHA_OK) return s;
  if ((s = check_view("o", o, out_dtype, B > 1, h > 1, S > 1)) != GHA_OK) return s;
  if ((s = check_device()) != GHA_OK) return s;

  gha::PrefillArgs a{};
  a.q = q->ptr; a.q_sb = q->sb; a.q_sh = q->sh; a.q_ss = q->ss;
  a.k = k->ptr; a.k_sb = k->sb; a.k_sh = k->sh; a.k_ss = k->ss;
  a.v = v->ptr; a.v_sb = v->sb; a.v_sh = v->sh; a.v_ss = v->ss;
  a.o = o->ptr; a.o_sb = o->sb; a.o_sh = o->sh; a.o_ss = o->ss;
  a.lse = lse; a.lse_heads = n_grp;
  a.S_q = S; a.S_k = S; a.h_kv = n_grp; a.group = per;
  a.heads_per_wg = 1; a.n_subgroups = 1;
  const GtaSources src = gta_prefill_sources(per, d_v);
  a.v_hpg = per; a.v_sph = src.sph;
  // both GTA kernels take 128 positions per work-group
  const int pos_per_wg = gha::gta_positions_per_wg();
  a.n_qblocks = (S + pos_per_wg - 1) / pos_per_wg;
  const int64_t nb = (int64_t)B * n_grp * a.n_qblocks;
  if (nb > (1LL << 30)) return fail(GHA_ERR_SHAPE, "problem too large for one launch");
  a.n_blocks = (int)nb;
  a.causal = causal ? 1 : 0;
  a.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)d_qk);
  a.B = B;
  if (!gha::gta_layout_supported(a, d_qk, d_v))
    return fail(GHA_ERR_STRIDE, "k/v rows overlap or one sequence spans 2 GiB or more (k ss=%lld, v ss=%lld, S=%d)",
                (long long)k->ss, (long long)v->ss, S);
  // Kernel choice (measured on the GTA workloads): the one-stream kernel,
  // two work-groups per CU, is the faster one unless a causal grid fits in
  // one round of them; then its heaviest q-blocks run out the clock alone,
  // and the exchange kernel, one work-group per CU and two rounds, balances
  // better.
  const int cus = gha::device_cus();
  const bool use_fused = !causal || cus <= 0 || a.n_blocks > 2 * cus;
  // launch l applies the scores to sources l nvs .. of every group: the v and
  // o views start at that source's head and column; the lse is written once
  const int64_t ob = elem_size(out_dtype);
  for (int l = 0; l < src.launches; ++l) {
    const int s0 = l * src.nvs;
    const int64_t vofs = (int64_t)(s0 / src.sph) * v->sh + (int64_t)(s0 % src.sph) * src.dvw;
    const int64_t oofs = (int64_t)(s0 / src.sph) * o->sh + (int64_t)(s0 % src.sph) * src.dvw;
    a.v = static_cast<const unsigned char*>(v->ptr) + vofs * 2;
    a.o = static_cast<unsigned char*>(o->ptr) + oofs * ob;
    a.lse = l == 0 ? lse : nullptr;
    const hipError_t e = use_fused ? gha::launch_gta_fused(a, d_qk, src.nvs, out_dtype == GHA_F32,
                                                           reinterpret_cast<hipStream_t>(stream))
                                   : gha::launch_gta(a, d_qk, src.nvs, out_dtype == GHA_F32,
                                                     reinterpret_cast<hipStream_t>(stream));
    const gha_status st = launched(e, "gta_shared_score_prefill");
    if (st != GHA_OK) return st;
  }
  return GHA_OK;
}

size_t gta_shared_score_decode_workspace_bytes(int B, int h, int n_grp, int s_q, int L_max_hint, int d_v) {
  if (B < 1 || h < 1 || n_grp < 1 || s_q < 1 || s_q > 32 || L_max_hint < 1 || !gta_dv_ok(d_v) || h % n_grp) return 0;
  if (!within_limits(B, h, n_grp, s_q, L_max_hint, 1)) return 0;
  // the launches over a group's value sources run one after another on the
  // stream and reuse one launch's workspace
  const GtaSources src = gta_decode_sources(h / n_grp, d_v, s_q);
  return stream_decode_ws(B, n_grp, 1, s_q, L_max_hint, src.nvs * src.dvw);
}

gha_status gta_shared_score_decode(const gha_tensor* q, const gha_tensor* k_cache, const gha_tensor* v_cache,
                                   const int32_t* seqlens_k, const gha_tensor* o, float* lse, int B, int h,
                                   int n_grp, int s_q, int L_cap, int L_max_hint, int d_qk, int d_v,
                                   gha_dtype in_dtype, gha_dtype out_dtype, float scale, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (B < 1 || h < 1 || n_grp < 1 || s_q < 1 || L_cap < 1 || L_max_hint < 1)
    return fail(GHA_ERR_SHAPE, "sizes must be positive");
  if (!within_limits(B, h, n_grp, s_q, L_cap, L_max_hint)) return limits_fail();
  if (h % n_grp) return fail(GHA_ERR_GROUPING, "h=%d is not a multiple of n_grp=%d", h, n_grp);
  const int per = h / n_grp;
  if (L_max_hint > L_cap || s_q > L_max_hint)
    return fail(GHA_ERR_SHAPE, "need s_q <= L_max_hint <= L_cap (s_q=%d L_max_hint=%d L_cap=%d)", s_q, L_max_hint, L_cap);
  if (s_q > 32) return fail(GHA_ERR_SHAPE, "s_q=%d above 32 new tokens per step", s_q);
  if ((d_qk != 64 && d_qk != 128) || !gta_dv_ok(d_v))
    return fail(GHA_ERR_HEAD_DIM, "need d_qk in {64,128} and d_v in {64,128,256} (d_qk=%d d_v=%d)", d_qk, d_v);
  if (in_dtype != GHA_BF16 || (out_dtype != GHA_BF16 && out_dtype != GHA_F32))
    return fail(GHA_ERR_DTYPE, "GTA decode takes bf16 inputs and bf16 or f32 outputs");
  if (seqlens_k == nullptr) return fail(GHA_ERR_NULL, "seqlens_k is null");
  gha_status s;
  if ((s = check_view("q", q, in_dtype, B > 1, n_grp > 1, s_q > 1)) != GHA_OK) return s;
  if ((s = check_view("k_cache", k_cache, in_dtype, B > 1, n_grp > 1, true)) != GHA_OK) return s;
  if ((s = check_view("v_cache", v_cache, in_dtype, B > 1, h > 1, true)) != GHA_OK) return s;
  if ((s = check_view("o", o, out_dtype, B > 1, h > 1, s_q > 1)) != GHA_OK) return s;
  if (k_cache->ss < d_qk || v_cache->ss < d_v)
    return fail(GHA_ERR_STRIDE, "cache rows overlap (k ss=%lld, v ss=%lld)", (long long)k_cache->ss, (long long)v_cache->ss);
  if (!span_ok(L_cap, k_cache->ss) || !span_ok(L_cap, v_cache->ss))
    return fail(GHA_ERR_SHAPE, "one sequence of a cache spans 2 GiB or more (L_cap=%d)", L_cap);
  const size_t need = gta_shared_score_decode_workspace_bytes(B, h, n_grp, s_q, L_max_hint, d_v);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(GHA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 15u) != 0) return fail(GHA_ERR_ALIGN, "workspace not 16-byte aligned");
  if ((s = check_device()) != GHA_OK) return s;
  if ((s = check_lengths_on_device(seqlens_k, B, s_q, L_cap, workspace, stream, "gta_shared_score_decode")) != GHA_OK) return s;

  gha::StreamDecodeArgs a{};
  a.q = q->ptr; a.q_sb = q->sb; a.q_sh = q->sh; a.q_ss = q->ss;
  a.k = k_cache->ptr; a.k_sb = k_cache->sb; a.k_sh = k_cache->sh; a.k_ss = k_cache->ss;
  a.v = v_cache->ptr; a.v_sb = v_cache->sb; a.v_sh = v_cache->sh; a.v_ss = v_cache->ss;
  a.seqlens = seqlens_k;
  a.o = o->ptr; a.o_sb = o->sb; a.o_sh = o->sh; a.o_ss = o->ss;
  a.lse = lse;
  a.B = B; a.n_groups = n_grp; a.qpg = 1; a.s_q = s_q; a.rows = s_q; a.L_cap = L_cap;
  const GtaSources src = gta_decode_sources(per, d_v, s_q);
  a.v_hpg = per; a.v_sph = src.sph;
  a.team = 1;
  a.n_wg = stream_decode_wgs(B, n_grp, 1, L_max_hint);
  stream_decode_carve(a, workspace, src.nvs * src.dvw);
  a.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)d_qk);
  if ((int64_t)B * ((L_cap + 127) / 128) >= (1LL << 31)) return fail(GHA_ERR_SHAPE, "problem too large for one launch");
  // launch l covers sources l nvs .. of every group (views start at that
  // source's head and column); the per-group lse is written once
  const int64_t ob = elem_size(out_dtype);
  for (int l = 0; l < src.launches; ++l) {
    const int s0 = l * src.nvs;
    const int64_t vofs = (int64_t)(s0 / src.sph) * v_cache->sh + (int64_t)(s0 % src.sph) * src.dvw;
    const int64_t oofs = (int64_t)(s0 / src.sph) * o->sh + (int64_t)(s0 % src.sph) * src.dvw;
    a.v = static_cast<const unsigned char*>(v_cache->ptr) + vofs * 2;
    a.o = static_cast<unsigned char*>(o->ptr) + oofs * ob;
    a.lse = l == 0 ? lse : nullptr;
    const gha_status st = launched(gha::launch_stream_decode(a, d_qk, 0, src.dvw, src.nvs, out_dtype == GHA_F32,
                                                             reinterpret_cast<hipStream_t>(stream)),
                                   "gta_shared_score_decode");
    if (st != GHA_OK) return st;
  }
  return GHA_OK;
}

size_t gqla_gqa_decode_workspace_bytes(int B, int h_q, int g, int s_q, int L_max_hint, int d_h) {
  if (B < 1 || h_q < 1 || g < 1 || s_q < 1 || L_max_hint < 1 || d_h != 128 || h_q % g) return 0;
  if (!within_limits(B, h_q, g, s_q, L_max_hint, 1) || (h_q / g) * s_q > 32) return 0;
  return stream_decode_ws(B, g, g, (h_q / g) * s_q, L_max_hint, d_h);
}

gha_status gqla_gqa_decode(const gha_tensor* q_c, const gha_tensor* q_r, const gha_tensor* k_c,
                           const gha_tensor* k_r, const gha_tensor* v_cache, const int32_t* seqlens_k,
                           const gha_tensor* o, float* lse, int B, int h_q, int g, int s_q, int L_cap,
                           int L_max_hint, int d_h, int d_r, gha_dtype in_dtype, gha_dtype out_dtype,
                           float scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 1 || h_q < 1 || g < 1 || s_q < 1 || L_cap < 1 || L_max_hint < 1)
    return fail(GHA_ERR_SHAPE, "sizes must be positive");
  if (!within_limits(B, h_q, g, s_q, L_cap, L_max_hint)) return limits_fail();
  if (h_q % g) return fail(GHA_ERR_GROUPING, "h_q=%d is not a multiple of g=%d", h_q, g);
  if (L_max_hint > L_cap || s_q > L_max_hint)
    return fail(GHA_ERR_SHAPE, "need s_q <= L_max_hint <= L_cap (s_q=%d L_max_hint=%d L_cap=%d)", s_q, L_max_hint, L_cap);
  const int rows = (h_q / g) * s_q;
  if (rows > 32) return fail(GHA_ERR_SHAPE, "(h_q/g)*s_q=%d above 32 query rows per group", rows);
  if (d_h != 128 || d_r != 64) return fail(GHA_ERR_HEAD_DIM, "need d_h == 128 and d_r == 64 (got %d, %d)", d_h, d_r);
  if (!(scale > 0.f)) return fail(GHA_ERR_SHAPE, "scale must be given (> 0): 1/sqrt(d_h + d_r) for the expanded key");
  if (in_dtype != GHA_BF16 || (out_dtype != GHA_BF16 && out_dtype != GHA_F32))
    return fail(GHA_ERR_DTYPE, "GQLA decode takes bf16 inputs and bf16 or f32 outputs");
  if (seqlens_k == nullptr) return fail(GHA_ERR_NULL, "seqlens_k is null");
  gha_status s;
  if ((s = check_view("q_c", q_c, in_dtype, B > 1, h_q > 1, s_q > 1)) != GHA_OK) return s;
  if ((s = check_view("q_r", q_r, in_dtype, B > 1, h_q > 1, s_q > 1)) != GHA_OK) return s;
  if ((s = check_view("k_c", k_c, in_dtype, B > 1, g > 1, true)) != GHA_OK) return s;
  if ((s = check_view("k_r", k_r, in_dtype, B > 1, false, true)) != GHA_OK) return s;
  if ((s = check_view("v_cache", v_cache, in_dtype, B > 1, g > 1, true)) != GHA_OK) return s;
  if ((s = check_view("o", o, out_dtype, B > 1, h_q > 1, s_q > 1)) != GHA_OK) return s;
  if (k_c->ss < d_h || k_r->ss < d_r || v_cache->ss < d_h)
    return fail(GHA_ERR_STRIDE, "cache rows overlap (k_c ss=%lld, k_r ss=%lld, v ss=%lld)", (long long)k_c->ss,
                (long long)k_r->ss, (long long)v_cache->ss);
  if (!span_ok(L_cap, k_c->ss) || !span_ok(L_cap, k_r->ss) || !span_ok(L_cap, v_cache->ss))
    return fail(GHA_ERR_SHAPE, "one sequence of a cache spans 2 GiB or more (L_cap=%d)", L_cap);
  const size_t need = gqla_gqa_decode_workspace_bytes(B, h_q, g, s_q, L_max_hint, d_h);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(GHA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 15u) != 0) return fail(GHA_ERR_ALIGN, "workspace not 16-byte aligned");
  if ((s = check_device()) != GHA_OK) return s;
  if ((s = check_lengths_on_device(seqlens_k, B, s_q, L_cap, workspace, stream, "gqla_gqa_decode")) != GHA_OK) return s;

  gha::StreamDecodeArgs a{};
  a.q = q_c->ptr; a.q_sb = q_c->sb; a.q_sh = q_c->sh; a.q_ss = q_c->ss;
  a.q2 = q_r->ptr; a.q2_sb = q_r->sb; a.q2_sh = q_r->sh; a.q2_ss = q_r->ss;
  a.k = k_c->ptr; a.k_sb = k_c->sb; a.k_sh = k_c->sh; a.k_ss = k_c->ss;
  a.k2 = k_r->ptr; a.k2_sb = k_r->sb; a.k2_ss = k_r->ss;
  a.v = v_cache->ptr; a.v_sb = v_cache->sb; a.v_sh = v_cache->sh; a.v_ss = v_cache->ss;
  a.seqlens = seqlens_k;
  a.o = o->ptr; a.o_sb = o->sb; a.o_sh = o->sh; a.o_ss = o->ss;
  a.lse = lse;
  a.B = B; a.n_groups = g; a.qpg = h_q / g; a.s_q = s_q; a.rows = rows; a.L_cap = L_cap;
  a.v_hpg = 1; a.v_sph = 1;
  a.team = g;  // every group reads the shared RoPE key
  a.n_wg = stream_decode_wgs(B, g, g, L_max_hint);
  stream_decode_carve(a, workspace, d_h);
  a.scale = scale;
  if ((int64_t)B * ((L_cap + 127) / 128) >= (1LL << 31)) return fail(GHA_ERR_SHAPE, "problem too large for one launch");
  return launched(gha::launch_stream_decode(a, d_h, d_r, d_h, 1, out_dtype == GHA_F32,
                                            reinterpret_cast<hipStream_t>(stream)),
                  "gqla_gqa_decode");
}

size_t latent_absorb_decode_workspace_bytes(int B, int h_q, int s_q, int L_max_hint, int r_kv) {
  if (B < 1 || h_q < 1 || s_q < 1 || L_max_hint < 1 || r_kv != 512) return 0;
  if (!within_limits(B, h_q, 1, s_q, L_max_hint, 1)) return 0;
  const int n_rb = latent_row_blocks(h_q, s_q);
  const int T = gha::latent_tile_tokens();
  const int n_wg = gha::latent_plan_wgs(n_rb, (int64_t)B * ((L_max_hint + T - 1) / T));
  const size_t rows = (size_t)n_rb * (n_wg + B) * gha::latent_rows_per_wg();
  return rows * (size_t)r_kv * 4 + rows * 4 + (size_t)(B + 1) * 4;
}

}  // extern "C"

namespace {
// every argument check of latent_absorb_decode, nothing launched
gha_status latent_absorb_decode_check(const gha_tensor* q_lat, const gha_tensor* q_rope,
                                      const gha_tensor* c_kv, const gha_tensor* k_rope,
                                      const int32_t* seqlens_k, const gha_tensor* o_lat,
                                      int B, int h_q, int s_q, int L_cap, int L_max_hint, int r_kv,
                                      int d_r, gha_dtype in_dtype, gha_dtype out_dtype, float scale,
                                      void* workspace, size_t workspace_bytes) {
  if (B < 1 || h_q < 1 || s_q < 1 || L_cap < 1 || L_max_hint < 1)
    return fail(GHA_ERR_SHAPE, "sizes must be positive");
  if (!within_limits(B, h_q, 1, s_q, L_cap, L_max_hint)) return limits_fail();
  if (L_max_hint > L_cap || s_q > L_max_hint)
    return fail(GHA_ERR_SHAPE, "need s_q <= L_max_hint <= L_cap (s_q=%d L_max_hint=%d L_cap=%d)", s_q, L_max_hint, L_cap);
  if (r_kv != 512 || d_r != 64) return fail(GHA_ERR_HEAD_DIM, "need r_kv == 512 and d_r == 64 (got %d, %d)", r_kv, d_r);
  if (!(scale > 0.f)) return fail(GHA_ERR_SHAPE, "scale must be given (> 0) for the absorbed path");
  if (in_dtype != GHA_BF16 || (out_dtype != GHA_BF16 && out_dtype != GHA_F32))
    return fail(GHA_ERR_DTYPE, "latent decode takes bf16 inputs and bf16 or f32 outputs");
  if (seqlens_k == nullptr) return fail(GHA_ERR_NULL, "seqlens_k is null");
  gha_status s;
  if ((s = check_view("q_lat", q_lat, in_dtype, B > 1, h_q > 1, s_q > 1)) != GHA_OK) return s;
  if ((s = check_view("q_rope", q_rope, in_dtype, B > 1, h_q > 1, s_q > 1)) != GHA_OK) return s;
  if ((s = check_view("c_kv", c_kv, in_dtype, B > 1, false, true)) != GHA_OK) return s;
  if ((s = check_view("k_rope", k_rope, in_dtype, B > 1, false, true)) != GHA_OK) return s;
  if ((s = check_view("o_lat", o_lat, out_dtype, B > 1, h_q > 1, s_q > 1)) != GHA_OK) return s;
  // cache rows are read with 32-bit buffer offsets and a range that ends at
  // each sequence's last token: rows must not overlap, and one sequence must
  // span less than 2^31 bytes
  if (c_kv->ss < r_kv || k_rope->ss < d_r)
    return fail(GHA_ERR_STRIDE, "cache rows overlap (c_kv ss=%lld, k_rope ss=%lld)", (long long)c_kv->ss, (long long)k_rope->ss);
  if (!gha::span_below((int64_t)L_cap + gha::latent_tile_tokens(), std::max(c_kv->ss, k_rope->ss), 2, 1LL << 31))
    return fail(GHA_ERR_SHAPE, "one sequence of the cache spans 2 GiB or more (L_cap=%d)", L_cap);
  const size_t need = latent_absorb_decode_workspace_bytes(B, h_q, s_q, L_max_hint, r_kv);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(GHA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 15u) != 0)
    return fail(GHA_ERR_ALIGN, "workspace not 16-byte aligned");
  const int T = gha::latent_tile_tokens();
  if ((int64_t)B * latent_row_blocks(h_q, s_q) * (gha::latent_rows_per_wg() / 4) > (1LL << 30) ||
      (int64_t)B * ((L_cap + T - 1) / T + gha::latent_segment_start_tiles()) >= (1LL << 31))
    return fail(GHA_ERR_SHAPE, "problem too large for one launch");
  return GHA_OK;
}
}  // namespace

extern "C" {

gha_status latent_absorb_decode(const gha_tensor* q_lat, const gha_tensor* q_rope,
                                const gha_tensor* c_kv, const gha_tensor* k_rope,
                                const int32_t* seqlens_k, const gha_tensor* o_lat, float* lse,
                                int B, int h_q, int s_q, int L_cap, int L_max_hint, int r_kv,
                                int d_r, gha_dtype in_dtype, gha_dtype out_dtype, float scale,
                                void* workspace, size_t workspace_bytes, void* stream) {
  gha_status s = latent_absorb_decode_check(q_lat, q_rope, c_kv, k_rope, seqlens_k, o_lat, B, h_q, s_q, L_cap,
                                            L_max_hint, r_kv, d_r, in_dtype, out_dtype, scale, workspace,
                                            workspace_bytes);
  if (s != GHA_OK) return s;
  if ((s = check_device()) != GHA_OK) return s;
  if ((s = check_lengths_on_device(seqlens_k, B, s_q, L_cap, workspace, stream, "latent_absorb_decode")) != GHA_OK) return s;

  gha::LatentArgs a{};
  a.q = q_lat->ptr; a.q_sb = q_lat->sb; a.q_sh = q_lat->sh; a.q_ss = q_lat->ss;
  a.qr = q_rope->ptr; a.qr_sb = q_rope->sb; a.qr_sh = q_rope->sh; a.qr_ss = q_rope->ss;
  a.c = c_kv->ptr; a.c_sb = c_kv->sb; a.c_ss = c_kv->ss;
  a.kr = k_rope->ptr; a.kr_sb = k_rope->sb; a.kr_ss = k_rope->ss;
  a.seqlens = seqlens_k;
  a.o = o_lat->ptr; a.o_sb = o_lat->sb; a.o_sh = o_lat->sh; a.o_ss = o_lat->ss;
  a.lse = lse;
  a.B = B; a.h_q = h_q; a.s_q = s_q;
  a.L_cap = L_cap;
  a.n_rb = latent_row_blocks(h_q, s_q);
  const int T = gha::latent_tile_tokens();
  a.n_wg = gha::latent_plan_wgs(a.n_rb, (int64_t)B * ((L_max_hint + T - 1) / T));
  const size_t n_part = (size_t)a.n_rb * (a.n_wg + B) * gha::latent_rows_per_wg();
  a.ws_o = reinterpret_cast<float*>(workspace);
  a.ws_lse = a.ws_o + n_part * r_kv;
  a.ws_tiles = reinterpret_cast<int32_t*>(a.ws_lse + n_part);
  a.scale = scale;
  return launched(gha::launch_latent_decode(a, out_dtype == GHA_F32, reinterpret_cast<hipStream_t>(stream)),
                  "latent_absorb_decode");
}

size_t gqla_absorb_decode_workspace_bytes(int B, int h_q, int s_q, int L_max_hint, int r_kv) {
  const size_t lat = latent_absorb_decode_workspace_bytes(B, h_q, s_q, L_max_hint, r_kv);
  if (lat == 0) return 0;
  const size_t rows = (size_t)B * s_q * h_q;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  // latent workspace, q~ and o_lat (bf16 each), W^UK transposed (at most
  // h_q groups of 128 x r_kv)
  return up(lat) + up(rows * r_kv * 2) + up(rows * r_kv * 2) + (size_t)h_q * 128 * r_kv * 2;
}

gha_status gqla_absorb_decode(const gha_tensor* q_c, const gha_tensor* q_rope, const void* w_uk,
                              const void* w_uv, const gha_tensor* c_kv, const gha_tensor* k_rope,
                              const int32_t* seqlens_k, const gha_tensor* o, float* lse, int B, int h_q,
                              int g, int s_q, int L_cap, int L_max_hint, int d_h, int r_kv, int d_r,
                              gha_dtype in_dtype, gha_dtype out_dtype, float scale, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (B < 1 || h_q < 1 || g < 1 || s_q < 1 || L_cap < 1 || L_max_hint < 1)
    return fail(GHA_ERR_SHAPE, "sizes must be positive");
  if (!within_limits(B, h_q, g, s_q, L_cap, L_max_hint)) return limits_fail();
  if (h_q % g) return fail(GHA_ERR_GROUPING, "h_q=%d is not a multiple of g=%d", h_q, g);
  if (d_h != 128 || r_kv != 512 || d_r != 64)
    return fail(GHA_ERR_HEAD_DIM, "need d_h == 128, r_kv == 512 and d_r == 64 (got %d, %d, %d)", d_h, r_kv, d_r);
  if (in_dtype != GHA_BF16 || (out_dtype != GHA_BF16 && out_dtype != GHA_F32))
    return fail(GHA_ERR_DTYPE, "takes bf16 inputs and bf16 or f32 outputs");
  if (w_uk == nullptr || w_uv == nullptr) return fail(GHA_ERR_NULL, "w_uk or w_uv is null");
  if ((reinterpret_cast<uintptr_t>(w_uk) & 15u) || (reinterpret_cast<uintptr_t>(w_uv) & 15u))
    return fail(GHA_ERR_ALIGN, "w_uk and w_uv must be 16-byte aligned");
  if ((int64_t)B * s_q * h_q >= (1LL << 26)) return fail(GHA_ERR_SHAPE, "problem too large for one launch");
  gha_status s;
  if ((s = check_view("q_c", q_c, in_dtype, B > 1, h_q > 1, s_q > 1)) != GHA_OK) return s;
  if ((s = check_view("o", o, out_dtype, B > 1, h_q > 1, s_q > 1)) != GHA_OK) return s;
  const size_t need = gqla_absorb_decode_workspace_bytes(B, h_q, s_q, L_max_hint, r_kv);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(GHA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(GHA_ERR_ALIGN, "workspace not 256-byte aligned");
  // carve: the latent decode's own workspace, then q~ and o_lat (bf16), then
  // W^UK transposed
  const size_t rows = (size_t)B * s_q * h_q;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t lat_ws = latent_absorb_decode_workspace_bytes(B, h_q, s_q, L_max_hint, r_kv);
  unsigned char* base = reinterpret_cast<unsigned char*>(workspace);
  void* q_abs = base + up(lat_ws);
  void* o_lat = base + up(lat_ws) + up(rows * r_kv * 2);
  void* w_t = base + up(lat_ws) + 2 * up(rows * r_kv * 2);
  const gha_tensor q_lat_t{q_abs, (int64_t)s_q * h_q * r_kv, (int64_t)r_kv, (int64_t)h_q * r_kv};
  const gha_tensor o_lat_t{o_lat, (int64_t)s_q * h_q * r_kv, (int64_t)r_kv, (int64_t)h_q * r_kv};
  // the attention part is validated in full before anything is launched
  if ((s = latent_absorb_decode_check(&q_lat_t, q_rope, c_kv, k_rope, seqlens_k, &o_lat_t, B, h_q, s_q, L_cap,
                                      L_max_hint, r_kv, d_r, in_dtype, GHA_BF16, scale, base, lat_ws)) != GHA_OK)
    return s;
  if ((s = check_device()) != GHA_OK) return s;
  if ((s = check_lengths_on_device(seqlens_k, B, s_q, L_cap, base, stream, "gqla_absorb_decode")) != GHA_OK) return s;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  gha::AbsorbArgs ab{};
  ab.in = q_c->ptr; ab.in_sb = q_c->sb; ab.in_sh = q_c->sh; ab.in_ss = q_c->ss;
  ab.w = w_uk;
  ab.wt = w_t;
  ab.out = q_abs;
  ab.B = B; ab.s_q = s_q; ab.h_q = h_q; ab.g = g;
  if ((s = launched(gha::launch_absorb_query(ab, st), "gqla_absorb_decode(query)")) != GHA_OK) return s;
  if ((s = latent_absorb_decode(&q_lat_t, q_rope, c_kv, k_rope, seqlens_k, &o_lat_t, lse, B, h_q, s_q, L_cap,
                                L_max_hint, r_kv, d_r, in_dtype, GHA_BF16, scale, base, lat_ws, stream)) != GHA_OK)
    return s;
  gha::AbsorbArgs ao{};
  ao.w = w_uv;
  ao.lat = o_lat;
  ao.out = o->ptr; ao.o_sb = o->sb; ao.o_sh = o->sh; ao.o_ss = o->ss;
  ao.B = B; ao.s_q = s_q; ao.h_q = h_q; ao.g = g;
  return launched(gha::launch_absorb_output(ao, out_dtype == GHA_F32, st), "gqla_absorb_decode(output)");
}

}  // extern "C"
