/* gha.h - C ABI of the grouped-head attention library for AMD Instinct MI355X
 * (gfx950).
 *
 * Every operation is exact causal scaled dot-product attention
 * o = softmax(scale * q k^T) v with fp32 accumulation; they differ in which
 * heads share what.  Six kinds:
 *
 *   gqa_prefill               grouped-query attention over a whole sequence:
 *                             consecutive groups of h_q/h_kv query heads share
 *                             one key head and one value head.  One group is
 *                             MQA, h_kv == h_q is MHA.  ("Grouped Query
 *                             Attention (GQA)", Ultralytics glossary, section
 *                             "How GQA works".)
 *   gqa_decode                the same for s_q new query tokens per sequence
 *                             against a contiguous KV cache with per-sequence
 *                             lengths; split-KV with a log-sum-exp merge.
 *   gta_shared_score_prefill  GTA's grouped shared attention matrix: heads are
 *                             split into groups, each group has one query/key
 *                             pair and so one score matrix, which is applied
 *                             to the value of every head in the group.  ("GTA:
 *                             Grouped-head latenT Attention" news article,
 *                             grouped shared attention matrix mechanism.)
 *   gta_shared_score_decode   the same shared score for s_q new tokens per
 *                             sequence against a contiguous cache of one key
 *                             per group and one value per head.
 *   gqla_gqa_decode           the GQA path of GQLA: per group a cached key k^C
 *                             and value, plus one RoPE key k^R per token shared
 *                             by every group; head i of group j uses the key
 *                             [k^C_j; k^R].  ("GQLA: Group-Query Latent
 *                             Attention ...", section 1, section 3.1 Eq. (1).)
 *   latent_absorb_decode      the absorbed (MQA-like) path of MLA/GQLA: every
 *                             query head attends straight over the cached
 *                             latent c^KV (width r_kv) plus the shared RoPE key
 *                             k^R (width d_r); the value is the latent itself.
 *                             ("GQLA: Group-Query Latent Attention ...",
 *                             section 1, section 3.1 Eq. (1), Figure 2 right.)
 *
 * and their variants, each declared with its own contract below:
 * gqa_decode_paged (block-table KV cache, optional sliding window),
 * gqa_decode_fp8 (E4M3 caches with per-tensor scales), gqla_gqa_prefill (the
 * GQLA expand path over a whole sequence), gqla_absorb_decode (GQLA absorbed
 * into the latent on the device) and gqa_decode_noalloc (gqa_decode with
 * library-owned scratch, for callers that cannot allocate).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors are described by gha_tensor: a device pointer plus element strides
 * for the batch, head and token axes.  The feature (last) axis must be
 * contiguous, and ptr and every stride must keep each row 16-byte aligned
 * (GHA_ERR_ALIGN otherwise).  Strides may be any non-negative values, so
 * (B, H, S, D), (B, S, H, D) and views into larger buffers are all accepted.
 *
 * Element types: GHA_BF16 inputs with GHA_BF16 or GHA_F32 outputs everywhere;
 * GHA_F32 inputs (with GHA_F32 outputs) for gqa_prefill only.
 *
 * Causal alignment is bottom-right: with S_k keys and S_q queries, query t
 * sees keys 0 .. t + (S_k - S_q).  For prefill with S_q == S_k that is the
 * usual u <= t; for decode, seqlens_k[b] counts the cache including the s_q
 * new tokens, so query t of sequence b sees keys 0 .. L_b - s_q + t.
 *
 * Outputs: o has the query's batch/head/token indexing with the value width;
 * lse (optional, may be NULL) receives log(sum_u exp(scale * q.k_u)) in
 * natural-log units, fp32, densely packed as documented per call.
 *
 * Ownership and errors: the caller owns every buffer (device memory, e.g.
 * from torch).  The library never allocates, frees or synchronises; it
 * enqueues kernels on `stream` (a hipStream_t, NULL for the default stream)
 * and returns.  Every argument is checked on the host before anything is
 * launched; on any error nothing is launched or written, the status says what
 * class of error it was and gha_last_error() (thread-local) gives the detail.
 * A failed launch returns GHA_ERR_HIP.  Results are deterministic: the split
 * plan depends only on the arguments and no atomics are used.
 */
#ifndef GHA_H_
#define GHA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GHA_OK = 0,
  GHA_ERR_NULL = 1,      /* a required pointer is NULL */
  GHA_ERR_SHAPE = 2,     /* a size is out of range or inconsistent */
  GHA_ERR_GROUPING = 3,  /* h_q % h_kv != 0, or h % n_grp != 0 */
  GHA_ERR_STRIDE = 4,    /* a negative stride */
  GHA_ERR_ALIGN = 5,     /* a row is not 16-byte aligned */
  GHA_ERR_DTYPE = 6,     /* unsupported input/output element types */
  GHA_ERR_HEAD_DIM = 7,  /* unsupported head / latent width */
  GHA_ERR_WORKSPACE = 8, /* workspace missing or too small */
  GHA_ERR_HIP = 9,       /* no usable device, or a launch failed */
  GHA_ERR_PRECONDITION = 10 /* debug checks: a sequence length outside [s_q, L_cap] */
} gha_status;

typedef enum { GHA_F32 = 0, GHA_BF16 = 1, GHA_FP8_E4M3 = 2 } gha_dtype;  /* E4M3: caches of gqa_decode_fp8 */

/* A strided view: element (b, h, s, c) lives at ptr[b*sb + h*sh + s*ss + c]. */
typedef struct {
  void* ptr;
  int64_t sb, sh, ss;
} gha_tensor;

/* Grouped-query attention over a sequence ("How GQA works": a group of
 * consecutive query heads shares one key head and one value head; inside each
 * head the computation is ordinary scaled dot-product attention).
 *   q (B, h_q, S_q, d), k (B, h_kv, S_k, d), v (B, h_kv, S_k, d),
 *   o (B, h_q, S_q, d); lse NULL or dense fp32 (B, h_q, S_q).
 * Query head i reads key/value head i / (h_q / h_kv).
 * Requires 1 <= S_q <= S_k when causal; d in {64, 128};
 * in/out: BF16/BF16, BF16/F32 or F32/F32.  scale <= 0 means 1/sqrt(d). */
gha_status gqa_prefill(const gha_tensor* q, const gha_tensor* k, const gha_tensor* v,
                       const gha_tensor* o, float* lse,
                       int B, int h_q, int h_kv, int S_q, int S_k, int d,
                       gha_dtype in_dtype, gha_dtype out_dtype,
                       float scale, int causal, void* stream);

/* One decode step of grouped-query attention against a contiguous KV cache
 * (the GQLA page's section 1: each generated token reads the whole cached
 * history).
 *   q (B, h_q, s_q, d); k_cache, v_cache (B, h_kv, L_cap, d);
 *   seqlens_k: device int32 (B,), s_q <= seqlens_k[b] <= L_cap, counting the
 *   s_q new tokens, whose keys are the last s_q cached;
 *   o (B, h_q, s_q, d); lse NULL or dense fp32 (B, h_q, s_q).
 * L_max_hint: an upper bound on max_b seqlens_k[b] (<= L_cap); it sizes the
 * split plan, and lengths above it are a precondition violation.
 * d == 128 or 64; in BF16, out BF16 or F32.  scale <= 0 means 1/sqrt(d).
 * workspace: device memory of at least gqa_decode_workspace_bytes(...) bytes
 * (the split partials); its contents on entry do not matter. */
gha_status gqa_decode(const gha_tensor* q, const gha_tensor* k_cache,
                      const gha_tensor* v_cache, const int32_t* seqlens_k,
                      const gha_tensor* o, float* lse,
                      int B, int h_q, int h_kv, int s_q, int L_cap, int L_max_hint,
                      int d, gha_dtype in_dtype, gha_dtype out_dtype, float scale,
                      void* workspace, size_t workspace_bytes, void* stream);

size_t gqa_decode_workspace_bytes(int B, int h_q, int h_kv, int s_q, int L_max_hint, int d);

/* One decode step of grouped-query attention against a paged KV cache, a
 * sliding window, or both (GQA page, "GQA vs related techniques": paged
 * attention allocates the cache in fixed-size blocks, and a sliding window
 * bounds the tokens each query attends to; the GQLA page's section 2 names
 * paged caches as complementary to the cache layout).
 *   block_table NULL: k_cache, v_cache are contiguous (B, h_kv, L_cap, d) as
 *   for gqa_decode, and bt_stride, page_size are ignored.
 *   block_table non-NULL: device int32 (B, bt_stride); key u of sequence b
 *   lives in page block_table[b * bt_stride + u / page_size] at token
 *   u % page_size; k_cache, v_cache describe the page pool with (sb, sh, ss)
 *   = (page, KV head, token in page) strides, e.g. (n_pages, h_kv,
 *   page_size, d) or (n_pages, page_size, h_kv, d) views.  page_size is a
 *   positive multiple of 32 and bt_stride * page_size >= L_cap.  Only the
 *   entries of pages holding keys some query sees are read; they must be
 *   valid page indices.
 *   window: 0 for none; else query t of sequence b sees only keys
 *   L_b - s_q + t - window + 1 .. L_b - s_q + t (its own key and the
 *   window - 1 before it).
 *   seqlens_k, q, o, lse, L_cap, L_max_hint, scale as in gqa_decode;
 *   (h_q / h_kv) * s_q <= 32; d in {64, 128}; in BF16, out BF16 or F32.
 * One page (or, unpaged, one sequence) of a cache must span less than 2 GiB.
 * workspace: at least gqa_decode_paged_workspace_bytes(...) bytes. */
gha_status gqa_decode_paged(const gha_tensor* q, const gha_tensor* k_cache,
                            const gha_tensor* v_cache, const int32_t* block_table,
                            int bt_stride, int page_size, const int32_t* seqlens_k,
                            const gha_tensor* o, float* lse,
                            int B, int h_q, int h_kv, int s_q, int L_cap, int L_max_hint,
                            int window, int d, gha_dtype in_dtype, gha_dtype out_dtype,
                            float scale, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes for gqa_decode_paged and gqa_decode_fp8 with these sizes
 * (the larger of the two plans; 0 for sizes either call rejects). */
size_t gqa_decode_paged_workspace_bytes(int B, int h_q, int h_kv, int s_q, int L_max_hint,
                                        int window, int d);

/* gqa_decode_paged over caches of 8-bit floats (the GQLA page's section 2
 * names quantized KV storage as complementary to the cache layout): k_cache
 * and v_cache hold OCP E4M3 codes (1 sign, 4 exponent bits with bias 7,
 * 3 mantissa bits; no infinities), one byte per element, strides in
 * elements; key u is code * k_scale and value u is code * v_scale, one scale
 * per tensor (k_scale, v_scale > 0).  Everything else (contiguous or paged
 * layout, window, q in BF16, out BF16 or F32, scale <= 0 meaning 1/sqrt(d))
 * as gqa_decode_paged; d in {64, 128}.  The workspace is that of
 * gqa_decode_paged_workspace_bytes(...). */
gha_status gqa_decode_fp8(const gha_tensor* q, const gha_tensor* k_cache, const gha_tensor* v_cache,
                          float k_scale, float v_scale, const int32_t* block_table, int bt_stride,
                          int page_size, const int32_t* seqlens_k, const gha_tensor* o, float* lse,
                          int B, int h_q, int h_kv, int s_q, int L_cap, int L_max_hint, int window,
                          int d, gha_dtype out_dtype, float scale, void* workspace,
                          size_t workspace_bytes, void* stream);

/* GTA shared-score attention (GTA news article, grouped shared attention
 * matrix: a group computes its attention scores once and every head of the
 * group uses that same matrix).
 *   q, k (B, n_grp, S, d_qk): one query and one key per group;
 *   v (B, h, S, d_v), o (B, h, S, d_v): per head; head i is in group
 *   i / (h / n_grp); lse NULL or dense fp32 (B, n_grp, S), one per group.
 * Requires h % n_grp == 0, d_qk in {64, 128}, d_v in {64, 128, 256}; any
 * number of heads per group; in BF16, out BF16 or F32.  scale <= 0 means
 * 1/sqrt(d_qk).  The scores are applied to the group's values in slices of
 * at most 256 columns; a group with more value columns than that takes
 * several launches on `stream`, each recomputing the group's scores. */
gha_status gta_shared_score_prefill(const gha_tensor* q, const gha_tensor* k,
                                    const gha_tensor* v, const gha_tensor* o, float* lse,
                                    int B, int h, int n_grp, int S, int d_qk, int d_v,
                                    gha_dtype in_dtype, gha_dtype out_dtype,
                                    float scale, int causal, void* stream);

/* One decode step of GTA shared-score attention against a contiguous cache
 * (GTA news article, grouped shared attention matrix; decode as in the GQLA
 * page's section 1: each new token reads the whole cached history).
 *   q (B, n_grp, s_q, d_qk): one query per group and new token;
 *   k_cache (B, n_grp, L_cap, d_qk): one key per group and token;
 *   v_cache (B, h, L_cap, d_v): one value per head; head i is in group
 *   i / (h / n_grp) and applies its group's score vector to its own values;
 *   seqlens_k: device int32 (B,), s_q <= seqlens_k[b] <= L_cap, counting the
 *   new tokens (bottom-right alignment as in gqa_decode);
 *   o (B, h, s_q, d_v); lse NULL or dense fp32 (B, n_grp, s_q), one per group.
 * d_qk in {64, 128}, d_v in {64, 128, 256}, any number of heads per group,
 * s_q <= 32; in BF16, out BF16 or F32; scale <= 0 means 1/sqrt(d_qk).  Rows
 * of a cache must not overlap (ss >= width) and one (batch, group or head)
 * sequence must span less than 2 GiB.  The scores are applied to the group's
 * values in slices of at most 512 columns (256 when s_q > 16); a wider group
 * takes several launches on `stream`, each reading the group's keys again.
 * workspace: at least gta_shared_score_decode_workspace_bytes(...) bytes of
 * device memory (one slice's partials, reused by the launches in turn); its
 * contents on entry do not matter. */
gha_status gta_shared_score_decode(const gha_tensor* q, const gha_tensor* k_cache,
                                   const gha_tensor* v_cache, const int32_t* seqlens_k,
                                   const gha_tensor* o, float* lse,
                                   int B, int h, int n_grp, int s_q, int L_cap, int L_max_hint,
                                   int d_qk, int d_v, gha_dtype in_dtype, gha_dtype out_dtype,
                                   float scale, void* workspace, size_t workspace_bytes,
                                   void* stream);

size_t gta_shared_score_decode_workspace_bytes(int B, int h, int n_grp, int s_q, int L_max_hint,
                                               int d_v);

/* One decode step of GQLA's GQA path (GQLA section 1: the per-group expanded
 * cache of 2 g d_h + d^R elements per token; section 3.1, Eq. (1): the group
 * key is the up-projected latent k^C concatenated with the decoupled RoPE key
 * k^R, which all groups share).  The score of head i (group j = i / (h_q/g))
 * with token u is scale * (q_c_i . k_c_{j,u} + q_r_i . k_r_u); its value is
 * v_{j,u}.
 *   q_c (B, h_q, s_q, d_h), q_r (B, h_q, s_q, d_r): the head's query parts;
 *   k_c (B, g, L_cap, d_h), v_cache (B, g, L_cap, d_h): per group;
 *   k_r (B, L_cap, d_r): shared (its head stride is ignored);
 *   seqlens_k as in gqa_decode; o (B, h_q, s_q, d_h);
 *   lse NULL or dense fp32 (B, h_q, s_q).
 * d_h == 128, d_r == 64, (h_q / g) * s_q <= 32; in BF16, out BF16 or F32.
 * scale must be given (> 0): 1/sqrt(d_h + d_r) is the scale of the expanded
 * key.  Rows must not overlap and one sequence must span less than 2 GiB.
 * workspace: at least gqla_gqa_decode_workspace_bytes(...) bytes. */
gha_status gqla_gqa_decode(const gha_tensor* q_c, const gha_tensor* q_r, const gha_tensor* k_c,
                           const gha_tensor* k_r, const gha_tensor* v_cache,
                           const int32_t* seqlens_k, const gha_tensor* o, float* lse,
                           int B, int h_q, int g, int s_q, int L_cap, int L_max_hint,
                           int d_h, int d_r, gha_dtype in_dtype, gha_dtype out_dtype,
                           float scale, void* workspace, size_t workspace_bytes, void* stream);

size_t gqla_gqa_decode_workspace_bytes(int B, int h_q, int g, int s_q, int L_max_hint, int d_h);

/* GQLA's GQA path over a whole sequence, the compute-friendly form used for
 * prefill (GQLA section 1; section 3.1, Eq. (1): the latent is expanded into
 * per-group keys k^C_j and values v_j, and one decoupled RoPE key k^R per
 * token is shared by all groups).  Head i (group j = i / (h_q / g)) attends
 * with query [q_c_i; q_r_i] over keys [k_c_j; k_r] and takes values v_j.
 *   q_c (B, h_q, S_q, d_h), q_r (B, h_q, S_q, d_r);
 *   k_c (B, g, S_k, d_h), v (B, g, S_k, d_h): per group;
 *   k_r (B, S_k, d_r): shared (its head stride is ignored);
 *   o (B, h_q, S_q, d_h); lse NULL or dense fp32 (B, h_q, S_q).
 * Causal alignment is bottom-right (query t sees keys 0 .. S_k - S_q + t);
 * requires S_q <= S_k when causal.  d_h == 128, d_r == 64; in BF16, out BF16
 * or F32.  scale must be given (> 0): 1/sqrt(d_h + d_r) is the scale of the
 * expanded key.  Rows must not overlap and one (batch, group) sequence must
 * span less than 2 GiB. */
gha_status gqla_gqa_prefill(const gha_tensor* q_c, const gha_tensor* q_r, const gha_tensor* k_c,
                            const gha_tensor* k_r, const gha_tensor* v, const gha_tensor* o,
                            float* lse, int B, int h_q, int g, int S_q, int S_k, int d_h, int d_r,
                            gha_dtype in_dtype, gha_dtype out_dtype, float scale, int causal,
                            void* stream);

/* Absorbed latent decode (GQLA section 1 and Figure 2, right: with W^UK folded
 * into the query and W^UV into the output, all h_q heads attend directly over
 * the cache of r_kv + d_r elements per token, which serves as the one shared
 * key and value).
 *   q_lat (B, s_q, h_q, r_kv): the absorbed query (W^UK_g(i))^T q^C_i;
 *   q_rope (B, s_q, h_q, d_r): the per-head RoPE query;
 *   c_kv (B, L_cap, r_kv) and k_rope (B, L_cap, d_r): the cache (their head
 *   stride is ignored; they may be two views of one (B, L_cap, r_kv + d_r)
 *   buffer);
 *   seqlens_k: device int32 (B,), s_q <= seqlens_k[b] <= L_cap;
 *   o_lat (B, s_q, h_q, r_kv): softmax-weighted latent, before W^UV;
 *   lse NULL or dense fp32 (B, s_q, h_q).
 * For gha_tensor the (sb, sh, ss) strides are always batch, head, token:
 * for q_lat laid out (B, s_q, h_q, r_kv) contiguously, sh = r_kv and
 * ss = h_q * r_kv.
 * The score of head i and token u is scale * (q_lat_i . c_u + q_rope_i . k^R_u);
 * scale must be given (> 0): the expanded head width d_h is not an argument
 * (1/sqrt(d_h + d_r) reproduces the expanded per-group path).
 * r_kv == 512, d_r == 64; in BF16, out BF16 or F32.
 * workspace: at least latent_absorb_decode_workspace_bytes(...) bytes. */
gha_status latent_absorb_decode(const gha_tensor* q_lat, const gha_tensor* q_rope,
                                const gha_tensor* c_kv, const gha_tensor* k_rope,
                                const int32_t* seqlens_k, const gha_tensor* o_lat,
                                float* lse, int B, int h_q, int s_q, int L_cap,
                                int L_max_hint, int r_kv, int d_r,
                                gha_dtype in_dtype, gha_dtype out_dtype, float scale,
                                void* workspace, size_t workspace_bytes, void* stream);

size_t latent_absorb_decode_workspace_bytes(int B, int h_q, int s_q, int L_max_hint,
                                            int r_kv);

/* The absorbed latent decode with both absorption products done on the
 * device (GQLA section 3.1, Eq. (1), and Figure 2, right: the query of head i
 * in group j = i / (h_q / g) is folded into the latent space as
 * q~_i = (W^UK_j)^T q_c_i, attention runs over the cached latent as in
 * latent_absorb_decode, and the head's output is O_i = W^UV_j o_lat_i).
 *   q_c (B, s_q, h_q, d_h): content queries, strides as for q_lat;
 *   q_rope (B, s_q, h_q, d_r); c_kv, k_rope, seqlens_k as latent_absorb_decode;
 *   w_uk, w_uv: device bf16, (g * d_h, r_kv) row-major each, rows
 *   j * d_h .. j * d_h + d_h - 1 being group j's block; 16-byte aligned;
 *   o (B, s_q, h_q, d_h); lse NULL or dense fp32 (B, s_q, h_q).
 * d_h == 128, r_kv == 512, d_r == 64; h_q % g == 0; in BF16, out BF16 or F32;
 * scale required (> 0).  q~ is rounded to bf16 before attention.
 * workspace: at least gqla_absorb_decode_workspace_bytes(...) bytes,
 * 256-byte aligned (the latent decode's workspace, q~ and o_lat). */
gha_status gqla_absorb_decode(const gha_tensor* q_c, const gha_tensor* q_rope, const void* w_uk,
                              const void* w_uv, const gha_tensor* c_kv, const gha_tensor* k_rope,
                              const int32_t* seqlens_k, const gha_tensor* o, float* lse,
                              int B, int h_q, int g, int s_q, int L_cap, int L_max_hint,
                              int d_h, int r_kv, int d_r, gha_dtype in_dtype, gha_dtype out_dtype,
                              float scale, void* workspace, size_t workspace_bytes, void* stream);

size_t gqla_absorb_decode_workspace_bytes(int B, int h_q, int s_q, int L_max_hint, int r_kv);

/* gqa_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments without the workspace, which comes instead from one
 * static device array of gqa_decode_noalloc_scratch_bytes() (16 MiB) per GPU,
 * held from the library's load until the process ends.  Sizes whose split
 * partials (for the kernel these cache views take) exceed it return
 * GHA_ERR_WORKSPACE and launch nothing; otherwise errors and results are
 * those of gqa_decode.  The call allocates and frees nothing.  Every call on
 * one GPU shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams or threads) race and give undefined results. */
gha_status gqa_decode_noalloc(const gha_tensor* q, const gha_tensor* k_cache,
                              const gha_tensor* v_cache, const int32_t* seqlens_k,
                              const gha_tensor* o, float* lse,
                              int B, int h_q, int h_kv, int s_q, int L_cap, int L_max_hint,
                              int d, gha_dtype in_dtype, gha_dtype out_dtype, float scale,
                              void* stream);

size_t gqa_decode_noalloc_scratch_bytes(void);

/* Status name, thread-local detail of the last error, library version. */
/* Debug checks of the decode length precondition on the device.
 *
 * Every decode entry point relies on s_q <= seqlens_k[b] <= L_cap for each
 * sequence b: the new tokens are the last s_q cached positions (bottom-right
 * alignment) and each step reads the whole cached history ("GQLA: Group-Query
 * Latent Attention ...", section 1).  The lengths live in device memory, so the
 * host validation cannot see them; without debug checks the kernels clamp a
 * length to [0, L_cap] and a row with no visible key gets zeros (lse -inf).
 *
 * With debug checks on, each decode entry point, after its host validation,
 * first launches a one-work-group kernel that tests every seqlens_k[b] on the
 * call's stream, waits for the stream, and returns GHA_ERR_PRECONDITION
 * (gha_last_error names the first failing b and its length) without
 * launching anything else when a length is out of range.  The kernel writes
 * its answer into the first 8 bytes of the call's workspace (for
 * gqa_decode_noalloc, of its scratch array).  Because the call then waits on
 * the stream, debug checks are for debugging: not for timing and not under
 * graph capture.
 *
 * gha_set_debug_checks(on) switches them on (non-zero) or off for the whole
 * process; until it is first called, they are on when the environment
 * variable GHA_DEBUG_CHECKS holds a non-zero integer.  gha_debug_checks()
 * returns 1 when they are on, else 0.  Prefill calls have no lengths and are
 * not affected. */
void gha_set_debug_checks(int on);
int gha_debug_checks(void);

const char* gha_status_string(gha_status s);
const char* gha_last_error(void);
int gha_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GHA_H_ */
