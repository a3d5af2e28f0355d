"""Plain, slow fp64 CPU oracle for grouped-head attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The HIP library never
calls it, links it or falls back to it, and it shares no code with the HIP
path: it imports nothing from ``grouped_head_latent_amd``.

Every function computes the exact definition in float64 on inputs that are
widened bit-for-bit from bf16 (or fp32).  There is no tiling, no online
softmax and no reordering: each output row is a two-pass softmax over its
visible keys followed by one weighted sum, evaluated with numpy matrix
products as the only library primitive.

Sources (the web pages the method is taken from):
  * "Grouped Query Attention (GQA)", Ultralytics glossary, section "How GQA
    works": a group of query heads shares one key head and one value head;
    inside each head the computation is unchanged scaled dot-product attention;
    one group gives MQA, as many groups as query heads gives MHA; the worked
    example uses causal masking and repeat-interleaves each key/value head to
    its consecutive group of query heads.
  * "GTA: Grouped-head latenT Attention" news article, section on the grouped
    shared attention matrix: heads are split into groups (four per group in the
    example) and a group computes its attention scores once and hands the same
    matrix to every head in the group.
  * "GQLA: Group-Query Latent Attention for Hardware-Adaptive Large Language
    Model Decoding", section 1 and section 3.1 with Eq. (1) and Figure 2: the
    latent c^KV is expanded by per-group up-projections W^UK, W^UV with g
    groups; a shared decoupled RoPE key k^R is concatenated to each group's
    key; the absorbed path folds W^UK into the query and W^UV into the output so
    all h_q heads attend straight over the cached latent, and both paths give
    the same outputs.

Readings where the pages are silent:
  * decode / chunked causal alignment is bottom-right: with L keys and s_q new
    queries, query t sees keys 0 .. L - s_q + t;
  * head i belongs to group floor(i / (heads per group)) (consecutive heads,
    as repeat_interleave in the GQA example makes them);
  * the absorbed path's scale is 1/sqrt(d_h + d^R), the scale of the expanded
    per-group key [k^C; k^R], passed explicitly by the caller;
  * the absorbed path's value is the latent c^KV alone (width r_kv); k^R is a
    key only.

Pinning: every function here is checked by ``tests/test_oracle_pins.py``
against brute force on tiny inputs, against torch's CPU scaled_dot_product_
attention in float64, against closed forms (constant V, zero Q, a single key)
and against the equivalences the pages state (GQA = MHA on repeated K/V, GTA =
MHA on repeated Q/K, absorbed latent = expanded per-group GQA).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "widen_bf16", "softmax_attention", "gqa_prefill", "gqa_decode",
    "gta_prefill", "gta_decode", "latent_absorb_decode", "gqla_gqa_decode", "gqla_gqa_prefill",
    "decode_e4m3", "gqa_decode_fp8",
    "absorb_query", "absorb_output", "expand_latent",
]


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of
    an IEEE fp32 word)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                      n_visible: np.ndarray, scale: float, first_visible=None):
    """The definition of scaled dot-product attention for a set of query rows
    that share one key/value head ("How GQA works": unchanged scaled
    dot-product attention inside each head).

    q: (n, dk) query rows; k: (m, dk); v: (m, dv); n_visible: (n,) integers,
    row r attends to keys first_visible[r] .. n_visible[r]-1 (the causal mask;
    n_visible = m means no mask; first_visible defaults to 0, a sliding window
    raises it).  Returns o (n, dv) and lse (n,) = log sum_u exp(s_u) in
    natural-log units of the scaled scores.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_visible = np.asarray(n_visible, dtype=np.int64)
    n, m = q.shape[0], k.shape[0]
    first = np.zeros(n, dtype=np.int64) if first_visible is None else np.asarray(first_visible, dtype=np.int64)
    if n == 0:
        return np.zeros((0, v.shape[1])), np.zeros((0,))
    if np.any(n_visible < 1) or np.any(n_visible > m) or np.any(first < 0) or np.any(first >= n_visible):
        raise ValueError("every query row must see between 1 and m keys")
    # step 1: scores s_u = scale * q . k_u
    s = scale * (q @ k.T)
    # causal mask: keys at or beyond n_visible[r] take no weight, nor (with a
    # sliding window) keys before first_visible[r]
    u = np.arange(m)[None, :]
    visible = (u < n_visible[:, None]) & (u >= first[:, None])
    s = np.where(visible, s, -np.inf)
    # step 2: softmax, two passes (max, then exponentials and their sum)
    mx = np.max(s, axis=1, keepdims=True)
    p = np.exp(s - mx)
    z = np.sum(p, axis=1, keepdims=True)
    # step 3: probability-weighted sum of the value rows
    o = (p / z) @ v
    lse = (mx + np.log(z))[:, 0]
    return o, lse


def _group_of(head: int, heads: int, groups: int) -> int:
    """Consecutive heads share a group: head i -> floor(i / (heads/groups))."""
    return head // (heads // groups)


def _heads_by_unit(pairs, unit_of):
    """Group the requested (b, head) pairs by the unit whose keys they read:
    {unit: [heads...]} in first-seen order.  Rows are independent, so the
    rows of one unit's heads can be evaluated in one call; the arithmetic of
    each row is unchanged."""
    units = {}
    for b, i in pairs:
        units.setdefault(unit_of(b, i), []).append(i)
    return units


def gqa_prefill(q, k, v, *, causal: bool = True, scale: float | None = None,
                heads=None):
    """Grouped-query attention ("How GQA works").

    q: (B, h_q, S_q, d); k, v: (B, h_kv, S_k, d[v]); h_q % h_kv == 0.
    Causal rows are aligned bottom-right: query t sees keys
    0 .. t + (S_k - S_q) (for S_q == S_k that is the usual u <= t).
    `heads` optionally restricts the evaluation to a list of (b, i) pairs
    (other rows of the result are left as NaN).
    Returns o (B, h_q, S_q, dv) and lse (B, h_q, S_q).
    """
    B, h_q, S_q, d = q.shape
    _, h_kv, S_k, _ = k.shape
    dv = v.shape[3]
    if h_q % h_kv:
        raise ValueError("h_q must be a multiple of h_kv")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.full((B, h_q, S_q, dv), np.nan)
    lse = np.full((B, h_q, S_q), np.nan)
    if causal:
        nvis = np.arange(S_q) + (S_k - S_q) + 1
    else:
        nvis = np.full(S_q, S_k)
    pairs = heads if heads is not None else [(b, i) for b in range(B) for i in range(h_q)]
    for b, i in pairs:
        j = _group_of(i, h_q, h_kv)
        o[b, i], lse[b, i] = softmax_attention(q[b, i], k[b, j], v[b, j], nvis, scale)
    return o, lse


def gqa_decode(q, k_cache, v_cache, seqlens, *, scale: float | None = None,
               heads=None, window: int = 0):
    """Decode step of grouped-query attention over a contiguous KV cache.

    q: (B, h_q, s_q, d); k_cache, v_cache: (B, h_kv, L_cap, d); seqlens: (B,)
    with s_q <= L_b <= L_cap.  The cache of sequence b holds L_b tokens, the
    last s_q of which are the new queries' own keys, so query t sees keys
    0 .. L_b - s_q + t.  Slots at or beyond L_b are never read.

    window > 0 is a sliding window ("GQA vs related techniques" names it as a
    complement to GQA; its extent is a reading): query t then sees only the
    last `window` of those keys, L_b - s_q + t - window + 1 .. L_b - s_q + t
    (its own key included).
    """
    B, h_q, s_q, d = q.shape
    h_kv = k_cache.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.full((B, h_q, s_q, v_cache.shape[3]), np.nan)
    lse = np.full((B, h_q, s_q), np.nan)
    pairs = heads if heads is not None else [(b, i) for b in range(B) for i in range(h_q)]
    for (b, j), hs in _heads_by_unit(pairs, lambda b, i: (b, _group_of(i, h_q, h_kv))).items():
        L = int(seqlens[b])
        if not (s_q <= L <= k_cache.shape[2]):
            raise ValueError("need s_q <= L_b <= L_cap")
        # rows (head, t) of the group's requested heads over the group's keys
        nvis = np.tile(np.arange(s_q) + (L - s_q) + 1, len(hs))
        first = np.maximum(nvis - window, 0) if window > 0 else None
        ob, lb = softmax_attention(q[b, hs].reshape(len(hs) * s_q, d), k_cache[b, j, :L],
                                   v_cache[b, j, :L], nvis, scale, first)
        o[b, hs] = ob.reshape(len(hs), s_q, -1)
        lse[b, hs] = lb.reshape(len(hs), s_q)
    return o, lse


def decode_e4m3(codes) -> np.ndarray:
    """8-bit floating point codes, E4M3 as in the OCP 8-bit floating point
    format (the quantized KV storage that the GQLA page's section 2 names as
    complementary; the format is a reading): sign bit, 4-bit exponent with
    bias 7, 3-bit mantissa; exponent 0 holds subnormals m/8 * 2^-6; the code
    S.1111.111 is NaN and there are no infinities.  Returns float64."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 15
    m = (b & 7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (m / 8.0) * 2.0 ** -6
    v = sign * np.where(e == 0, subnormal, normal)
    return np.where((e == 15) & ((b & 7) == 7), np.nan, v)


def gqa_decode_fp8(q, k_codes, v_codes, k_scale: float, v_scale: float, seqlens, *,
                   scale: float | None = None, heads=None, window: int = 0):
    """GQA decode over an 8-bit cache: key u is decode_e4m3(k_codes[u]) * k_scale
    and value u is decode_e4m3(v_codes[u]) * v_scale (one scale per tensor, a
    reading); otherwise exactly gqa_decode."""
    return gqa_decode(q, decode_e4m3(k_codes) * k_scale, decode_e4m3(v_codes) * v_scale, seqlens,
                      scale=scale, heads=heads, window=window)


def gta_prefill(q, k, v, *, causal: bool = True, scale: float | None = None,
                heads=None):
    """GTA shared-score attention (GTA article, grouped shared attention
    matrix): each group has one query/key projection, so one score matrix per
    group, computed once and applied to the value of every head in the group.

    q, k: (B, n_grp, S, d_qk); v: (B, h, S, d_v); h % n_grp == 0.
    Returns o (B, h, S, d_v) and lse (B, n_grp, S) (one per shared matrix).
    """
    B, n_grp, S, d_qk = q.shape
    h = v.shape[1]
    if h % n_grp:
        raise ValueError("h must be a multiple of n_grp")
    if scale is None:
        scale = 1.0 / np.sqrt(d_qk)
    nvis = np.arange(S) + 1 if causal else np.full(S, S)
    o = np.full((B, h, S, v.shape[3]), np.nan)
    lse = np.full((B, n_grp, S), np.nan)
    pairs = heads if heads is not None else [(b, i) for b in range(B) for i in range(h)]
    for b, i in pairs:
        j = _group_of(i, h, n_grp)
        o[b, i], lse[b, j] = softmax_attention(q[b, j], k[b, j], v[b, i], nvis, scale)
    return o, lse


def gta_decode(q, k_cache, v_cache, seqlens, *, scale: float | None = None,
               heads=None):
    """Decode step of GTA shared-score attention (GTA article, grouped shared
    attention matrix) over a contiguous cache: each group has one query and
    one cached key per token, so one score vector per new token, and every
    head of the group applies it to its own cached values.

    q: (B, n_grp, s_q, d_qk); k_cache: (B, n_grp, L_cap, d_qk);
    v_cache: (B, h, L_cap, d_v); seqlens: (B,) with s_q <= L_b <= L_cap,
    counting the new tokens, aligned bottom-right as in gqa_decode.
    Returns o (B, h, s_q, d_v) and lse (B, n_grp, s_q).
    """
    B, n_grp, s_q, d_qk = q.shape
    h = v_cache.shape[1]
    if h % n_grp:
        raise ValueError("h must be a multiple of n_grp")
    if scale is None:
        scale = 1.0 / np.sqrt(d_qk)
    o = np.full((B, h, s_q, v_cache.shape[3]), np.nan)
    lse = np.full((B, n_grp, s_q), np.nan)
    pairs = heads if heads is not None else [(b, i) for b in range(B) for i in range(h)]
    for b, i in pairs:
        L = int(seqlens[b])
        if not (s_q <= L <= k_cache.shape[2]):
            raise ValueError("need s_q <= L_b <= L_cap")
        j = _group_of(i, h, n_grp)
        nvis = np.arange(s_q) + (L - s_q) + 1
        o[b, i], lse[b, j] = softmax_attention(q[b, j], k_cache[b, j, :L], v_cache[b, i, :L],
                                               nvis, scale)
    return o, lse


def gqla_gqa_decode(q_c, q_r, k_c, k_r, v_cache, seqlens, *, scale: float,
                    heads=None):
    """GQLA's GQA-path decode (section 1 and section 3.1, Eq. (1)): g groups,
    each with its own cached key k^C and value, plus one decoupled RoPE key
    k^R per token shared by every group.  Head i of group j = g(i) scores
        scale * (q^C_i . k^C_{j,u} + q^R_i . k^R_u),
    the dot product of [q^C_i; q^R_i] with the group's key [k^C_j; k^R], and
    takes the group's value v_{j,u}.

    q_c: (B, h_q, s_q, d_h); q_r: (B, h_q, s_q, d_r); k_c: (B, g, L_cap, d_h);
    k_r: (B, L_cap, d_r); v_cache: (B, g, L_cap, d_v); seqlens as gqa_decode.
    Returns o (B, h_q, s_q, d_v) and lse (B, h_q, s_q).
    """
    B, h_q, s_q, _ = q_c.shape
    g = k_c.shape[1]
    if h_q % g:
        raise ValueError("h_q must be a multiple of g")
    o = np.full((B, h_q, s_q, v_cache.shape[3]), np.nan)
    lse = np.full((B, h_q, s_q), np.nan)
    pairs = heads if heads is not None else [(b, i) for b in range(B) for i in range(h_q)]
    for (b, j), hs in _heads_by_unit(pairs, lambda b, i: (b, _group_of(i, h_q, g))).items():
        L = int(seqlens[b])
        if not (s_q <= L <= k_c.shape[2]):
            raise ValueError("need s_q <= L_b <= L_cap")
        # rows (head, t): query [q^C_i; q^R_i]; keys [k^C_j; k^R] of the group
        qi = np.concatenate([q_c[b, hs], q_r[b, hs]], axis=2).reshape(len(hs) * s_q, -1)
        kj = np.concatenate([k_c[b, j, :L], k_r[b, :L]], axis=1)
        nvis = np.tile(np.arange(s_q) + (L - s_q) + 1, len(hs))
        ob, lb = softmax_attention(qi, kj, v_cache[b, j, :L], nvis, scale)
        o[b, hs] = ob.reshape(len(hs), s_q, -1)
        lse[b, hs] = lb.reshape(len(hs), s_q)
    return o, lse


def gqla_gqa_prefill(q_c, q_r, k_c, k_r, v, *, scale: float, causal: bool = True,
                     heads=None):
    """GQLA's GQA path over a whole sequence, the compute-friendly form for
    prefill (section 1; Eq. (1) of section 3.1 expands the latent into per-
    group keys and values, with one decoupled RoPE key shared by the groups).
    Head i of group j = g(i) attends with query [q^C_i; q^R_i] over keys
    [k^C_j; k^R] (width d_h + d^R) and values v_j.

    q_c: (B, h_q, S_q, d_h); q_r: (B, h_q, S_q, d_r); k_c: (B, g, S_k, d_h);
    k_r: (B, S_k, d_r); v: (B, g, S_k, d_v).  Causal alignment is bottom-right
    (query t sees keys 0 .. S_k - S_q + t).  Returns o (B, h_q, S_q, d_v) and
    lse (B, h_q, S_q).
    """
    B, h_q, S_q, _ = q_c.shape
    g, S_k = k_c.shape[1], k_c.shape[2]
    if h_q % g:
        raise ValueError("h_q must be a multiple of g")
    if causal and S_q > S_k:
        raise ValueError("causal needs S_q <= S_k")
    o = np.full((B, h_q, S_q, v.shape[3]), np.nan)
    lse = np.full((B, h_q, S_q), np.nan)
    nvis = np.arange(S_q) + (S_k - S_q) + 1 if causal else np.full(S_q, S_k)
    pairs = heads if heads is not None else [(b, i) for b in range(B) for i in range(h_q)]
    for (b, j), hs in _heads_by_unit(pairs, lambda b, i: (b, _group_of(i, h_q, g))).items():
        kj = np.concatenate([k_c[b, j], k_r[b]], axis=1)   # the group's key [k^C_j; k^R]
        for i in hs:
            qi = np.concatenate([q_c[b, i], q_r[b, i]], axis=1)
            o[b, i], lse[b, i] = softmax_attention(qi, kj, v[b, j], nvis, scale)
    return o, lse


def latent_absorb_decode(q_lat, q_rope, c_kv, k_rope, seqlens, *, scale: float,
                         heads=None):
    """MQA-absorbed latent decode (GQLA section 1 and Figure 2, right): every
    query head attends directly over the cached latent.

    The score of head i with token u is
        scale * (q_lat[i] . c_u + q_rope[i] . k_rope_u),
    i.e. a dot product of the concatenations [q_lat; q_rope] and [c_u; k^R_u]
    (the expanded key [W^UK c; k^R] of Eq. (1) with W^UK moved onto the
    query), and the value is the latent c_u itself.

    q_lat: (B, s_q, h_q, r_kv); q_rope: (B, s_q, h_q, d_r);
    c_kv: (B, L_cap, r_kv); k_rope: (B, L_cap, d_r); seqlens: (B,).
    Returns o_lat (B, s_q, h_q, r_kv) and lse (B, s_q, h_q).
    """
    B, s_q, h_q, r_kv = q_lat.shape
    o = np.full((B, s_q, h_q, r_kv), np.nan)
    lse = np.full((B, s_q, h_q), np.nan)
    pairs = heads if heads is not None else [(b, i) for b in range(B) for i in range(h_q)]
    for b, hs in _heads_by_unit(pairs, lambda b, i: b).items():
        L = int(seqlens[b])
        if not (s_q <= L <= c_kv.shape[1]):
            raise ValueError("need s_q <= L_b <= L_cap")
        # rows (t, head) of every requested head over the one shared cache
        qi = np.concatenate([q_lat[b][:, hs], q_rope[b][:, hs]], axis=2).reshape(s_q * len(hs), -1)
        kb = np.concatenate([c_kv[b, :L], k_rope[b, :L]], axis=1)
        nvis = np.repeat(np.arange(s_q) + (L - s_q) + 1, len(hs))
        ob, lb = softmax_attention(qi, kb, c_kv[b, :L], nvis, scale)
        o[b][:, hs] = ob.reshape(s_q, len(hs), -1)
        lse[b][:, hs] = lb.reshape(s_q, len(hs))
    return o, lse


def absorb_query(q_c, w_uk, g: int):
    """Fold W^UK into the query (GQLA Figure 2, right): for head i in group
    j = g(i), q~_i = (W^UK_j)^T q^C_i, where W^UK (g*d_h, r_kv) stacks the
    groups' (d_h, r_kv) blocks as in Eq. (1).

    q_c: (..., h_q, d_h) -> (..., h_q, r_kv).
    """
    h_q, d_h = q_c.shape[-2], q_c.shape[-1]
    out = np.empty(q_c.shape[:-1] + (w_uk.shape[1],))
    for i in range(h_q):
        j = _group_of(i, h_q, g)
        w = w_uk[j * d_h:(j + 1) * d_h]            # (d_h, r_kv)
        out[..., i, :] = q_c[..., i, :] @ w
    return out


def absorb_output(o_lat, w_uv, g: int, d_h: int):
    """Apply W^UV after attention (GQLA Figure 2, right): O_i = W^UV_j o_lat_i.

    o_lat: (..., h_q, r_kv) -> (..., h_q, d_h).
    """
    h_q = o_lat.shape[-2]
    out = np.empty(o_lat.shape[:-1] + (d_h,))
    for i in range(h_q):
        j = _group_of(i, h_q, g)
        w = w_uv[j * d_h:(j + 1) * d_h]            # (d_h, r_kv)
        out[..., i, :] = o_lat[..., i, :] @ w.T
    return out


def expand_latent(c_kv, k_rope, w_uk, w_uv, g: int):
    """The per-group expanded cache of GQLA's GQA path (section 3.1): for
    group j, K_j = [c W^UK_j^T ; k^R] (width d_h + d^R) and V_j = c W^UV_j^T
    (width d_h), from Eq. (1) (k^C = W^UK c, shared k^R concatenated).

    c_kv: (B, L, r_kv); k_rope: (B, L, d_r) -> K (B, g, L, d_h+d_r),
    V (B, g, L, d_h).
    """
    d_h = w_uk.shape[0] // g
    B, L, _ = c_kv.shape
    K = np.empty((B, g, L, d_h + k_rope.shape[2]))
    V = np.empty((B, g, L, d_h))
    for j in range(g):
        K[:, j, :, :d_h] = c_kv @ w_uk[j * d_h:(j + 1) * d_h].T
        K[:, j, :, d_h:] = k_rope
        V[:, j] = c_kv @ w_uv[j * d_h:(j + 1) * d_h].T
    return K, V
