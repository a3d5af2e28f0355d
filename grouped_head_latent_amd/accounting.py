"""Algorithmic work and traffic of grouped-head attention.

These formulas define every TFLOP/s and GB/s figure the benchmark reports: the
work the method must do and the bytes it must move at least once, not what a
kernel happens to execute or fetch.  They also reproduce the KV-cache and
arithmetic-intensity figures the pages print, which the test suite checks.

Sources:
  * "Grouped Query Attention (GQA)", Ultralytics glossary: cached values per
    token per layer are 2 * kv_heads * head_dim (section "How GQA works",
    worked example) and the Llama 3.1 8B cache sizes (section "How GQA shrinks
    the KV cache").
  * "GQLA: Group-Query Latent Attention ...", section 1: per-token cache of
    r_kv + d^R elements on the absorbed path and 2*g*d_h + d^R on the
    per-group GQA path; the absorbed path's arithmetic intensity at
    (h_q, d_h, r_kv, d^R) = (128, 128, 512, 64) with one query token; the
    abstract's per-token cache ratio on LLaMA-3-8B.
"""
from __future__ import annotations

import numpy as np

BF16_BYTES = 2
F32_BYTES = 4

# MI355X datasheet peaks (dense; no structured-sparsity doubling).
PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2516.6
PEAK_FP32_VALU_TFLOPS = 157.3


def kv_values_per_token(kv_heads: int, head_dim: int) -> int:
    """Cached key and value elements per token per layer."""
    return 2 * kv_heads * head_dim


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int,
                       elem_bytes: int = BF16_BYTES) -> int:
    return layers * kv_values_per_token(kv_heads, head_dim) * elem_bytes


def latent_elems_per_token(r_kv: int, d_r: int) -> int:
    """Absorbed-path cache: the latent plus the shared RoPE key."""
    return r_kv + d_r


def gqla_gqa_path_elems_per_token(g: int, d_h: int, d_r: int) -> int:
    """Per-group expanded cache: g keys and g values plus the shared RoPE key."""
    return 2 * g * d_h + d_r


def absorb_intensity(h_q: int, r_kv: int, d_r: int, s_q: int = 1,
                     elem_bytes: int = BF16_BYTES) -> float:
    """FLOP per cache byte of the absorbed decode: each cached token costs a
    (r_kv + d^R)-long score dot product and an r_kv-long value update for each
    of h_q * s_q query rows, and is read once."""
    flops = 2 * h_q * s_q * ((r_kv + d_r) + r_kv)
    return flops / ((r_kv + d_r) * elem_bytes)


# ---- per-call algorithmic counts -------------------------------------------

def causal_pairs(s_q: int, s_k: int, causal: bool = True) -> int:
    """(query, key) pairs visible under bottom-right causal alignment."""
    if not causal:
        return s_q * s_k
    off = s_k - s_q
    # query t sees off + t + 1 keys
    return s_q * (off + 1) + s_q * (s_q - 1) // 2


def gqa_prefill_flops(B, h_q, S_q, S_k, d, dv=None, causal=True) -> float:
    dv = d if dv is None else dv
    return 2.0 * B * h_q * causal_pairs(S_q, S_k, causal) * (d + dv)


def gqa_prefill_bytes(B, h_q, h_kv, S_q, S_k, d, dv=None, in_bytes=BF16_BYTES,
                      out_bytes=BF16_BYTES) -> float:
    dv = d if dv is None else dv
    return float(B * (h_q * S_q * d * in_bytes + h_kv * S_k * (d + dv) * in_bytes
                      + h_q * S_q * dv * out_bytes))


def gta_prefill_flops(B, h, n_grp, S, d_qk, d_v, causal=True) -> float:
    """One score matrix per group (n_grp * d_qk per pair) and one value update
    per head (h * d_v per pair)."""
    return 2.0 * B * causal_pairs(S, S, causal) * (n_grp * d_qk + h * d_v)


def gta_prefill_bytes(B, h, n_grp, S, d_qk, d_v, in_bytes=BF16_BYTES,
                      out_bytes=BF16_BYTES) -> float:
    return float(B * S * (2 * n_grp * d_qk * in_bytes + h * d_v * in_bytes
                          + h * d_v * out_bytes))


def decode_pairs(seqlens, s_q: int) -> int:
    L = np.asarray(seqlens, dtype=np.int64)
    return int(np.sum(s_q * L - s_q * (s_q - 1) // 2))


def windowed_keys(seqlens, s_q: int, window: int) -> int:
    """Cached keys some new query sees: all L_b, or with a sliding window the
    last window + s_q - 1 of them."""
    L = np.asarray(seqlens, dtype=np.int64)
    return int(np.sum(L if window <= 0 else np.minimum(L, window + s_q - 1)))


def windowed_pairs(seqlens, s_q: int, window: int) -> int:
    """Visible (query, key) pairs of a decode step: query t of sequence b sees
    L_b - s_q + t + 1 keys, at most `window` of them with a sliding window."""
    if window <= 0:
        return decode_pairs(seqlens, s_q)
    L = np.asarray(seqlens, dtype=np.int64)
    t = np.arange(s_q, dtype=np.int64)
    return int(np.sum(np.minimum(L[:, None] - s_q + t[None, :] + 1, window)))


def gqa_decode_bytes(seqlens, h_q, h_kv, s_q, d, in_bytes=BF16_BYTES,
                     out_bytes=BF16_BYTES, window: int = 0) -> float:
    L = windowed_keys(seqlens, s_q, window)
    B = len(seqlens)
    return float(L * h_kv * 2 * d * in_bytes + B * h_q * s_q * d * (in_bytes + out_bytes))


def gqa_decode_fp8_bytes(seqlens, h_q, h_kv, s_q, d, window: int = 0) -> float:
    """As gqa_decode_bytes with one byte per cached element (bf16 queries and
    outputs)."""
    L = windowed_keys(seqlens, s_q, window)
    B = len(seqlens)
    return float(L * h_kv * 2 * d + B * h_q * s_q * d * (BF16_BYTES + BF16_BYTES))


def gqa_decode_flops(seqlens, h_q, s_q, d, window: int = 0) -> float:
    return 2.0 * h_q * windowed_pairs(seqlens, s_q, window) * (d + d)


def latent_decode_bytes(seqlens, h_q, s_q, r_kv, d_r, in_bytes=BF16_BYTES,
                        out_bytes=BF16_BYTES) -> float:
    L = int(np.sum(np.asarray(seqlens, dtype=np.int64)))
    B = len(seqlens)
    return float(L * (r_kv + d_r) * in_bytes
                 + B * s_q * h_q * ((r_kv + d_r) * in_bytes + r_kv * out_bytes))


def latent_decode_flops(seqlens, h_q, s_q, r_kv, d_r) -> float:
    return 2.0 * h_q * decode_pairs(seqlens, s_q) * ((r_kv + d_r) + r_kv)


def absorbing_decode_bytes(seqlens, h_q, g, s_q, d_h, r_kv, d_r, in_bytes=BF16_BYTES,
                           out_bytes=BF16_BYTES) -> float:
    """The latent cache read once, the content and RoPE queries, both
    up-projection blocks (g d_h x r_kv each), and the d_h-wide outputs."""
    L = int(np.sum(np.asarray(seqlens, dtype=np.int64)))
    B = len(seqlens)
    return float(L * (r_kv + d_r) * in_bytes + 2 * g * d_h * r_kv * in_bytes
                 + B * s_q * h_q * ((d_h + d_r) * in_bytes + d_h * out_bytes))


def absorbing_decode_flops(seqlens, h_q, s_q, d_h, r_kv, d_r) -> float:
    """Attention over the latent plus the two absorption products per row."""
    B = len(seqlens)
    return latent_decode_flops(seqlens, h_q, s_q, r_kv, d_r) + 2.0 * 2 * B * s_q * h_q * d_h * r_kv


def gta_decode_bytes(seqlens, h, n_grp, s_q, d_qk, d_v, in_bytes=BF16_BYTES,
                     out_bytes=BF16_BYTES) -> float:
    """Per token one key per group and one value per head, read once; plus
    the queries (one per group) and the outputs (one per head)."""
    L = int(np.sum(np.asarray(seqlens, dtype=np.int64)))
    B = len(seqlens)
    return float(L * (n_grp * d_qk + h * d_v) * in_bytes
                 + B * s_q * (n_grp * d_qk * in_bytes + h * d_v * out_bytes))


def gta_decode_flops(seqlens, h, n_grp, s_q, d_qk, d_v) -> float:
    """One score per group and visible pair, one value update per head."""
    return 2.0 * decode_pairs(seqlens, s_q) * (n_grp * d_qk + h * d_v)


def gqla_decode_bytes(seqlens, h_q, g, s_q, d_h, d_r, in_bytes=BF16_BYTES,
                      out_bytes=BF16_BYTES) -> float:
    """The per-group expanded cache, 2 g d_h + d^R elements per token, read
    once; plus queries [q^C; q^R] and outputs."""
    L = int(np.sum(np.asarray(seqlens, dtype=np.int64)))
    B = len(seqlens)
    return float(L * gqla_gqa_path_elems_per_token(g, d_h, d_r) * in_bytes
                 + B * s_q * h_q * ((d_h + d_r) * in_bytes + d_h * out_bytes))


def gqla_prefill_flops(B, h_q, S_q, S_k, d_h, d_r, causal=True) -> float:
    """Scores over the expanded key [k^C; k^R] (d_h + d^R) and values of d_h."""
    return 2.0 * B * h_q * causal_pairs(S_q, S_k, causal) * ((d_h + d_r) + d_h)


def gqla_prefill_bytes(B, h_q, g, S_q, S_k, d_h, d_r, in_bytes=BF16_BYTES,
                       out_bytes=BF16_BYTES) -> float:
    """Queries [q^C; q^R], per-group keys and values, the shared RoPE key, and
    the outputs, each moved once."""
    return float(B * (h_q * S_q * (d_h + d_r) * in_bytes + g * S_k * 2 * d_h * in_bytes
                      + S_k * d_r * in_bytes + h_q * S_q * d_h * out_bytes))


def gqla_decode_flops(seqlens, h_q, s_q, d_h, d_r) -> float:
    return 2.0 * h_q * decode_pairs(seqlens, s_q) * ((d_h + d_r) + d_h)
