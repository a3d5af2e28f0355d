"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Nothing here compares the oracle with itself under another name: each check
uses an independent route (pure-Python brute force, torch's CPU
scaled_dot_product_attention in float64, closed forms, or an equivalence the
pages state), and the planted-mistake tests at the end show that a plausible
error in the oracle fails at least one pin.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def rnd(shape, seed, stream, std=1.0):
    return oracle.widen_bf16(synth.normal_bf16(shape, seed, stream, std))


# ---------------------------------------------------------------- brute force

def brute_attention(q, k, v, scale, causal_offset=None, window=0):
    """Pure-Python loops: q (n, d), k (m, d), v (m, dv) nested lists.  Row t
    sees keys u <= t + causal_offset (None: all keys), and with window > 0
    only the last `window` of them."""
    out, lses = [], []
    for t, qt in enumerate(q):
        keys = range(len(k)) if causal_offset is None else range(min(len(k), t + causal_offset + 1))
        if window > 0:
            keys = keys[max(0, len(keys) - window):]
        scores = []
        for u in keys:
            acc = 0.0
            for c in range(len(qt)):
                acc += qt[c] * k[u][c]
            scores.append(acc * scale)
        mx = max(scores)
        w = [math.exp(s - mx) for s in scores]
        z = sum(w)
        row = [0.0] * len(v[0])
        for wi, u in zip(w, keys):
            for c in range(len(row)):
                row[c] += wi / z * v[u][c]
        out.append(row)
        lses.append(mx + math.log(z))
    return out, lses


@pytest.mark.parametrize("S,d,h_q,h_kv,causal", [(1, 1, 1, 1, True), (3, 2, 2, 1, True),
                                                  (4, 4, 4, 2, True), (4, 3, 2, 2, False)])
def test_prefill_matches_brute_force(S, d, h_q, h_kv, causal):
    q = rnd((1, h_q, S, d), 11, 1)
    k = rnd((1, h_kv, S, d), 11, 2)
    v = rnd((1, h_kv, S, d), 11, 3)
    scale = 1 / math.sqrt(d)
    o, lse = oracle.gqa_prefill(q, k, v, causal=causal)
    G = h_q // h_kv
    for i in range(h_q):
        j = i // G
        bo, bl = brute_attention(q[0, i].tolist(), k[0, j].tolist(), v[0, j].tolist(), scale,
                                 0 if causal else None)
        np.testing.assert_allclose(o[0, i], np.array(bo), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[0, i], np.array(bl), rtol=0, atol=1e-13)


def test_decode_matches_brute_force():
    B, h_q, h_kv, s_q, d, L_cap = 2, 4, 2, 2, 3, 5
    q = rnd((B, h_q, s_q, d), 12, 1)
    kc = rnd((B, h_kv, L_cap, d), 12, 2)
    vc = rnd((B, h_kv, L_cap, d), 12, 3)
    seqlens = np.array([2, 5])
    o, lse = oracle.gqa_decode(q, kc, vc, seqlens)
    for b in range(B):
        L = seqlens[b]
        for i in range(h_q):
            j = i // 2
            bo, bl = brute_attention(q[b, i].tolist(), kc[b, j, :L].tolist(), vc[b, j, :L].tolist(),
                                     1 / math.sqrt(d), causal_offset=L - s_q)
            np.testing.assert_allclose(o[b, i], bo, atol=1e-13, rtol=0)
            np.testing.assert_allclose(lse[b, i], bl, atol=1e-13, rtol=0)


@pytest.mark.parametrize("window", [1, 2, 3])
def test_windowed_decode_matches_brute_force(window):
    B, h_q, h_kv, s_q, d, L_cap = 2, 4, 2, 2, 3, 6
    q = rnd((B, h_q, s_q, d), 14, 1)
    kc = rnd((B, h_kv, L_cap, d), 14, 2)
    vc = rnd((B, h_kv, L_cap, d), 14, 3)
    seqlens = np.array([2, 6])
    o, lse = oracle.gqa_decode(q, kc, vc, seqlens, window=window)
    for b in range(B):
        L = seqlens[b]
        for i in range(h_q):
            j = i // 2
            bo, bl = brute_attention(q[b, i].tolist(), kc[b, j, :L].tolist(), vc[b, j, :L].tolist(),
                                     1 / math.sqrt(d), causal_offset=L - s_q, window=window)
            np.testing.assert_allclose(o[b, i], bo, atol=1e-13, rtol=0)
            np.testing.assert_allclose(lse[b, i], bl, atol=1e-13, rtol=0)


def test_windowed_decode_equals_decode_of_the_window():
    """A one-query decode with window W sees exactly the last W cached keys:
    it equals a plain decode over the cache cut to those keys; a window at
    least as long as the sequence changes nothing; window 1 returns the
    query's own value."""
    B, h_q, h_kv, d, L_cap, W = 3, 4, 2, 8, 40, 13
    q = rnd((B, h_q, 1, d), 15, 1)
    kc, vc = rnd((B, h_kv, L_cap, d), 15, 2), rnd((B, h_kv, L_cap, d), 15, 3)
    seqlens = np.array([40, 13, 5])
    o_w, l_w = oracle.gqa_decode(q, kc, vc, seqlens, window=W)
    for b in range(B):
        L = int(seqlens[b])
        lo = max(0, L - W)
        o_c, l_c = oracle.gqa_decode(q[b:b + 1], kc[b:b + 1, :, lo:L], vc[b:b + 1, :, lo:L], np.array([L - lo]))
        np.testing.assert_allclose(o_w[b], o_c[0], atol=1e-14)
        np.testing.assert_allclose(l_w[b], l_c[0], atol=1e-14)
    o_all, l_all = oracle.gqa_decode(q, kc, vc, seqlens)
    o_big, l_big = oracle.gqa_decode(q, kc, vc, seqlens, window=L_cap)
    np.testing.assert_array_equal(o_all, o_big)
    np.testing.assert_array_equal(l_all, l_big)
    o_1, _ = oracle.gqa_decode(q, kc, vc, seqlens, window=1)
    for b in range(B):
        L = int(seqlens[b])
        for i in range(h_q):
            np.testing.assert_array_equal(o_1[b, i, 0], vc[b, i // 2, L - 1])


def bf16_widening_matches(widen) -> bool:
    """bf16 is the top 16 bits of an IEEE-754 binary32 word (sign, 8 exponent
    bits with bias 127, 7 mantissa bits).  Checks `widen` on values the format
    fixes, then on every one of the 65,536 bit patterns against torch's
    bfloat16 -> float64, and on a strided 2-D view."""
    fixed = {0x0000: 0.0, 0x3F80: 1.0, 0x4000: 2.0, 0x3F00: 0.5, 0xBF80: -1.0, 0x3FC0: 1.5,
             0x4080: 4.0, 0x3F81: 1.0 + 2.0 ** -7, 0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126,
             0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127, 0x7F80: math.inf, 0xFF80: -math.inf}
    for bits, v in fixed.items():
        if widen(np.array([bits], dtype=np.uint16))[0] != v:
            return False
    if not np.signbit(widen(np.array([0x8000], dtype=np.uint16))[0]):
        return False
    if not np.isnan(widen(np.array([0x7FC0, 0xFFC1, 0x7F81], dtype=np.uint16))).all():
        return False
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(allbits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = widen(allbits)
    keep = ~np.isnan(ref)
    if got.dtype != np.float64 or not np.array_equal(np.isnan(got), ~keep):
        return False
    if not (np.array_equal(got[keep], ref[keep]) and np.array_equal(np.signbit(got[keep]), np.signbit(ref[keep]))):
        return False
    grid, rgrid = allbits.reshape(256, 256)[:, ::3], ref.reshape(256, 256)[:, ::3]
    g = widen(grid)
    return g.shape == grid.shape and np.array_equal(g[~np.isnan(rgrid)], rgrid[~np.isnan(rgrid)])


def test_bf16_widening_against_the_format_and_torch():
    assert bf16_widening_matches(oracle.widen_bf16)


@pytest.mark.parametrize("wrong", [
    lambda b: np.asarray(b).astype(np.float64),                                          # integer value
    lambda b: (np.asarray(b, np.uint32) << 15).view(np.float32).astype(np.float64),        # shift by 15
    lambda b: np.abs((np.asarray(b, np.uint32) << 16).view(np.float32).astype(np.float64)),  # sign dropped
    lambda b: (np.asarray(b, np.uint32) << 16).view(np.float32).astype(np.float16).astype(np.float64),  # narrowed
])
def test_planted_bf16_widening_mistakes_are_caught(wrong):
    """Plausible slips in the widening each fail the pin above."""
    assert not bf16_widening_matches(wrong)


def test_e4m3_decoder_against_the_format_and_torch():
    # values the OCP 8-bit float format fixes for E4M3
    fixed = {0x00: 0.0, 0x38: 1.0, 0x40: 2.0, 0x30: 0.5, 0x7E: 448.0, 0xFE: -448.0,
             0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x3C: 1.5, 0x81: -(2.0 ** -9)}
    for c, v in fixed.items():
        assert oracle.decode_e4m3([c])[0] == v, hex(c)
    assert np.isnan(oracle.decode_e4m3([0x7F, 0xFF])).all()
    assert np.signbit(oracle.decode_e4m3([0x80])[0])
    # every code against torch's float8_e4m3fn
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.decode_e4m3(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])


def test_fp8_decode_is_decode_of_the_dequantized_cache():
    B, h_q, h_kv, s_q, d, L_cap = 2, 4, 2, 2, 8, 30
    rng = np.random.default_rng(3)
    q = rnd((B, h_q, s_q, d), 16, 1)
    kc = rng.integers(0, 256, (B, h_kv, L_cap, d)).astype(np.uint8)
    vc = rng.integers(0, 256, (B, h_kv, L_cap, d)).astype(np.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x38  # no NaN codes
    vc[(vc & 0x7F) == 0x7F] = 0x38
    seqlens = np.array([7, 30])
    o, lse = oracle.gqa_decode_fp8(q, kc, vc, 0.01, 0.25, seqlens, window=9)
    for b in range(B):
        L = int(seqlens[b])
        for i in range(h_q):
            j = i // 2
            k = (torch.from_numpy(kc[b, j, :L].copy()).view(torch.float8_e4m3fn).to(torch.float64) * 0.01).tolist()
            v = (torch.from_numpy(vc[b, j, :L].copy()).view(torch.float8_e4m3fn).to(torch.float64) * 0.25).tolist()
            bo, bl = brute_attention(q[b, i].tolist(), k, v, 1 / math.sqrt(d), causal_offset=L - s_q, window=9)
            np.testing.assert_allclose(o[b, i], bo, atol=1e-12, rtol=1e-12)
            np.testing.assert_allclose(lse[b, i], bl, atol=1e-12, rtol=1e-12)


def test_latent_matches_brute_force():
    B, s_q, h_q, r, dr, L_cap = 1, 2, 3, 4, 2, 4
    ql = rnd((B, s_q, h_q, r), 13, 1)
    qr = rnd((B, s_q, h_q, dr), 13, 2)
    c = rnd((B, L_cap, r), 13, 3)
    kr = rnd((B, L_cap, dr), 13, 4)
    seqlens = np.array([3])
    scale = 0.3
    o, lse = oracle.latent_absorb_decode(ql, qr, c, kr, seqlens, scale=scale)
    L = 3
    for i in range(h_q):
        for t in range(s_q):
            # score written out term by term: latent part plus rope part
            scores = []
            for u in range(L - s_q + t + 1):
                s = sum(ql[0, t, i, x] * c[0, u, x] for x in range(r))
                s += sum(qr[0, t, i, x] * kr[0, u, x] for x in range(dr))
                scores.append(scale * s)
            mx = max(scores)
            w = [math.exp(s - mx) for s in scores]
            z = sum(w)
            row = [sum(w[u] / z * c[0, u, x] for u in range(len(w))) for x in range(r)]
            np.testing.assert_allclose(o[0, t, i], row, atol=1e-13, rtol=0)
            assert abs(lse[0, t, i] - (mx + math.log(z))) < 1e-13


def test_gta_matches_brute_force():
    B, n_grp, h, S, dqk, dv = 1, 2, 4, 3, 2, 3
    q = rnd((B, n_grp, S, dqk), 14, 1)
    k = rnd((B, n_grp, S, dqk), 14, 2)
    v = rnd((B, h, S, dv), 14, 3)
    o, lse = oracle.gta_prefill(q, k, v)
    for i in range(h):
        j = i // 2
        bo, bl = brute_attention(q[0, j].tolist(), k[0, j].tolist(), v[0, i].tolist(),
                                 1 / math.sqrt(dqk), 0)
        np.testing.assert_allclose(o[0, i], bo, atol=1e-13, rtol=0)
        np.testing.assert_allclose(lse[0, j], bl, atol=1e-13, rtol=0)


def test_gta_decode_matches_brute_force():
    B, n_grp, h, s_q, dqk, dv, L_cap = 2, 2, 4, 2, 3, 2, 5
    q = rnd((B, n_grp, s_q, dqk), 17, 1)
    kc = rnd((B, n_grp, L_cap, dqk), 17, 2)
    vc = rnd((B, h, L_cap, dv), 17, 3)
    seqlens = np.array([2, 5])
    o, lse = oracle.gta_decode(q, kc, vc, seqlens)
    for b in range(B):
        L = int(seqlens[b])
        for i in range(h):
            j = i // 2
            bo, bl = brute_attention(q[b, j].tolist(), kc[b, j, :L].tolist(), vc[b, i, :L].tolist(),
                                     1 / math.sqrt(dqk), causal_offset=L - s_q)
            np.testing.assert_allclose(o[b, i], bo, atol=1e-13, rtol=0)
            np.testing.assert_allclose(lse[b, j], bl, atol=1e-13, rtol=0)


def test_gqla_gqa_decode_matches_brute_force():
    """Scores written out term by term: the group's key part plus the RoPE
    part that every group shares."""
    B, h_q, g, s_q, d_h, d_r, dv, L_cap = 1, 4, 2, 2, 3, 2, 3, 5
    qc = rnd((B, h_q, s_q, d_h), 18, 1)
    qr = rnd((B, h_q, s_q, d_r), 18, 2)
    kc = rnd((B, g, L_cap, d_h), 18, 3)
    kr = rnd((B, L_cap, d_r), 18, 4)
    vc = rnd((B, g, L_cap, dv), 18, 5)
    seqlens = np.array([4])
    scale = 0.37
    o, lse = oracle.gqla_gqa_decode(qc, qr, kc, kr, vc, seqlens, scale=scale)
    L = 4
    for i in range(h_q):
        j = i // 2
        for t in range(s_q):
            scores = []
            for u in range(L - s_q + t + 1):
                sc = sum(qc[0, i, t, x] * kc[0, j, u, x] for x in range(d_h))
                sc += sum(qr[0, i, t, x] * kr[0, u, x] for x in range(d_r))
                scores.append(scale * sc)
            mx = max(scores)
            w = [math.exp(x - mx) for x in scores]
            z = sum(w)
            row = [sum(w[u] / z * vc[0, j, u, x] for u in range(len(w))) for x in range(dv)]
            np.testing.assert_allclose(o[0, i, t], row, atol=1e-13, rtol=0)
            assert abs(lse[0, i, t] - (mx + math.log(z))) < 1e-13


# ------------------------------------------------ library routine: torch SDPA

def sdpa(q, k, v, mask, scale, enable_gqa=False):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=None if mask is None else torch.from_numpy(mask),
        scale=scale, enable_gqa=enable_gqa).numpy()


@pytest.mark.parametrize("h_q,h_kv", [(8, 2), (8, 1), (8, 8), (6, 3)])
def test_prefill_matches_torch_sdpa_fp64(h_q, h_kv):
    B, S, d = 2, 37, 16
    q, k, v = rnd((B, h_q, S, d), 21, 1), rnd((B, h_kv, S, d), 21, 2), rnd((B, h_kv, S, d), 21, 3)
    o, _ = oracle.gqa_prefill(q, k, v, causal=True)
    mask = np.tril(np.ones((S, S), dtype=bool))
    ref = sdpa(q, k, v, mask, 1 / math.sqrt(d), enable_gqa=True)
    np.testing.assert_allclose(o, ref, atol=1e-12, rtol=0)


def test_decode_matches_torch_sdpa_bottom_right():
    B, h_q, h_kv, s_q, d, L_cap = 3, 4, 1, 2, 8, 40
    q = rnd((B, h_q, s_q, d), 22, 1)
    kc, vc = rnd((B, h_kv, L_cap, d), 22, 2), rnd((B, h_kv, L_cap, d), 22, 3)
    seqlens = np.array([2, 17, 40])
    o, _ = oracle.gqa_decode(q, kc, vc, seqlens)
    for b, L in enumerate(seqlens):
        mask = np.arange(L)[None, :] <= (np.arange(s_q)[:, None] + L - s_q)
        ref = sdpa(q[b:b + 1], kc[b:b + 1, :, :L], vc[b:b + 1, :, :L], mask, 1 / math.sqrt(d),
                   enable_gqa=True)
        np.testing.assert_allclose(o[b], ref[0], atol=1e-12, rtol=0)


# -------------------------------------------- the page's worked GQA example

def test_page_gqa_example_equals_repeated_heads():
    """Shapes of the worked example (seed 0 of our own generator: the page's
    values come from torch's RNG, which is not reproduced)."""
    g = GOLDEN["gqa_example_output_shape"]
    shp = g["inputs"]
    q = oracle.widen_bf16(synth.normal_bf16(shp["q"], 0, synth.STREAM["q"]))
    k = oracle.widen_bf16(synth.normal_bf16(shp["k"], 0, synth.STREAM["k"]))
    v = oracle.widen_bf16(synth.normal_bf16(shp["v"], 0, synth.STREAM["v"]))
    o, _ = oracle.gqa_prefill(q, k, v, causal=True)
    assert list(o.shape) == g["value"]
    G = shp["group_size"]
    o_mha, _ = oracle.gqa_prefill(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), causal=True)
    assert np.max(np.abs(o - o_mha)) <= GOLDEN["gqa_example_equals_repeated_heads"]["atol"]
    assert np.max(np.abs(o - o_mha)) < 1e-14


def test_single_group_is_mqa_and_full_groups_is_mha():
    B, h_q, S, d = 1, 4, 9, 8
    q = rnd((B, h_q, S, d), 23, 1)
    k1, v1 = rnd((B, 1, S, d), 23, 2), rnd((B, 1, S, d), 23, 3)
    o_mqa, _ = oracle.gqa_prefill(q, k1, v1)
    for i in range(h_q):   # MQA: every head against the one K/V head
        oi, _ = oracle.gqa_prefill(q[:, i:i + 1], k1, v1)
        np.testing.assert_array_equal(o_mqa[:, i], oi[:, 0])
    kf, vf = rnd((B, h_q, S, d), 23, 4), rnd((B, h_q, S, d), 23, 5)
    o_mha, _ = oracle.gqa_prefill(q, kf, vf)
    for i in range(h_q):   # MHA: head i against K/V head i
        oi, _ = oracle.gqa_prefill(q[:, i:i + 1], kf[:, i:i + 1], vf[:, i:i + 1])
        np.testing.assert_array_equal(o_mha[:, i], oi[:, 0])


# ---------------------------------------------------------- closed forms

def test_constant_value_rows_sum_to_one_and_lse_identity():
    B, h_q, h_kv, S, d = 2, 4, 2, 33, 16
    q, k = rnd((B, h_q, S, d), 24, 1), rnd((B, h_kv, S, d), 24, 2)
    v = np.ones((B, h_kv, S, 5))
    o, lse = oracle.gqa_prefill(q, k, v)
    np.testing.assert_allclose(o, 1.0, atol=1e-14)
    # sum_u exp(s_u - lse) = 1, with s recomputed by einsum (independent route)
    G = h_q // h_kv
    s = np.einsum("bhtc,bhuc->bhtu", q, np.repeat(k, G, axis=1)) / math.sqrt(d)
    s = np.where(np.tril(np.ones((S, S), bool)), s, -np.inf)
    np.testing.assert_allclose(np.sum(np.exp(s - lse[..., None]), axis=-1), 1.0, atol=1e-13)


def test_single_key_returns_first_value():
    q, k, v = rnd((1, 2, 5, 4), 25, 1), rnd((1, 1, 5, 4), 25, 2), rnd((1, 1, 5, 4), 25, 3)
    o, _ = oracle.gqa_prefill(q, k, v, causal=True)
    np.testing.assert_array_equal(o[0, :, 0], np.broadcast_to(v[0, 0, 0], (2, 4)))
    kc, vc = rnd((2, 1, 3, 4), 25, 4), rnd((2, 1, 3, 4), 25, 5)
    od, _ = oracle.gqa_decode(q[:, :, :1].repeat(2, 0), kc, vc, np.array([1, 1]))
    for b in range(2):
        np.testing.assert_allclose(od[b, :, 0], np.broadcast_to(vc[b, 0, 0], (2, 4)), atol=1e-15)


def test_zero_query_gives_prefix_mean():
    B, h, S, d = 1, 2, 20, 6
    q = np.zeros((B, h, S, d))
    k, v = rnd((B, h, S, d), 26, 2), rnd((B, h, S, d), 26, 3)
    o, lse = oracle.gqa_prefill(q, k, v, causal=True)
    prefix_mean = np.cumsum(v, axis=2) / np.arange(1, S + 1)[None, None, :, None]
    np.testing.assert_allclose(o, prefix_mean, atol=1e-14)
    np.testing.assert_allclose(lse, np.log(np.arange(1, S + 1))[None, None, :].repeat(h, 1), atol=1e-14)


def test_decode_is_last_rows_of_causal_prefill():
    """Bottom-right reading: a decode step over L cached tokens with s_q new
    queries equals rows L-s_q .. L-1 of causal prefill over the same L tokens."""
    B, h_q, h_kv, d, L, s_q = 1, 4, 2, 8, 23, 2
    q_full = rnd((B, h_q, L, d), 27, 1)
    k, v = rnd((B, h_kv, L, d), 27, 2), rnd((B, h_kv, L, d), 27, 3)
    o_pre, lse_pre = oracle.gqa_prefill(q_full, k, v, causal=True)
    o_dec, lse_dec = oracle.gqa_decode(q_full[:, :, L - s_q:], k, v, np.array([L]))
    np.testing.assert_allclose(o_dec, o_pre[:, :, L - s_q:], atol=1e-14)
    np.testing.assert_allclose(lse_dec, lse_pre[:, :, L - s_q:], atol=1e-14)


def test_single_query_decode_is_permutation_invariant():
    B, h_q, h_kv, d, L = 1, 4, 2, 8, 31
    q = rnd((B, h_q, 1, d), 28, 1)
    k, v = rnd((B, h_kv, L, d), 28, 2), rnd((B, h_kv, L, d), 28, 3)
    perm = np.random.default_rng(0).permutation(L)
    o1, l1 = oracle.gqa_decode(q, k, v, np.array([L]))
    o2, l2 = oracle.gqa_decode(q, k[:, :, perm], v[:, :, perm], np.array([L]))
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)


def test_lse_merges_key_splits():
    """Attention over keys [0, a) and [a, m) separately, merged with their lse,
    equals attention over all m keys (the identity a split-KV decode uses)."""
    n, m, d, a = 5, 40, 8, 17
    q, k, v = rnd((n, d), 29, 1), rnd((m, d), 29, 2), rnd((m, d), 29, 3)
    full_o, full_l = oracle.softmax_attention(q, k, v, np.full(n, m), 0.25)
    o1, l1 = oracle.softmax_attention(q, k[:a], v[:a], np.full(n, a), 0.25)
    o2, l2 = oracle.softmax_attention(q, k[a:], v[a:], np.full(n, m - a), 0.25)
    L = np.logaddexp(l1, l2)
    merged = np.exp(l1 - L)[:, None] * o1 + np.exp(l2 - L)[:, None] * o2
    np.testing.assert_allclose(merged, full_o, atol=1e-14)
    np.testing.assert_allclose(L, full_l, atol=1e-13)


# ------------------------------------------------------------------- GTA

def test_gta_equals_mha_with_shared_query_key_and_concat_value():
    """GTA article (grouped shared attention matrix): one score matrix per
    group applied to each head's V.  Equal to (a) MHA with the group's q/k
    repeated to each head and (b) one attention whose value is the group's
    heads' values concatenated."""
    B, n_grp, h, S, dqk, dv = 2, 4, 16, 29, 16, 8
    q, k = rnd((B, n_grp, S, dqk), 31, 1), rnd((B, n_grp, S, dqk), 31, 2)
    v = rnd((B, h, S, dv), 31, 3)
    o, lse = oracle.gta_prefill(q, k, v)
    per = h // n_grp
    o_mha, lse_mha = oracle.gqa_prefill(np.repeat(q, per, 1), np.repeat(k, per, 1), v)
    np.testing.assert_allclose(o, o_mha, atol=1e-14)
    np.testing.assert_allclose(lse, lse_mha[:, ::per], atol=1e-14)
    vcat = v.reshape(B, n_grp, per, S, dv).transpose(0, 1, 3, 2, 4).reshape(B, n_grp, S, per * dv)
    o_cat, _ = oracle.gqa_prefill(q, k, vcat)
    o_split = o_cat.reshape(B, n_grp, S, per, dv).transpose(0, 1, 3, 2, 4).reshape(B, h, S, dv)
    np.testing.assert_allclose(o, o_split, atol=1e-14)


# ---------------------------------------------------------------- latent

def latent_case(B=2, s_q=2, h_q=16, g=4, d_h=8, r_kv=32, d_r=4, L_cap=24, seed=41):
    q_c = rnd((B, s_q, h_q, d_h), seed, synth.STREAM["q_c"])
    q_r = rnd((B, s_q, h_q, d_r), seed, synth.STREAM["q_rope"])
    c = rnd((B, L_cap, r_kv), seed, synth.STREAM["latent"])
    kr = rnd((B, L_cap, d_r), seed, synth.STREAM["k_rope"])
    w_uk = rnd((g * d_h, r_kv), seed, synth.STREAM["w_uk"], 0.02)
    w_uv = rnd((g * d_h, r_kv), seed, synth.STREAM["w_uv"], 0.02)
    return q_c, q_r, c, kr, w_uk, w_uv


def test_absorbed_latent_equals_expanded_gqa_path():
    """GQLA Figure 2 / section 1: the absorbed MQA path and the per-group GQA
    path are algebraically equal; here both are evaluated in fp64."""
    g, d_h, d_r = 4, 8, 4
    q_c, q_r, c, kr, w_uk, w_uv = latent_case(g=g, d_h=d_h, d_r=d_r)
    B, s_q, h_q, _ = q_c.shape
    seqlens = np.array([5, 24])
    scale = 1 / math.sqrt(d_h + d_r)
    q_lat = oracle.absorb_query(q_c, w_uk, g)
    o_lat, lse_lat = oracle.latent_absorb_decode(q_lat, q_r, c, kr, seqlens, scale=scale)
    O_abs = oracle.absorb_output(o_lat, w_uv, g, d_h)
    K, V = oracle.expand_latent(c, kr, w_uk, w_uv, g)
    q_full = np.concatenate([q_c, q_r], axis=-1).transpose(0, 2, 1, 3)  # (B, h_q, s_q, d_h+d_r)
    O_exp, lse_exp = oracle.gqa_decode(q_full, K, V, seqlens, scale=scale)
    np.testing.assert_allclose(O_abs, O_exp.transpose(0, 2, 1, 3), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(lse_lat, lse_exp.transpose(0, 2, 1), rtol=0, atol=1e-12)


def test_gqla_gqa_path_equals_absorbed_latent_path():
    """GQLA Figure 2: the GQA path over the per-group expanded cache with the
    shared RoPE key (k^C_j = W^UK_j c, v_j = W^UV_j c) gives the same outputs as
    the absorbed latent path."""
    g, d_h, d_r = 4, 8, 4
    q_c, q_r, c, kr, w_uk, w_uv = latent_case(g=g, d_h=d_h, d_r=d_r)
    seqlens = np.array([5, 24])
    scale = 1 / math.sqrt(d_h + d_r)
    o_lat, lse_lat = oracle.latent_absorb_decode(oracle.absorb_query(q_c, w_uk, g), q_r, c, kr, seqlens,
                                                 scale=scale)
    O_abs = oracle.absorb_output(o_lat, w_uv, g, d_h)
    K, V = oracle.expand_latent(c, kr, w_uk, w_uv, g)
    O_gqa, lse_gqa = oracle.gqla_gqa_decode(q_c.transpose(0, 2, 1, 3), q_r.transpose(0, 2, 1, 3),
                                            K[..., :d_h], kr, V, seqlens, scale=scale)
    np.testing.assert_allclose(O_gqa.transpose(0, 2, 1, 3), O_abs, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(lse_gqa.transpose(0, 2, 1), lse_lat, rtol=0, atol=1e-12)


def test_gqla_gqa_prefill_matches_brute_force():
    B, h_q, g, S, dh, dr = 1, 4, 2, 4, 3, 2
    qc, qr = rnd((B, h_q, S, dh), 31, 1), rnd((B, h_q, S, dr), 31, 2)
    kc, kr, v = rnd((B, g, S, dh), 31, 3), rnd((B, S, dr), 31, 4), rnd((B, g, S, dh), 31, 5)
    scale = 0.37
    for causal in (True, False):
        o, lse = oracle.gqla_gqa_prefill(qc, qr, kc, kr, v, scale=scale, causal=causal)
        for i in range(h_q):
            j = i // 2
            for t in range(S):
                keys = range(t + 1) if causal else range(S)
                # the score written out: group key part plus shared RoPE part
                sc = [scale * (sum(qc[0, i, t, x] * kc[0, j, u, x] for x in range(dh))
                               + sum(qr[0, i, t, x] * kr[0, u, x] for x in range(dr))) for u in keys]
                mx = max(sc)
                w = [math.exp(z - mx) for z in sc]
                row = [sum(w[n] / sum(w) * v[0, j, u, x] for n, u in enumerate(keys)) for x in range(dh)]
                np.testing.assert_allclose(o[0, i, t], row, atol=1e-13, rtol=0)
                assert abs(lse[0, i, t] - (mx + math.log(sum(w)))) < 1e-13


def test_gqla_gqa_decode_is_last_rows_of_gqla_prefill():
    B, h_q, g, L, dh, dr, s_q = 2, 8, 2, 29, 16, 8, 3
    qc, qr = rnd((B, h_q, L, dh), 32, 1), rnd((B, h_q, L, dr), 32, 2)
    kc, kr, v = rnd((B, g, L, dh), 32, 3), rnd((B, L, dr), 32, 4), rnd((B, g, L, dh), 32, 5)
    o_p, l_p = oracle.gqla_gqa_prefill(qc, qr, kc, kr, v, scale=0.2)
    o_d, l_d = oracle.gqla_gqa_decode(qc[:, :, L - s_q:], qr[:, :, L - s_q:], kc, kr, v, np.array([L, L]), scale=0.2)
    np.testing.assert_allclose(o_d, o_p[:, :, L - s_q:], atol=1e-14)
    np.testing.assert_allclose(l_d, l_p[:, :, L - s_q:], atol=1e-14)


def test_gta_decode_is_last_rows_of_gta_prefill():
    """Bottom-right alignment: decoding the last s_q tokens of a sequence gives
    the last s_q rows of the causal shared-score prefill."""
    B, n_grp, h, L, d, s_q = 1, 2, 4, 12, 8, 3
    q, k, v = rnd((B, n_grp, L, d), 44, 1), rnd((B, n_grp, L, d), 44, 2), rnd((B, h, L, d), 44, 3)
    o_pre, lse_pre = oracle.gta_prefill(q, k, v)
    o_dec, lse_dec = oracle.gta_decode(q[:, :, L - s_q:], k, v, np.array([L]))
    np.testing.assert_allclose(o_dec, o_pre[:, :, L - s_q:], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse_dec, lse_pre[:, :, L - s_q:], rtol=0, atol=1e-14)


def test_absorb_query_uses_group_blocks():
    """q~_i = W^UK_{g(i)}^T q^C_i: written per element to pin the transpose."""
    g, d_h, r = 2, 3, 5
    w = rnd((g * d_h, r), 42, 1)
    qc = rnd((4, d_h), 42, 2)
    out = oracle.absorb_query(qc, w, g)
    for i in range(4):
        j = i // 2
        for x in range(r):
            ref = sum(w[j * d_h + a, x] * qc[i, a] for a in range(d_h))
            assert abs(out[i, x] - ref) < 1e-14


# ------------------------------------------------ planted mistakes (CPU only)

def test_planted_wrong_group_mapping_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "_group_of", lambda i, heads, groups: i % groups)
    q, k, v = rnd((1, 8, 16, 64), 0, 1), rnd((1, 2, 16, 64), 0, 2), rnd((1, 2, 16, 64), 0, 3)
    o, _ = oracle.gqa_prefill(q, k, v)
    ref = sdpa(q, k, v, np.tril(np.ones((16, 16), bool)), 1 / 8, enable_gqa=True)
    assert np.max(np.abs(o - ref)) > 1e-3


def test_planted_missing_rope_term_is_caught(monkeypatch):
    orig = oracle.softmax_attention

    def no_rope(q, k, v, nvis, scale):
        r = v.shape[1]
        return orig(q[:, :r], k[:, :r], v, nvis, scale)
    monkeypatch.setattr(oracle, "softmax_attention", no_rope)
    g, d_h, d_r = 4, 8, 4
    q_c, q_r, c, kr, w_uk, w_uv = latent_case(g=g, d_h=d_h, d_r=d_r)
    seqlens = np.array([5, 24])
    scale = 1 / math.sqrt(d_h + d_r)
    o_lat, _ = oracle.latent_absorb_decode(oracle.absorb_query(q_c, w_uk, g), q_r, c, kr, seqlens, scale=scale)
    monkeypatch.setattr(oracle, "softmax_attention", orig)
    K, V = oracle.expand_latent(c, kr, w_uk, w_uv, g)
    q_full = np.concatenate([q_c, q_r], axis=-1).transpose(0, 2, 1, 3)
    O_exp, _ = oracle.gqa_decode(q_full, K, V, seqlens, scale=scale)
    diff = oracle.absorb_output(o_lat, w_uv, g, d_h) - O_exp.transpose(0, 2, 1, 3)
    assert np.max(np.abs(diff)) > 1e-4


def test_planted_top_left_decode_alignment_is_caught():
    """A decode that aligned its causal mask top-left (as SDPA's is_causal does
    for non-square shapes) would differ from the prefill rows."""
    B, h_q, h_kv, d, L, s_q = 1, 2, 1, 8, 12, 2
    q_full = rnd((B, h_q, L, d), 43, 1)
    k, v = rnd((B, h_kv, L, d), 43, 2), rnd((B, h_kv, L, d), 43, 3)
    o_pre, _ = oracle.gqa_prefill(q_full, k, v)
    wrong = oracle.softmax_attention(q_full[0, 0, L - s_q:], k[0, 0], v[0, 0], np.arange(s_q) + 1, 1 / math.sqrt(d))[0]
    assert np.max(np.abs(wrong - o_pre[0, 0, L - s_q:])) > 1e-3


def test_row_subsets_equal_the_full_evaluation():
    """Evaluating a subset of (batch, head) rows gives exactly those rows of
    the full evaluation (rows are independent), in every decode form that
    evaluates a unit's heads together; rows outside the subset stay NaN."""
    B, h_q, h_kv, s_q, d, L_cap = 2, 8, 2, 2, 4, 9
    q = rnd((B, h_q, s_q, d), 40, 1)
    kc, vc = rnd((B, h_kv, L_cap, d), 40, 2), rnd((B, h_kv, L_cap, d), 40, 3)
    seqlens = np.array([3, 9])
    pairs = [(1, 6), (0, 1), (1, 0), (1, 7)]
    full, full_lse = oracle.gqa_decode(q, kc, vc, seqlens)
    part, part_lse = oracle.gqa_decode(q, kc, vc, seqlens, heads=pairs)
    for b, i in pairs:
        np.testing.assert_array_equal(part[b, i], full[b, i])
        np.testing.assert_array_equal(part_lse[b, i], full_lse[b, i])
    assert np.isnan(part[0, 0]).all()
    ql, qr = rnd((B, s_q, h_q, 6), 40, 4), rnd((B, s_q, h_q, 2), 40, 5)
    c, kr = rnd((B, L_cap, 6), 40, 6), rnd((B, L_cap, 2), 40, 7)
    full, full_lse = oracle.latent_absorb_decode(ql, qr, c, kr, seqlens, scale=0.4)
    part, part_lse = oracle.latent_absorb_decode(ql, qr, c, kr, seqlens, scale=0.4, heads=pairs)
    for b, i in pairs:
        np.testing.assert_allclose(part[b, :, i], full[b, :, i], rtol=0, atol=1e-15)
        np.testing.assert_allclose(part_lse[b, :, i], full_lse[b, :, i], rtol=0, atol=1e-15)
    assert np.isnan(part[0, :, 0]).all()
    qc, qrr = rnd((B, h_q, s_q, 4), 40, 8), rnd((B, h_q, s_q, 2), 40, 9)
    kcc, krr, vv = rnd((B, h_kv, L_cap, 4), 40, 10), rnd((B, L_cap, 2), 40, 11), rnd((B, h_kv, L_cap, 3), 40, 12)
    full, _ = oracle.gqla_gqa_decode(qc, qrr, kcc, krr, vv, seqlens, scale=0.4)
    part, _ = oracle.gqla_gqa_decode(qc, qrr, kcc, krr, vv, seqlens, scale=0.4, heads=pairs)
    for b, i in pairs:
        np.testing.assert_allclose(part[b, i], full[b, i], rtol=0, atol=1e-15)
