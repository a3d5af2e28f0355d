"""Seeded inputs for the GPU parity tests and the benchmark, made on the host
by ``synth`` and copied to the device.  Nothing here computes attention."""
from __future__ import annotations

import numpy as np

import oracle
import synth


def bf16_to_torch(bits: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).to(device)


# bf16 bits -> float64, for handing the kernels' exact inputs to the oracle:
# the oracle's own widening, which its pins check over every bit pattern
widen = oracle.widen_bf16


def cache_bits(B, H, L_cap, d, seqlens, seed, stream):
    return synth.cache_bf16(B, H, L_cap, d, seqlens, seed, stream)


def latent_cache_bits(B, L_cap, width, seqlens, seed, stream):
    return synth.latent_cache_bf16(B, L_cap, width, seqlens, seed, stream)


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 numbers (8 significant bits) around |x|."""
    return 0.5 * np.exp2(np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126))) - 7)


def tolerance_ok(got: np.ndarray, ref: np.ndarray, max_abs=1e-2, mean_abs=1e-3, bf16_out=False):
    """The parity bar for bf16 inputs with fp32 accumulation: every element
    within `max_abs` (1e-2) of the fp64 reference and the mean error within
    `mean_abs` (1e-3).  For bf16 outputs an element may instead be off by up
    to half a bf16 ulp of the reference (the output rounding alone reaches
    that once |o| >= 4): allowed = max(1e-2, ulp(|o_ref|) / 2).  Non-finite
    outputs always fail."""
    got = got.astype(np.float64)
    if not np.all(np.isfinite(got)):
        return False, float("inf"), float("inf")
    err = np.abs(got - ref)
    allowed = np.maximum(max_abs, bf16_half_ulp(ref)) if bf16_out else max_abs
    ok_max = bool(np.all(err <= allowed))
    mean = float(err.mean()) if err.size else 0.0
    return ok_max and mean <= mean_abs, float(err.max(initial=0.0)), mean


BF16_NAN = 0x7FC0
E4M3_NAN = 0x7F


def page_pool(cache: np.ndarray, seqlens, page_size: int, seed: int, *, window: int = 0, s_q: int = 1,
              tokens_major: bool = False):
    """Scatter a contiguous cache (B, H, L_cap, d) of bf16 bits into a shuffled
    pool of pages.  Returns (pool, block_table): pool is (n_pages, H,
    page_size, d), or (n_pages, page_size, H, d) with tokens_major; row b of
    block_table (B, ceil(L_cap / page_size)) lists the pages of sequence b.
    Page 0 of the pool is all NaN, and every table entry no query may read
    (pages past the sequence end, and with a sliding window pages wholly
    before the earliest visible key) points at it: a kernel that read such a
    page would return NaN."""
    B, H, L_cap, d = cache.shape
    n_pps = (L_cap + page_size - 1) // page_size
    rng = np.random.default_rng(seed)
    order = rng.permutation(B * n_pps) + 1            # page 0 is the NaN page
    nan = BF16_NAN if cache.dtype == np.uint16 else E4M3_NAN  # bf16 bits or E4M3 codes
    pool = np.full((B * n_pps + 1, H, page_size, d), nan, dtype=cache.dtype)
    table = np.zeros((B, n_pps), dtype=np.int32)
    padded = np.full((B, H, n_pps * page_size, d), nan, dtype=cache.dtype)
    padded[:, :, :L_cap] = cache
    for b in range(B):
        L = int(seqlens[b])
        first = max(0, L - s_q + 1 - window) if window > 0 else 0
        for p in range(n_pps):
            if p * page_size >= L or (p + 1) * page_size <= first:
                continue
            dst = order[b * n_pps + p]
            table[b, p] = dst
            pool[dst] = padded[b, :, p * page_size:(p + 1) * page_size]
    if tokens_major:
        pool = np.ascontiguousarray(pool.transpose(0, 2, 1, 3))
    return pool, table


def e4m3_codes(bits: np.ndarray, scale: float) -> np.ndarray:
    """bf16 bits -> OCP E4M3 codes of value / scale (round to nearest, clamped
    to +-448; NaN stays NaN), made with torch's float8_e4m3fn on the host."""
    import torch
    x = oracle.widen_bf16(bits) / scale
    x = np.where(np.isnan(x), np.nan, np.clip(x, -448.0, 448.0))
    return torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
