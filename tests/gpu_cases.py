"""Seeded inputs for the GPU parity tests and the benchmark, made on the host
by ``synth`` and copied to the device.  Nothing here computes attention."""
from __future__ import annotations

import numpy as np

import synth



def bf16_to_torch(bits: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).to(device)


def widen(bits: np.ndarray) -> np.ndarray:
    """bf16 bits -> float64 (for handing the same values to the oracle)."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def cache_bits(B, H, L_cap, d, seqlens, seed, stream):
    return synth.cache_bf16(B, H, L_cap, d, seqlens, seed, stream)


def latent_cache_bits(B, L_cap, width, seqlens, seed, stream):
    return synth.latent_cache_bf16(B, L_cap, width, seqlens, seed, stream)


def tolerance_ok(got: np.ndarray, ref: np.ndarray, max_abs=1e-2, mean_abs=1e-3, bf16_out=False):
    """The parity bar for bf16 inputs with fp32 accumulation: max |err| <= 1e-2
    and mean |err| <= 1e-3.  For bf16 outputs each element may also be off by
    half a bf16 ulp of the reference value (the output rounding itself)."""
    err = np.abs(got.astype(np.float64) - ref)
    if bf16_out:
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
        allowed = np.maximum(max_abs, 0.5 * ulp + 1e-3)
        ok_max = bool(np.all(err <= allowed))
    else:
        ok_max = bool(err.max(initial=0.0) <= max_abs)
    return ok_max and err.mean() <= mean_abs, float(err.max(initial=0.0)), float(err.mean())
