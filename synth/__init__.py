"""Seeded synthetic inputs shared by the oracle and the HIP path.

The module holds no attention arithmetic: it draws numbers and rounds them.
Every element is a pure function of (seed, stream, flat index), computed by the
counter-based SplitMix64 generator in ``synth.c`` (Steele, Lea and Flood,
OOPSLA 2014) with Box-Muller normals, so a slice of a tensor can be made
without making the rest.  Values are rounded fp64 -> fp32 (RNE) -> bf16 (RNE).

The C source is compiled with gcc into ``libsynth.so`` next to this file by
``build()``; nothing here runs on a GPU.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

# Stream ids: one per tensor role, so that tensors of one workload differ.
STREAM = {
    "q": 1, "k": 2, "v": 3, "seqlens": 4, "q_rope": 5, "latent": 6,
    "w_uk": 7, "w_uv": 8, "q_c": 9, "k_rope": 10, "extra": 11,
}


def build(force: bool = True) -> str:
    """Compile synth.c into libsynth.so (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        u64, i32 = ctypes.c_uint64, ctypes.c_int32
        lib.synth_splitmix64_at.restype = u64
        lib.synth_splitmix64_at.argtypes = [u64, u64]
        lib.synth_normal_bf16.restype = None
        lib.synth_normal_bf16.argtypes = [ctypes.c_void_p, u64, u64, u64, u64, ctypes.c_double]
        lib.synth_normal_f32.restype = None
        lib.synth_normal_f32.argtypes = [ctypes.c_void_p, u64, u64, u64, u64, ctypes.c_double]
        lib.synth_uniform_i32.restype = None
        lib.synth_uniform_i32.argtypes = [ctypes.c_void_p, u64, i32, i32, u64, u64]
        lib.synth_round_bf16.restype = None
        lib.synth_round_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, u64]
        _lib = lib
    return _lib


def splitmix64_at(seed: int, n: int) -> int:
    """n-th output of the SplitMix64 sequence seeded with `seed`."""
    return int(_load().synth_splitmix64_at(seed, n))


def normal_bf16(shape, seed: int, stream: int, stddev: float = 1.0,
                offset: int = 0) -> np.ndarray:
    """bf16 bit patterns (uint16) of stddev*N(0,1); element e of the result is
    stream element offset+e."""
    out = np.empty(shape, dtype=np.uint16)
    if out.size:
        _load().synth_normal_bf16(out.ctypes.data, offset, out.size, seed, stream, stddev)
    return out


def normal_f32(shape, seed: int, stream: int, stddev: float = 1.0,
               offset: int = 0) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    if out.size:
        _load().synth_normal_f32(out.ctypes.data, offset, out.size, seed, stream, stddev)
    return out


def uniform_i32(n: int, lo: int, hi: int, seed: int, stream: int) -> np.ndarray:
    """Integers uniform on the inclusive range [lo, hi]."""
    out = np.empty((n,), dtype=np.int32)
    if n:
        _load().synth_uniform_i32(out.ctypes.data, n, lo, hi, seed, stream)
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 values -> bf16 bit patterns (RNE)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    if x.size:
        _load().synth_round_bf16(x.ctypes.data, out.ctypes.data, x.size)
    return out


BF16_NAN = np.uint16(0x7FC0)


def normal_bf16_rows(shape, seed: int, stream: int, index, stddev: float = 1.0) -> np.ndarray:
    """Gather slices of a larger bf16 tensor of full shape `shape` without
    making all of it: `index` is a tuple of leading indices (ints), the result
    is the sub-tensor tensor[index] as bf16 bits."""
    shape = tuple(int(s) for s in shape)
    n_lead = len(index)
    inner = int(np.prod(shape[n_lead:], dtype=np.int64))
    flat = 0
    for ax, i in enumerate(index):
        flat = flat * shape[ax] + int(i)
    return normal_bf16(shape[n_lead:], seed, stream, stddev, offset=flat * inner)


def cache_bf16(B: int, H: int, L_cap: int, d: int, seqlens, seed: int, stream: int,
               stddev: float = 1.0) -> np.ndarray:
    """A contiguous (B, H, L_cap, d) bf16 KV cache of stddev*N(0,1): slots
    [0, L_b) of sequence b hold the stream's values for the full-shape tensor
    (so any slice can be regenerated alone); every slot at or beyond L_b is
    NaN, so a kernel that reads past a sequence's length poisons its output."""
    out = np.full((B, H, L_cap, d), BF16_NAN, dtype=np.uint16)
    for b in range(B):
        L = int(seqlens[b])
        for h in range(H):
            out[b, h, :L] = normal_bf16((L, d), seed, stream, stddev, offset=((b * H + h) * L_cap) * d)
    return out


def latent_cache_bf16(B: int, L_cap: int, width: int, seqlens, seed: int, stream: int) -> np.ndarray:
    """A (B, L_cap, width) bf16 latent cache, NaN beyond each sequence's length."""
    out = np.full((B, L_cap, width), BF16_NAN, dtype=np.uint16)
    for b in range(B):
        L = int(seqlens[b])
        out[b, :L] = normal_bf16((L, width), seed, stream, offset=b * L_cap * width)
    return out
