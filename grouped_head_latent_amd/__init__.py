"""Grouped-head attention for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libgha.so``, whose C ABI is declared in
``include/gha.h``.  The functions below only marshal arguments: they turn
torch tensors (device memory) into pointer-and-stride descriptors, allocate
outputs and workspaces with torch when the caller does not pass them, and call
the library on torch's current stream.  Every step of the computation runs in
the library's HIP kernels; there is no fallback of any kind.  If the library
is missing or cannot be loaded, every call raises.

Entry points (same names as the C ABI):
  gqa_prefill, gqa_decode, gqa_decode_paged, gqa_decode_fp8,
  gta_shared_score_prefill, gta_shared_score_decode, gqla_gqa_decode,
  gqla_gqa_prefill, latent_absorb_decode, gqla_absorb_decode, and the
  *_workspace_bytes queries of the decode calls; set_debug_checks and
  debug_checks switch the device-side check of the decode lengths.  Every
  wrapper checks, before the library is called, that all tensors sit on the
  query's GPU and carry the dtypes the call expects.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "gqa_prefill", "gqa_decode", "gqa_decode_paged", "gqa_decode_fp8", "gta_shared_score_prefill", "gta_shared_score_decode",
    "gqla_gqa_decode", "gqla_gqa_prefill", "latent_absorb_decode", "gqla_absorb_decode",
    "gqa_decode_noalloc", "gqa_decode_noalloc_scratch_bytes",
    "gqa_decode_workspace_bytes", "gqa_decode_paged_workspace_bytes", "gta_shared_score_decode_workspace_bytes",
    "gqla_gqa_decode_workspace_bytes", "latent_absorb_decode_workspace_bytes",
    "set_debug_checks", "debug_checks",
    "GhaError", "library_path", "load_library", "GHA_F32", "GHA_BF16",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgha.so")

GHA_F32, GHA_BF16 = 0, 1
STATUS = ["GHA_OK", "GHA_ERR_NULL", "GHA_ERR_SHAPE", "GHA_ERR_GROUPING", "GHA_ERR_STRIDE",
          "GHA_ERR_ALIGN", "GHA_ERR_DTYPE", "GHA_ERR_HEAD_DIM", "GHA_ERR_WORKSPACE", "GHA_ERR_HIP",
          "GHA_ERR_PRECONDITION"]


class GhaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        name = STATUS[status] if 0 <= status < len(STATUS) else str(status)
        super().__init__(f"{name}: {detail}")


class GhaTensor(ctypes.Structure):
    """gha_tensor: device pointer plus batch/head/token element strides."""
    _fields_ = [("ptr", ctypes.c_void_p), ("sb", ctypes.c_int64),
                ("sh", ctypes.c_int64), ("ss", ctypes.c_int64)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libgha.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m grouped_head_latent_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, F, S, V = ctypes.POINTER(GhaTensor), ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
    lib.gqa_prefill.argtypes = [P, P, P, P, V, I, I, I, I, I, I, I, I, F, I, V]
    lib.gqa_prefill.restype = I
    lib.gqa_decode.argtypes = [P, P, P, V, P, V, I, I, I, I, I, I, I, I, I, F, V, S, V]
    lib.gqa_decode.restype = I
    lib.gqa_decode_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.gqa_decode_workspace_bytes.restype = S
    lib.gqa_decode_paged.argtypes = [P, P, P, V, I, I, V, P, V, I, I, I, I, I, I, I, I, I, I, F, V, S, V]
    lib.gqa_decode_paged.restype = I
    lib.gqa_decode_paged_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.gqa_decode_paged_workspace_bytes.restype = S
    lib.gqa_decode_fp8.argtypes = [P, P, P, F, F, V, I, I, V, P, V, I, I, I, I, I, I, I, I, I, F, V, S, V]
    lib.gqa_decode_fp8.restype = I
    lib.gta_shared_score_prefill.argtypes = [P, P, P, P, V, I, I, I, I, I, I, I, I, F, I, V]
    lib.gta_shared_score_prefill.restype = I
    lib.gta_shared_score_decode.argtypes = [P, P, P, V, P, V, I, I, I, I, I, I, I, I, I, I, F, V, S, V]
    lib.gta_shared_score_decode.restype = I
    lib.gta_shared_score_decode_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.gta_shared_score_decode_workspace_bytes.restype = S
    lib.gqla_gqa_decode.argtypes = [P, P, P, P, P, V, P, V, I, I, I, I, I, I, I, I, I, I, F, V, S, V]
    lib.gqla_gqa_decode.restype = I
    lib.gqla_gqa_decode_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.gqla_gqa_decode_workspace_bytes.restype = S
    lib.gqla_gqa_prefill.argtypes = [P, P, P, P, P, P, V, I, I, I, I, I, I, I, I, I, F, I, V]
    lib.gqla_gqa_prefill.restype = I
    lib.latent_absorb_decode.argtypes = [P, P, P, P, V, P, V, I, I, I, I, I, I, I, I, I, F, V, S, V]
    lib.latent_absorb_decode.restype = I
    lib.latent_absorb_decode_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.latent_absorb_decode_workspace_bytes.restype = S
    lib.gqla_absorb_decode.argtypes = [P, P, V, V, P, P, V, P, V, I, I, I, I, I, I, I, I, I, I, I, F, V, S, V]
    lib.gqla_absorb_decode.restype = I
    lib.gqla_absorb_decode_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.gqla_absorb_decode_workspace_bytes.restype = S
    lib.gqa_decode_noalloc.argtypes = [P, P, P, V, P, V, I, I, I, I, I, I, I, I, I, F, V]
    lib.gqa_decode_noalloc.restype = I
    lib.gqa_decode_noalloc_scratch_bytes.argtypes = []
    lib.gqa_decode_noalloc_scratch_bytes.restype = S
    lib.gha_status_string.argtypes = [I]
    lib.gha_status_string.restype = ctypes.c_char_p
    lib.gha_last_error.argtypes = []
    lib.gha_last_error.restype = ctypes.c_char_p
    lib.gha_version.argtypes = []
    lib.gha_version.restype = I
    lib.gha_set_debug_checks.argtypes = [I]
    lib.gha_set_debug_checks.restype = None
    lib.gha_debug_checks.argtypes = []
    lib.gha_debug_checks.restype = I
    _lib = lib
    return lib


def set_debug_checks(on: bool) -> None:
    """Switch the device-side check s_q <= seqlens_k[b] <= L_cap of every
    decode call on or off, for the whole process (gha_set_debug_checks).
    With it on, a decode call waits for the check and raises GhaError
    (GHA_ERR_PRECONDITION) before anything else runs on a bad length."""
    load_library().gha_set_debug_checks(1 if on else 0)


def debug_checks() -> bool:
    """Whether the device-side length checks are on (gha_debug_checks)."""
    return bool(load_library().gha_debug_checks())


def _check(status: int):
    if status != 0:
        raise GhaError(status, _lib.gha_last_error().decode())


# ---------------------------------------------------------------- marshalling

def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return GHA_BF16
    if t.dtype == torch.float32:
        return GHA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _desc(t, axes=(0, 1, 2)) -> GhaTensor:
    """Descriptor of a 4-D (or, with axes, 3-D) tensor with a contiguous last
    axis; `axes` names the tensor axes that are batch, head and token (None
    for an absent axis, stride 0)."""
    if t.stride(-1) != 1:
        raise ValueError("the last axis must be contiguous")
    st = [0 if a is None else t.stride(a) for a in axes]
    return GhaTensor(t.data_ptr(), st[0], st[1], st[2])


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _out_code(out_dtype):
    import torch
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"outputs are bf16 or fp32, not {out_dtype}")
    return GHA_F32 if out_dtype == torch.float32 else GHA_BF16


def _same_device(ref, **tensors):
    """Every given tensor must live on `ref`'s GPU: a host tensor or one on
    another device would hand the kernels a pointer they cannot read."""
    if not ref.is_cuda:
        raise ValueError("inputs must be GPU tensors")
    for name, t in tensors.items():
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, not on {ref.device} with the query")


def _need_dtype(allowed, **tensors):
    """Each given tensor must have one of the `allowed` dtypes."""
    for name, t in tensors.items():
        if t is not None and t.dtype not in allowed:
            raise TypeError(f"{name} has dtype {t.dtype}; expected one of {allowed}")


def _need_same_dtype(ref_name, ref, **tensors):
    for name, t in tensors.items():
        if t.dtype != ref.dtype:
            raise TypeError(f"{name} has dtype {t.dtype} but {ref_name} has {ref.dtype}")


def _check_common(q, q_name, *, inputs, seqlens=None, extra=None, out=None, out_dtype=None, workspace=None):
    """The checks every wrapper makes before calling the library: all tensors
    on q's GPU, inputs of q's dtype (bf16), int32 lengths, bf16 or fp32
    outputs, a byte workspace."""
    import torch
    _need_same_dtype(q_name, q, **inputs)
    if seqlens is not None and seqlens.dtype != torch.int32:
        raise TypeError("seqlens must be int32")
    _need_dtype((torch.bfloat16, torch.float32), out=out)
    if out_dtype is not None:
        _out_code(out_dtype)
    _need_dtype((torch.int32,), **{k: t for k, t in (extra or {}).items() if k == "block_table"})
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    _same_device(q, **inputs, **(extra or {}), seqlens=seqlens, out=out, workspace=workspace)


# ------------------------------------------------------------------ wrappers

def gqa_prefill(q, k, v, *, causal: bool = True, scale: float | None = None, out=None,
                out_dtype=None, return_lse: bool = False, stream=None):
    """q (B, h_q, S_q, d), k/v (B, h_kv, S_k, d) device tensors (bf16, or fp32
    for the fp32 path).  Returns o (B, h_q, S_q, d) [and lse (B, h_q, S_q)]."""
    import torch
    lib = load_library()
    _need_dtype((torch.bfloat16, torch.float32), q=q)
    _check_common(q, "q", inputs=dict(k=k, v=v), out=out, out_dtype=out_dtype)
    B, h_q, S_q, d = q.shape
    h_kv, S_k = k.shape[1], k.shape[2]
    out_dtype = out_dtype or (torch.float32 if q.dtype == torch.float32 else torch.bfloat16)
    o = out if out is not None else torch.empty((B, h_q, S_q, d), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, h_q, S_q), dtype=torch.float32, device=q.device) if return_lse else None
    _check(lib.gqa_prefill(_desc(q), _desc(k), _desc(v), _desc(o), _ptr(lse), B, h_q, h_kv, S_q,
                           S_k, d, _dtype_code(q), _out_code(o.dtype), float(scale or 0.0),
                           int(bool(causal)), _stream(stream)))
    return (o, lse) if return_lse else o


def gqa_decode_workspace_bytes(B, h_q, h_kv, s_q, L_max, d) -> int:
    return int(load_library().gqa_decode_workspace_bytes(B, h_q, h_kv, s_q, L_max, d))


def gqa_decode(q, k_cache, v_cache, seqlens, *, L_max: int | None = None,
               scale: float | None = None, out=None, out_dtype=None, workspace=None,
               return_lse: bool = False, stream=None):
    """q (B, h_q, s_q, d); caches (B, h_kv, L_cap, d); seqlens int32 device (B,).
    L_max: an upper bound on the lengths (default L_cap)."""
    import torch
    lib = load_library()
    _need_dtype((torch.bfloat16,), q=q)
    _check_common(q, "q", inputs=dict(k_cache=k_cache, v_cache=v_cache), seqlens=seqlens, out=out, out_dtype=out_dtype,
                  workspace=workspace)
    B, h_q, s_q, d = q.shape
    h_kv, L_cap = k_cache.shape[1], k_cache.shape[2]
    L_max = L_cap if L_max is None else int(L_max)
    out_dtype = out_dtype or torch.bfloat16
    o = out if out is not None else torch.empty((B, h_q, s_q, d), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, h_q, s_q), dtype=torch.float32, device=q.device) if return_lse else None
    need = gqa_decode_workspace_bytes(B, h_q, h_kv, s_q, L_max, d)
    ws = workspace if workspace is not None else torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check(lib.gqa_decode(_desc(q), _desc(k_cache), _desc(v_cache), _ptr(seqlens), _desc(o),
                          _ptr(lse), B, h_q, h_kv, s_q, L_cap, L_max, d, _dtype_code(q),
                          _out_code(o.dtype), float(scale or 0.0), _ptr(ws), ws.numel() * ws.element_size(),
                          _stream(stream)))
    return (o, lse) if return_lse else o


def gqa_decode_noalloc(q, k_cache, v_cache, seqlens, *, out, L_max: int | None = None,
                       scale: float | None = None, lse=None, stream=None):
    """gqa_decode with its workspace in the library's static per-GPU scratch
    array: allocates nothing, so `out` (and `lse`, if wanted) must be given.
    q (B, h_q, s_q, d); caches (B, h_kv, L_cap, d); seqlens int32 device (B,).
    Calls on one GPU that overlap in time race on the shared scratch."""
    import torch
    lib = load_library()
    _need_dtype((torch.bfloat16,), q=q)
    _check_common(q, "q", inputs=dict(k_cache=k_cache, v_cache=v_cache), seqlens=seqlens, out=out,
                  extra=dict(lse=lse))
    _need_dtype((torch.float32,), lse=lse)
    B, h_q, s_q, d = q.shape
    h_kv, L_cap = k_cache.shape[1], k_cache.shape[2]
    L_max = L_cap if L_max is None else int(L_max)
    _check(lib.gqa_decode_noalloc(_desc(q), _desc(k_cache), _desc(v_cache), _ptr(seqlens), _desc(out), _ptr(lse),
                                  B, h_q, h_kv, s_q, L_cap, L_max, d, _dtype_code(q), _out_code(out.dtype),
                                  float(scale or 0.0), _stream(stream)))
    return out


def gqa_decode_noalloc_scratch_bytes() -> int:
    return int(load_library().gqa_decode_noalloc_scratch_bytes())


def gqa_decode_paged_workspace_bytes(B, h_q, h_kv, s_q, L_max, window, d) -> int:
    return int(load_library().gqa_decode_paged_workspace_bytes(B, h_q, h_kv, s_q, L_max, window, d))


def gqa_decode_paged(q, k_cache, v_cache, seqlens, *, block_table=None, page_size: int = 0,
                     L_cap: int | None = None, L_max: int | None = None, window: int = 0,
                     scale: float | None = None, out=None, out_dtype=None, workspace=None,
                     return_lse: bool = False, stream=None):
    """q (B, h_q, s_q, d); seqlens int32 device (B,).
    block_table None: caches (B, h_kv, L_cap, d).  Otherwise block_table int32
    device (B, pages per sequence) and caches are page pools viewed as
    (n_pages, h_kv, page_size, d).  window > 0: sliding window of that many
    keys.  L_cap: longest sequence the cache holds (default: the cache's
    length, or pages per sequence times page_size); L_max: an upper bound on
    the lengths (default L_cap)."""
    import torch
    lib = load_library()
    _need_dtype((torch.bfloat16,), q=q)
    _check_common(q, "q", inputs=dict(k_cache=k_cache, v_cache=v_cache), seqlens=seqlens, out=out, out_dtype=out_dtype,
                  workspace=workspace, extra=dict(block_table=block_table))
    B, h_q, s_q, d = q.shape
    h_kv = k_cache.shape[1]
    if block_table is None:
        bt_stride, page_size = 0, 0
        L_cap = k_cache.shape[2] if L_cap is None else int(L_cap)
    else:
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(1) != 1:
            raise TypeError("block_table must be an int32 (B, pages) tensor with contiguous rows")
        page_size = int(page_size or k_cache.shape[2])
        bt_stride = block_table.stride(0)
        L_cap = block_table.shape[1] * page_size if L_cap is None else int(L_cap)
    L_max = L_cap if L_max is None else int(L_max)
    out_dtype = out_dtype or torch.bfloat16
    o = out if out is not None else torch.empty((B, h_q, s_q, d), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, h_q, s_q), dtype=torch.float32, device=q.device) if return_lse else None
    need = gqa_decode_paged_workspace_bytes(B, h_q, h_kv, s_q, L_max, int(window), d)
    ws = workspace if workspace is not None else torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check(lib.gqa_decode_paged(_desc(q), _desc(k_cache), _desc(v_cache), _ptr(block_table), bt_stride,
                                page_size, _ptr(seqlens), _desc(o), _ptr(lse), B, h_q, h_kv, s_q, L_cap,
                                L_max, int(window), d, _dtype_code(q), _out_code(o.dtype),
                                float(scale or 0.0), _ptr(ws), ws.numel() * ws.element_size(),
                                _stream(stream)))
    return (o, lse) if return_lse else o


def gqa_decode_fp8(q, k_codes, v_codes, seqlens, *, k_scale: float, v_scale: float, block_table=None,
                   page_size: int = 0, L_cap: int | None = None, L_max: int | None = None, window: int = 0,
                   scale: float | None = None, out=None, out_dtype=None, workspace=None,
                   return_lse: bool = False, stream=None):
    """gqa_decode_paged over caches of OCP E4M3 codes (uint8 tensors of the
    same shapes as the bf16 caches); key = code * k_scale, value = code *
    v_scale."""
    import torch
    lib = load_library()
    if k_codes.dtype != torch.uint8 or v_codes.dtype != torch.uint8:
        raise TypeError("the caches hold uint8 E4M3 codes")
    _need_dtype((torch.bfloat16,), q=q)
    _check_common(q, "q", inputs={}, seqlens=seqlens, out=out, out_dtype=out_dtype, workspace=workspace,
                  extra=dict(k_codes=k_codes, v_codes=v_codes, block_table=block_table))
    B, h_q, s_q, d = q.shape
    h_kv = k_codes.shape[1]
    if block_table is None:
        bt_stride, page_size = 0, 0
        L_cap = k_codes.shape[2] if L_cap is None else int(L_cap)
    else:
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(1) != 1:
            raise TypeError("block_table must be an int32 (B, pages) tensor with contiguous rows")
        page_size = int(page_size or k_codes.shape[2])
        bt_stride = block_table.stride(0)
        L_cap = block_table.shape[1] * page_size if L_cap is None else int(L_cap)
    L_max = L_cap if L_max is None else int(L_max)
    out_dtype = out_dtype or torch.bfloat16
    o = out if out is not None else torch.empty((B, h_q, s_q, d), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, h_q, s_q), dtype=torch.float32, device=q.device) if return_lse else None
    need = gqa_decode_paged_workspace_bytes(B, h_q, h_kv, s_q, L_max, int(window), d)
    ws = workspace if workspace is not None else torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check(lib.gqa_decode_fp8(_desc(q), _desc(k_codes), _desc(v_codes), float(k_scale), float(v_scale),
                              _ptr(block_table), bt_stride, page_size, _ptr(seqlens), _desc(o), _ptr(lse), B, h_q,
                              h_kv, s_q, L_cap, L_max, int(window), d, _out_code(o.dtype), float(scale or 0.0),
                              _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return (o, lse) if return_lse else o


def gta_shared_score_prefill(q, k, v, *, causal: bool = True, scale: float | None = None,
                             out=None, out_dtype=None, return_lse: bool = False, stream=None):
    """q, k (B, n_grp, S, d_qk); v (B, h, S, d_v).  Returns o (B, h, S, d_v)
    [and lse (B, n_grp, S)]."""
    import torch
    lib = load_library()
    _need_dtype((torch.bfloat16,), q=q)
    _check_common(q, "q", inputs=dict(k=k, v=v), out=out, out_dtype=out_dtype)
    B, n_grp, S, d_qk = q.shape
    h, d_v = v.shape[1], v.shape[3]
    out_dtype = out_dtype or torch.bfloat16
    o = out if out is not None else torch.empty((B, h, S, d_v), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, n_grp, S), dtype=torch.float32, device=q.device) if return_lse else None
    _check(lib.gta_shared_score_prefill(_desc(q), _desc(k), _desc(v), _desc(o), _ptr(lse), B, h,
                                        n_grp, S, d_qk, d_v, _dtype_code(q), _out_code(o.dtype),
                                        float(scale or 0.0), int(bool(causal)), _stream(stream)))
    return (o, lse) if return_lse else o


def gta_shared_score_decode_workspace_bytes(B, h, n_grp, s_q, L_max, d_v) -> int:
    return int(load_library().gta_shared_score_decode_workspace_bytes(B, h, n_grp, s_q, L_max, d_v))


def gta_shared_score_decode(q, k_cache, v_cache, seqlens, *, L_max: int | None = None,
                            scale: float | None = None, out=None, out_dtype=None, workspace=None,
                            return_lse: bool = False, stream=None):
    """q (B, n_grp, s_q, d_qk); k_cache (B, n_grp, L_cap, d_qk); v_cache
    (B, h, L_cap, d_v); seqlens int32 device (B,).  Returns o (B, h, s_q, d_v)
    [and lse (B, n_grp, s_q)]."""
    import torch
    lib = load_library()
    _need_dtype((torch.bfloat16,), q=q)
    _check_common(q, "q", inputs=dict(k_cache=k_cache, v_cache=v_cache), seqlens=seqlens, out=out, out_dtype=out_dtype,
                  workspace=workspace)
    B, n_grp, s_q, d_qk = q.shape
    h, L_cap, d_v = v_cache.shape[1], v_cache.shape[2], v_cache.shape[3]
    L_max = L_cap if L_max is None else int(L_max)
    out_dtype = out_dtype or torch.bfloat16
    o = out if out is not None else torch.empty((B, h, s_q, d_v), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, n_grp, s_q), dtype=torch.float32, device=q.device) if return_lse else None
    need = gta_shared_score_decode_workspace_bytes(B, h, n_grp, s_q, L_max, d_v)
    ws = workspace if workspace is not None else torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check(lib.gta_shared_score_decode(_desc(q), _desc(k_cache), _desc(v_cache), _ptr(seqlens), _desc(o),
                                       _ptr(lse), B, h, n_grp, s_q, L_cap, L_max, d_qk, d_v, _dtype_code(q),
                                       _out_code(o.dtype), float(scale or 0.0), _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream(stream)))
    return (o, lse) if return_lse else o


def gqla_gqa_decode_workspace_bytes(B, h_q, g, s_q, L_max, d_h) -> int:
    return int(load_library().gqla_gqa_decode_workspace_bytes(B, h_q, g, s_q, L_max, d_h))


def gqla_gqa_decode(q_c, q_r, k_c, k_r, v_cache, seqlens, *, scale: float, L_max: int | None = None,
                    out=None, out_dtype=None, workspace=None, return_lse: bool = False, stream=None):
    """q_c (B, h_q, s_q, d_h), q_r (B, h_q, s_q, d_r); k_c, v_cache (B, g, L_cap, d_h);
    k_r (B, L_cap, d_r), shared by the groups; seqlens int32 device (B,).
    Returns o (B, h_q, s_q, d_h) [and lse (B, h_q, s_q)]."""
    import torch
    lib = load_library()
    _need_dtype((torch.bfloat16,), q_c=q_c)
    _check_common(q_c, "q_c", inputs=dict(q_r=q_r, k_c=k_c, k_r=k_r, v_cache=v_cache), seqlens=seqlens,
                  out=out, out_dtype=out_dtype, workspace=workspace)
    B, h_q, s_q, d_h = q_c.shape
    d_r = q_r.shape[3]
    g, L_cap = k_c.shape[1], k_c.shape[2]
    L_max = L_cap if L_max is None else int(L_max)
    out_dtype = out_dtype or torch.bfloat16
    o = out if out is not None else torch.empty((B, h_q, s_q, d_h), dtype=out_dtype, device=q_c.device)
    lse = torch.empty((B, h_q, s_q), dtype=torch.float32, device=q_c.device) if return_lse else None
    need = gqla_gqa_decode_workspace_bytes(B, h_q, g, s_q, L_max, d_h)
    ws = workspace if workspace is not None else torch.empty(max(need, 16), dtype=torch.uint8, device=q_c.device)
    _check(lib.gqla_gqa_decode(_desc(q_c), _desc(q_r), _desc(k_c), _desc(k_r, (0, None, 1)), _desc(v_cache),
                               _ptr(seqlens), _desc(o), _ptr(lse), B, h_q, g, s_q, L_cap, L_max, d_h, d_r,
                               _dtype_code(q_c), _out_code(o.dtype), float(scale), _ptr(ws),
                               ws.numel() * ws.element_size(), _stream(stream)))
    return (o, lse) if return_lse else o


def gqla_gqa_prefill(q_c, q_r, k_c, k_r, v, *, scale: float, causal: bool = True, out=None,
                     out_dtype=None, return_lse: bool = False, stream=None):
    """q_c (B, h_q, S_q, d_h), q_r (B, h_q, S_q, d_r); k_c, v (B, g, S_k, d_h);
    k_r (B, S_k, d_r) shared by the groups.  Returns o (B, h_q, S_q, d_h)
    [and lse (B, h_q, S_q)]."""
    import torch
    lib = load_library()
    _need_dtype((torch.bfloat16,), q_c=q_c)
    _check_common(q_c, "q_c", inputs=dict(q_r=q_r, k_c=k_c, k_r=k_r, v=v), out=out, out_dtype=out_dtype)
    B, h_q, S_q, d_h = q_c.shape
    g, S_k = k_c.shape[1], k_c.shape[2]
    d_r = q_r.shape[3]
    out_dtype = out_dtype or torch.bfloat16
    o = out if out is not None else torch.empty((B, h_q, S_q, d_h), dtype=out_dtype, device=q_c.device)
    lse = torch.empty((B, h_q, S_q), dtype=torch.float32, device=q_c.device) if return_lse else None
    _check(lib.gqla_gqa_prefill(_desc(q_c), _desc(q_r), _desc(k_c), _desc(k_r, (0, None, 1)), _desc(v), _desc(o),
                                _ptr(lse), B, h_q, g, S_q, S_k, d_h, d_r, _dtype_code(q_c), _out_code(o.dtype),
                                float(scale), int(bool(causal)), _stream(stream)))
    return (o, lse) if return_lse else o


def latent_absorb_decode_workspace_bytes(B, h_q, s_q, L_max, r_kv) -> int:
    return int(load_library().latent_absorb_decode_workspace_bytes(B, h_q, s_q, L_max, r_kv))


def latent_absorb_decode(q_lat, q_rope, c_kv, k_rope, seqlens, *, scale: float,
                         L_max: int | None = None, out=None, out_dtype=None, workspace=None,
                         return_lse: bool = False, stream=None):
    """q_lat (B, s_q, h_q, r_kv), q_rope (B, s_q, h_q, d_r); c_kv (B, L_cap, r_kv),
    k_rope (B, L_cap, d_r) (may be views of one (B, L_cap, r_kv + d_r) buffer);
    seqlens int32 device (B,).  Returns o_lat (B, s_q, h_q, r_kv) [and lse
    (B, s_q, h_q)]."""
    import torch
    lib = load_library()
    _need_dtype((torch.bfloat16,), q_lat=q_lat)
    _check_common(q_lat, "q_lat", inputs=dict(q_rope=q_rope, c_kv=c_kv, k_rope=k_rope), seqlens=seqlens,
                  out=out, out_dtype=out_dtype, workspace=workspace)
    B, s_q, h_q, r_kv = q_lat.shape
    d_r = q_rope.shape[3]
    L_cap = c_kv.shape[1]
    L_max = L_cap if L_max is None else int(L_max)
    out_dtype = out_dtype or torch.bfloat16
    o = out if out is not None else torch.empty((B, s_q, h_q, r_kv), dtype=out_dtype, device=q_lat.device)
    lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device=q_lat.device) if return_lse else None
    need = latent_absorb_decode_workspace_bytes(B, h_q, s_q, L_max, r_kv)
    ws = workspace if workspace is not None else torch.empty(max(need, 16), dtype=torch.uint8, device=q_lat.device)
    # (batch, head, token) axes: q-like tensors are (B, s_q, h_q, .), caches (B, L, .)
    _check(lib.latent_absorb_decode(
        _desc(q_lat, (0, 2, 1)), _desc(q_rope, (0, 2, 1)), _desc(c_kv, (0, None, 1)),
        _desc(k_rope, (0, None, 1)), _ptr(seqlens), _desc(o, (0, 2, 1)), _ptr(lse),
        B, h_q, s_q, L_cap, L_max, r_kv, d_r, _dtype_code(q_lat), _out_code(o.dtype),
        float(scale), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return (o, lse) if return_lse else o


def gqla_absorb_decode_workspace_bytes(B, h_q, s_q, L_max, r_kv=512) -> int:
    return int(load_library().gqla_absorb_decode_workspace_bytes(B, h_q, s_q, L_max, r_kv))


def gqla_absorb_decode(q_c, q_rope, w_uk, w_uv, c_kv, k_rope, seqlens, *, g: int, scale: float,
                       L_max: int | None = None, out=None, out_dtype=None, workspace=None,
                       return_lse: bool = False, stream=None):
    """q_c (B, s_q, h_q, d_h), q_rope (B, s_q, h_q, d_r); w_uk, w_uv (g*d_h,
    r_kv) bf16; c_kv (B, L_cap, r_kv), k_rope (B, L_cap, d_r) (may be views of
    one (B, L_cap, r_kv + d_r) buffer).  Returns O (B, s_q, h_q, d_h) [and lse
    (B, s_q, h_q)]."""
    import torch
    lib = load_library()
    _need_dtype((torch.bfloat16,), q_c=q_c)
    _check_common(q_c, "q_c", inputs=dict(q_rope=q_rope, w_uk=w_uk, w_uv=w_uv, c_kv=c_kv, k_rope=k_rope),
                  seqlens=seqlens, out=out, out_dtype=out_dtype, workspace=workspace)
    B, s_q, h_q, d_h = q_c.shape
    d_r = q_rope.shape[3]
    L_cap, r_kv = c_kv.shape[1], c_kv.shape[2]
    L_max = L_cap if L_max is None else int(L_max)
    for w in (w_uk, w_uv):
        if not w.is_contiguous() or w.shape != (g * d_h, r_kv):
            raise ValueError("w_uk and w_uv must be contiguous (g * d_h, r_kv)")
    out_dtype = out_dtype or torch.bfloat16
    o = out if out is not None else torch.empty((B, s_q, h_q, d_h), dtype=out_dtype, device=q_c.device)
    lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device=q_c.device) if return_lse else None
    need = gqla_absorb_decode_workspace_bytes(B, h_q, s_q, L_max, r_kv)
    ws = workspace if workspace is not None else torch.empty(max(need, 256), dtype=torch.uint8, device=q_c.device)
    _check(lib.gqla_absorb_decode(
        _desc(q_c, (0, 2, 1)), _desc(q_rope, (0, 2, 1)), _ptr(w_uk), _ptr(w_uv), _desc(c_kv, (0, None, 1)),
        _desc(k_rope, (0, None, 1)), _ptr(seqlens), _desc(o, (0, 2, 1)), _ptr(lse), B, h_q, g, s_q, L_cap, L_max,
        d_h, r_kv, d_r, _dtype_code(q_c), _out_code(o.dtype), float(scale), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))
    return (o, lse) if return_lse else o
