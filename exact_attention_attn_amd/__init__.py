"""MI355X (gfx950) exact attention: thin Python binding over the C ABI in include/attn.h.

The functions here only marshal torch tensors (device pointers, sizes, the
current HIP stream) into the C calls of ``libattn_mi355x.so``; every step of
the computation runs in the library's HIP kernels.  Importing this package
does not load the library; the first call does, and fails loudly when it has
not been built (``python -m exact_attention_attn_amd.build``).
"""

from __future__ import annotations

import ctypes
import os
import threading

__all__ = ["attn_fwd", "attn_fwd_max_logit", "attn_fwd_varlen", "attn_bwd", "attn_decode_splitkv",
           "attn_decode_splitkv_paged", "attn_decode_plan", "attn_combine", "attn_decode_noalloc",
           "attn_strerror", "AttnError", "library_path", "load_library", "ATTN_BF16", "ATTN_F32",
           "MAX_SPLITS", "NOALLOC_SCRATCH_BYTES"]

ATTN_BF16 = 0
ATTN_F32 = 1
MAX_SPLITS = 64
NOALLOC_SCRATCH_BYTES = 135266304  # ATTN_NOALLOC_SCRATCH_BYTES of include/attn.h
SPLITS_POLICIES = {"auto": 0, "keys": 1, "count": 2}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libattn_mi355x.so"
_lock = threading.Lock()
_lib = None

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float

_SIGNATURES = {
    "attn_fwd": [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _i, _vp],
    "attn_fwd_max_logit": [_vp] * 8 + [_i] * 7 + [_f, _i, _i, _vp],
    "attn_decode_splitkv": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp],
    "attn_combine": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp],
    "attn_decode_plan": [_vp, _vp] + [_i] * 8 + [_vp],
    "attn_fwd_varlen": [_vp] * 8 + [_i] * 8 + [_f, _i, _i, _vp],
    "attn_bwd": [_vp] * 12 + [_i] * 7 + [_f, _i, _i, _vp],
    "attn_decode_splitkv_paged": [_vp] * 8 + [_i] * 9 + [_f, _i, _vp],
    "attn_decode_noalloc": [_vp] * 8 + [_i] * 7 + [_f, _i, _i, _vp],
    "attn_strerror": [_i],
    "attn_version": [],
}


class AttnError(RuntimeError):
    """A non-zero return code of the C library."""

    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn}: {attn_strerror(code)} (code {code})")


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def load_library() -> ctypes.CDLL:
    """Load the built HIP library (raises if it is missing: there is no fallback)."""
    global _lib
    with _lock:
        if _lib is None:
            path = library_path()
            if not os.path.exists(path):
                raise RuntimeError(
                    f"{path} is missing: build it with `python -m exact_attention_attn_amd.build`")
            lib = ctypes.CDLL(path)
            for name, args in _SIGNATURES.items():
                fn = getattr(lib, name)
                fn.argtypes = args
                fn.restype = ctypes.c_char_p if name in ("attn_strerror", "attn_version") else ctypes.c_int
            _lib = lib
    return _lib


def attn_strerror(code: int) -> str:
    return load_library().attn_strerror(int(code)).decode()


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}: bfloat16 or float32")


def _dev(t, name: str, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _same_dtype(q, **others):
    """Only q's element type reaches the C ABI: the other inputs must share it."""
    for name, t in others.items():
        if t.dtype != q.dtype:
            raise TypeError(f"{name} must have q's dtype {q.dtype}, got {t.dtype}")


def _stream(stream):
    import torch

    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _check(fn: str, rc: int):
    if rc != 0:
        raise AttnError(fn, rc)


def attn_fwd(q, k, v, sinks, out, lse=None, *, window: int = 0, scale: float | None = None,
             stream=None) -> None:
    """O and LSE of causal (+ sliding-window) GQA attention with a per-head sink.

    q [B,Hq,Lq,D], k/v [B,Hkv,Lk,D] (bf16 or fp32, same dtype), sinks [Hq] fp32 or
    None, out [B,Hq,Lq,D] (bf16 or fp32), lse [B,Hq,Lq] fp32 or None.
    """
    import torch

    B, Hq, Lq, D = q.shape
    _, Hkv, Lk, _ = k.shape
    if tuple(v.shape) != tuple(k.shape) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q/k/v/out")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    if sinks is not None and tuple(sinks.shape) != (Hq,):
        raise ValueError("sinks must be [Hq]")
    if lse is not None and tuple(lse.shape) != (B, Hq, Lq):
        raise ValueError("lse must be [B,Hq,Lq]")
    if scale is None:
        scale = D ** -0.5
    rc = load_library().attn_fwd(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(sinks, "sinks", torch.float32),
        _dev(out, "out"), _dev(lse, "lse", torch.float32), B, Hq, Hkv, Lq, Lk, D, int(window),
        float(scale), _dtype_code(q), _dtype_code(out), _stream(stream))
    _check("attn_fwd", rc)


def attn_fwd_max_logit(q, k, v, sinks, out, lse=None, max_row=None, max_head=None, *,
                       window: int = 0, scale: float | None = None, stream=None) -> None:
    """attn_fwd plus the largest pre-softmax logit scale*<q,k> over the visible keys.

    max_row [B,Hq,Lq] fp32 or None; max_head [B,Hq] fp32 or None (overwritten
    with -inf on the stream, then raised atomically).  out and lse are those
    of attn_fwd.
    """
    import torch

    B, Hq, Lq, D = q.shape
    _, Hkv, Lk, _ = k.shape
    if tuple(v.shape) != tuple(k.shape) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q/k/v/out")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    if sinks is not None and tuple(sinks.shape) != (Hq,):
        raise ValueError("sinks must be [Hq]")
    if lse is not None and tuple(lse.shape) != (B, Hq, Lq):
        raise ValueError("lse must be [B,Hq,Lq]")
    if max_row is not None and tuple(max_row.shape) != (B, Hq, Lq):
        raise ValueError("max_row must be [B,Hq,Lq]")
    if max_head is not None and tuple(max_head.shape) != (B, Hq):
        raise ValueError("max_head must be [B,Hq]")
    if scale is None:
        scale = D ** -0.5
    rc = load_library().attn_fwd_max_logit(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(sinks, "sinks", torch.float32),
        _dev(out, "out"), _dev(lse, "lse", torch.float32),
        _dev(max_row, "max_row", torch.float32), _dev(max_head, "max_head", torch.float32),
        B, Hq, Hkv, Lq, Lk, D, int(window), float(scale), _dtype_code(q), _dtype_code(out),
        _stream(stream))
    _check("attn_fwd_max_logit", rc)


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, sinks, out, lse=None, *,
                    max_seqlen_q: int, window: int = 0, scale: float | None = None,
                    stream=None) -> None:
    """attn_fwd over a packed batch: q [Hq,total_q,D], k/v [Hkv,total_k,D] (bf16),
    cu_seqlens_q/k [B+1] int32 (device), out [Hq,total_q,D], lse [Hq,total_q] or None."""
    import torch

    Hq, total_q, D = q.shape
    Hkv, total_k, _ = k.shape
    B = cu_seqlens_q.shape[0] - 1
    if tuple(cu_seqlens_k.shape) != (B + 1,):
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both be [B+1]")
    if tuple(v.shape) != tuple(k.shape) or tuple(out.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q/k/v/out")
    if sinks is not None and tuple(sinks.shape) != (Hq,):
        raise ValueError("sinks must be [Hq]")
    if lse is not None and tuple(lse.shape) != (Hq, total_q):
        raise ValueError("lse must be [Hq,total_q]")
    _same_dtype(q, k=k, v=v)
    if scale is None:
        scale = D ** -0.5
    rc = load_library().attn_fwd_varlen(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32),
        _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32), _dev(sinks, "sinks", torch.float32),
        _dev(out, "out"), _dev(lse, "lse", torch.float32), B, Hq, Hkv, total_q, total_k,
        int(max_seqlen_q), D, int(window), float(scale), _dtype_code(q), _dtype_code(out),
        _stream(stream))
    _check("attn_fwd_varlen", rc)


def attn_decode_splitkv_paged(q, k_pages, v_pages, block_table, seqlens_k, num_splits, o_part,
                              lse_part, *, window: int = 0, scale: float | None = None,
                              stream=None) -> None:
    """attn_decode_splitkv over a paged cache: pages [num_pages,Hkv,page_size,D] bf16,
    block_table [B,max_pages] int32.  Pass Lk_max = max_pages * page_size to attn_combine."""
    import torch

    B, Hq, one, D = q.shape
    if one != 1:
        raise ValueError("decode takes one query per sequence: q must be [B,Hq,1,D]")
    num_pages, Hkv, page_size, _ = k_pages.shape
    max_pages = block_table.shape[1]
    max_splits = o_part.shape[2]
    if tuple(v_pages.shape) != tuple(k_pages.shape):
        raise ValueError("k_pages and v_pages shapes differ")
    if tuple(block_table.shape) != (B, max_pages):
        raise ValueError("block_table must be [B,max_pages]")
    if tuple(o_part.shape) != (B, Hq, max_splits, D) or tuple(lse_part.shape) != (B, Hq, max_splits):
        raise ValueError("o_part must be [B,Hq,max_splits,D] and lse_part [B,Hq,max_splits]")
    _check_decode_inputs(q, k_pages, v_pages, seqlens_k, num_splits)
    if scale is None:
        scale = D ** -0.5
    rc = load_library().attn_decode_splitkv_paged(
        _dev(q, "q"), _dev(k_pages, "k_pages"), _dev(v_pages, "v_pages"),
        _dev(block_table, "block_table", torch.int32), _dev(seqlens_k, "seqlens_k", torch.int32),
        _dev(num_splits, "num_splits", torch.int32), _dev(o_part, "o_part", torch.float32),
        _dev(lse_part, "lse_part", torch.float32), B, Hq, Hkv, num_pages, page_size, max_pages, D,
        max_splits, int(window), float(scale), _dtype_code(q), _stream(stream))
    _check("attn_decode_splitkv_paged", rc)


def attn_bwd(q, k, v, sinks, out, dout, lse, dq, dk, dv, dsink=None, delta=None, *,
             window: int = 0, scale: float | None = None, stream=None) -> None:
    """dQ, dK, dV (and dsink) of attn_fwd for a given dO.

    q, dout [B,Hq,Lq,D] bf16; k, v [B,Hkv,Lk,D] bf16; out, lse: what attn_fwd
    returned (out bf16 or fp32 -- fp32 keeps dsink exact); dq, dk, dv fp32;
    dsink [Hq] fp32 or None; delta [B,Hq,Lq] fp32 workspace (allocated here
    when None).
    """
    import torch

    B, Hq, Lq, D = q.shape
    _, Hkv, Lk, _ = k.shape
    for name, t, shape in (("v", v, k.shape), ("out", out, q.shape), ("dout", dout, q.shape),
                           ("dq", dq, q.shape), ("dk", dk, k.shape), ("dv", dv, k.shape),
                           ("lse", lse, (B, Hq, Lq))):
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must be {tuple(shape)}")
    if sinks is not None and tuple(sinks.shape) != (Hq,):
        raise ValueError("sinks must be [Hq]")
    if dsink is not None and tuple(dsink.shape) != (Hq,):
        raise ValueError("dsink must be [Hq]")
    _same_dtype(q, k=k, v=v)
    if delta is None:
        delta = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    if scale is None:
        scale = D ** -0.5
    rc = load_library().attn_bwd(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(sinks, "sinks", torch.float32), _dev(out, "out"),
        _dev(dout, "dout", torch.bfloat16), _dev(lse, "lse", torch.float32),
        _dev(dq, "dq", torch.float32), _dev(dk, "dk", torch.float32), _dev(dv, "dv", torch.float32),
        _dev(dsink, "dsink", torch.float32), _dev(delta, "delta", torch.float32),
        B, Hq, Hkv, Lq, Lk, D, int(window), float(scale), _dtype_code(q), _dtype_code(out),
        _stream(stream))
    _check("attn_bwd", rc)


def _check_decode_inputs(q, k_cache, v_cache, seqlens_k, num_splits):
    """What the C ABI cannot check from pointers: element types of the cache
    and per-sequence arrays of exactly B int32 (the kernels read B of each)."""
    import torch

    B = q.shape[0]
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    for name, t in (("seqlens_k", seqlens_k), ("num_splits", num_splits)):
        if t.dtype != torch.int32 or tuple(t.shape) != (B,):
            raise ValueError(f"{name} must be int32 of shape ({B},), got {t.dtype} {tuple(t.shape)}")


def attn_decode_splitkv(q, k_cache, v_cache, seqlens_k, num_splits, o_part, lse_part, *,
                        window: int = 0, scale: float | None = None, stream=None) -> None:
    """Per-split partial outputs and sink-free LSEs of one decode step.

    q [B,Hq,1,D] bf16; caches [B,Hkv,Lk_max,D] bf16; seqlens_k, num_splits [B] int32;
    o_part [B,Hq,max_splits,D] fp32; lse_part [B,Hq,max_splits] fp32.
    """
    import torch

    B, Hq, one, D = q.shape
    if one != 1:
        raise ValueError("decode takes one query per sequence: q must be [B,Hq,1,D]")
    _, Hkv, Lk_max, _ = k_cache.shape
    max_splits = o_part.shape[2]
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache and v_cache shapes differ")
    if tuple(o_part.shape) != (B, Hq, max_splits, D) or tuple(lse_part.shape) != (B, Hq, max_splits):
        raise ValueError("o_part must be [B,Hq,max_splits,D] and lse_part [B,Hq,max_splits]")
    _check_decode_inputs(q, k_cache, v_cache, seqlens_k, num_splits)
    if scale is None:
        scale = D ** -0.5
    rc = load_library().attn_decode_splitkv(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(seqlens_k, "seqlens_k", torch.int32), _dev(num_splits, "num_splits", torch.int32),
        _dev(o_part, "o_part", torch.float32), _dev(lse_part, "lse_part", torch.float32),
        B, Hq, Hkv, Lk_max, D, max_splits, int(window), float(scale), _dtype_code(q),
        _stream(stream))
    _check("attn_decode_splitkv", rc)


def attn_decode_plan(seqlens_k, num_splits, *, Hq: int, Hkv: int, Lk_max: int,
                     max_splits: int = MAX_SPLITS, window: int = 0, policy: str = "auto",
                     param: int = 0, stream=None) -> None:
    """Write num_splits [B] int32 for attn_decode_splitkv on the device.

    policy "count" (param splits each), "keys" (ceil(n/param) splits for n
    visible keys) or "auto" (workload-aware rule; param = work-group count of
    the decode, 0 for the library's own), as include/attn.h states.
    """
    import torch

    B = seqlens_k.shape[0]
    if tuple(num_splits.shape) != (B,):
        raise ValueError("num_splits must be [B]")
    if policy not in SPLITS_POLICIES:
        raise ValueError(f"policy must be one of {sorted(SPLITS_POLICIES)}")
    rc = load_library().attn_decode_plan(
        _dev(seqlens_k, "seqlens_k", torch.int32), _dev(num_splits, "num_splits", torch.int32),
        B, int(Hq), int(Hkv), int(Lk_max), int(max_splits), int(window), SPLITS_POLICIES[policy],
        int(param), _stream(stream))
    _check("attn_decode_plan", rc)


def attn_combine(o_part, lse_part, seqlens_k, num_splits, sinks, out, lse=None, *, Lk_max: int,
                 window: int = 0, stream=None) -> None:
    """Merge the valid splits of each (b, h) and add the sink once.

    out [B,Hq,1,D] (bf16 or fp32); lse [B,Hq] fp32 or None.  Lk_max and window
    must be the values given to attn_decode_splitkv.
    """
    import torch

    B, Hq, max_splits, D = o_part.shape
    if tuple(out.shape) != (B, Hq, 1, D):
        raise ValueError("out must be [B,Hq,1,D]")
    if lse is not None and tuple(lse.shape) != (B, Hq):
        raise ValueError("lse must be [B,Hq]")
    if tuple(lse_part.shape) != (B, Hq, max_splits):
        raise ValueError("lse_part must be [B,Hq,max_splits]")
    for name, t in (("seqlens_k", seqlens_k), ("num_splits", num_splits)):
        if t.dtype != torch.int32 or tuple(t.shape) != (B,):
            raise ValueError(f"{name} must be int32 of shape ({B},)")
    if sinks is not None and tuple(sinks.shape) != (Hq,):
        raise ValueError("sinks must be [Hq]")
    rc = load_library().attn_combine(
        _dev(o_part, "o_part", torch.float32), _dev(lse_part, "lse_part", torch.float32),
        _dev(seqlens_k, "seqlens_k", torch.int32), _dev(num_splits, "num_splits", torch.int32),
        _dev(sinks, "sinks", torch.float32), _dev(out, "out"), _dev(lse, "lse", torch.float32),
        B, Hq, D, int(Lk_max), max_splits, int(window), _dtype_code(out), _stream(stream))
    _check("attn_combine", rc)


def attn_decode_noalloc(q, k_cache, v_cache, seqlens_k, num_splits, sinks, out, lse=None, *,
                        max_splits: int = MAX_SPLITS, window: int = 0, scale: float | None = None,
                        stream=None) -> None:
    """attn_decode_splitkv + attn_combine in one call that allocates nothing:
    the split workspace is the library's fixed device array (NOALLOC_SCRATCH_BYTES;
    larger workloads raise AttnError with code 6).  Calls that overlap in time
    on one GPU share that array and race.

    q [B,Hq,1,D] bf16; caches [B,Hkv,Lk_max,D] bf16; seqlens_k, num_splits [B]
    int32; sinks [Hq] fp32 or None; out [B,Hq,1,D] (bf16 or fp32); lse [B,Hq] or None.
    """
    import torch

    B, Hq, one, D = q.shape
    if one != 1:
        raise ValueError("decode takes one query per sequence: q must be [B,Hq,1,D]")
    _, Hkv, Lk_max, _ = k_cache.shape
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache and v_cache shapes differ")
    _check_decode_inputs(q, k_cache, v_cache, seqlens_k, num_splits)
    if tuple(out.shape) != (B, Hq, 1, D):
        raise ValueError("out must be [B,Hq,1,D]")
    if lse is not None and tuple(lse.shape) != (B, Hq):
        raise ValueError("lse must be [B,Hq]")
    if sinks is not None and tuple(sinks.shape) != (Hq,):
        raise ValueError("sinks must be [Hq]")
    if scale is None:
        scale = D ** -0.5
    rc = load_library().attn_decode_noalloc(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(seqlens_k, "seqlens_k", torch.int32), _dev(num_splits, "num_splits", torch.int32),
        _dev(sinks, "sinks", torch.float32), _dev(out, "out"), _dev(lse, "lse", torch.float32),
        B, Hq, Hkv, Lk_max, D, int(max_splits), int(window), float(scale), _dtype_code(q),
        _dtype_code(out), _stream(stream))
    _check("attn_decode_noalloc", rc)
