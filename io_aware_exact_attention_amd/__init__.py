"""Python binding of libmiattn (fused exact attention forward for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP kernels of
libmiattn.so.  PyTorch supplies device memory and the current stream.  There is no
fallback: if the library is not built, importing the entry points raises.

Entry points (same names and argument order as include/miattn.h):
    attn_fwd_prefill(q, k, v, o, lse, causal, scale, stream=None)
    attn_fwd_decode(q, kcache, vcache, block_table, seqlens, o, lse, max_seqlen, scale,
                    num_splits=0, workspace=None, page_size=16, num_pages=None, stream=None)
    attn_decode_workspace_bytes(B, Hq, d, max_seqlen, num_splits)
    attn_decode_num_splits(B, Hq, Hkv, d, max_seqlen, num_splits)
    attn_status_string(status)
Conveniences that allocate the outputs with torch and call the above:
    prefill(q, k, v, causal=True, scale=None) -> (o, lse)
    decode(q, kcache, vcache, seqlens, max_seqlen, block_table=None, scale=None,
           num_splits=0) -> (o, lse)
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# MIATTN_LIB names another build of the same library to load instead (the host-sanitizer
# build that the CPU tests use); by default the in-tree libmiattn.so.
LIB_PATH = os.environ.get("MIATTN_LIB") or os.path.join(_PKG_DIR, "libmiattn.so")

ATTN_OK = 0
_lib = None


class AttnError(RuntimeError):
    """A libmiattn call returned a non-zero status."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {attn_status_string(status)} (status {status})")


def load_library():
    """Load libmiattn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -c "
                           "'import __graft_entry__ as g; g.build()'` from the repository root")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.attn_fwd_prefill.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32,
                                     vp]
    lib.attn_fwd_prefill.restype = i32
    lib.attn_fwd_prefill_f16.argtypes = lib.attn_fwd_prefill.argtypes
    lib.attn_fwd_prefill_f16.restype = i32
    lib.attn_fwd_prefill_fp8.argtypes = [vp] * 5 + [i32] * 7 + [f32] * 4 + [vp]
    lib.attn_fwd_prefill_fp8.restype = i32
    lib.attn_fwd_prefill_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp] + [i32] * 10 + [f32, vp]
    lib.attn_fwd_prefill_paged.restype = i32
    lib.attn_fwd_prefill_paged_f16.argtypes = lib.attn_fwd_prefill_paged.argtypes
    lib.attn_fwd_prefill_paged_f16.restype = i32
    lib.attn_fwd_prefill_paged_fp8.argtypes = [vp] * 7 + [i32] * 10 + [f32] * 4 + [vp]
    lib.attn_fwd_prefill_paged_fp8.restype = i32
    lib.attn_fwd_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                    i32, f32, i32, vp, ctypes.c_size_t, vp]
    lib.attn_fwd_decode.restype = i32
    lib.attn_fwd_decode_noalloc.argtypes = [vp] * 7 + [i32] * 8 + [f32, i32, vp]
    lib.attn_fwd_decode_noalloc.restype = i32
    lib.attn_fwd_decode_f16.argtypes = lib.attn_fwd_decode.argtypes
    lib.attn_fwd_decode_f16.restype = i32
    lib.attn_fwd_decode_fp8.argtypes = [vp] * 7 + [i32] * 8 + [f32, f32, f32, i32, vp,
                                                               ctypes.c_size_t, vp]
    lib.attn_fwd_decode_fp8.restype = i32
    lib.attn_decode_workspace_bytes.argtypes = [i32] * 5
    lib.attn_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_decode_num_splits.argtypes = [i32] * 6
    lib.attn_decode_num_splits.restype = i32
    lib.attn_fwd_prefill_varlen.argtypes = [vp] * 7 + [i32] * 9 + [f32, vp]
    lib.attn_fwd_prefill_varlen.restype = i32
    lib.attn_fwd_prefill_varlen_f16.argtypes = lib.attn_fwd_prefill_varlen.argtypes
    lib.attn_fwd_prefill_varlen_f16.restype = i32
    lib.attn_fwd_prefill_varlen_fp8.argtypes = [vp] * 7 + [i32] * 9 + [f32] * 4 + [vp]
    lib.attn_fwd_prefill_varlen_fp8.restype = i32
    lib.attn_bwd.argtypes = [vp] * 9 + [i32] * 7 + [f32, vp, ctypes.c_size_t, vp]
    lib.attn_bwd.restype = i32
    lib.attn_bwd_f16.argtypes = lib.attn_bwd.argtypes
    lib.attn_bwd_f16.restype = i32
    lib.attn_bwd_workspace_bytes.argtypes = [i32] * 3
    lib.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_status_string.argtypes = [i32]
    lib.attn_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def attn_status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


def _stream_handle(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return ctypes.c_void_p(handle)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def _check(t, name, dtype, ndim, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if (t.dtype not in dtype) if isinstance(dtype, tuple) else (t.dtype != dtype):
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# -------------------------------------------------------------------------------- prefill
def _prefill_call(fn, dtype, q, k, v, o, lse, causal, scale, stream, fp8_scales=None):
    lib = load_library()
    _check(q, "q", dtype, 4)
    dev = q.device
    _check(k, "k", dtype, 4, dev)
    _check(v, "v", dtype, 4, dev)
    _check(o, "o", torch.bfloat16 if fp8_scales else dtype, 4, dev)
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if Bk != B or dk != d or tuple(v.shape) != tuple(k.shape) or tuple(o.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q, k, v, o")
    if lse is not None:
        _check(lse, "lse", torch.float32, 3, dev)
        if tuple(lse.shape) != (B, Hq, Nq):
            raise ValueError("lse must be [B, Hq, Nq]")
    extra = [float(x) for x in fp8_scales] if fp8_scales else []
    st = getattr(lib, fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk,
                          d, 1 if causal else 0, float(scale), *extra, _stream_handle(stream))
    if st != ATTN_OK:
        raise AttnError(st, fn)


def attn_fwd_prefill(q, k, v, o, lse, causal: bool, scale: float, stream=None) -> None:
    """q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d], o [B,Hq,Nq,d] bf16; lse [B,Hq,Nq] fp32 or None."""
    _prefill_call("attn_fwd_prefill", torch.bfloat16, q, k, v, o, lse, causal, scale, stream)


def attn_fwd_prefill_f16(q, k, v, o, lse, causal: bool, scale: float, stream=None) -> None:
    """attn_fwd_prefill with fp16 q, k, v, o."""
    _prefill_call("attn_fwd_prefill_f16", torch.float16, q, k, v, o, lse, causal, scale, stream)


def attn_fwd_prefill_fp8(q, k, v, o, lse, causal: bool, scale: float, q_scale: float,
                         k_scale: float, v_scale: float, stream=None) -> None:
    """attn_fwd_prefill over FP8 inputs: q, k, v hold OCP E4M3 codes (torch.uint8 or
    torch.float8_e4m3fn) standing for q_scale * e4m3(code) (k_scale, v_scale); o is bf16."""
    _prefill_call("attn_fwd_prefill_fp8", (torch.uint8, torch.float8_e4m3fn), q, k, v, o, lse,
                  causal, scale, stream, (q_scale, k_scale, v_scale))


def prefill_fp8(q, k, v, q_scale: float, k_scale: float, v_scale: float, causal: bool = True,
                scale: float | None = None):
    """Allocate O (bf16) and LSE and run attn_fwd_prefill_fp8.  scale None means 1/sqrt(d)."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    attn_fwd_prefill_fp8(q, k, v, o, lse, causal, scale, q_scale, k_scale, v_scale)
    return o, lse


def prefill(q, k, v, causal: bool = True, scale: float | None = None):
    """Allocate O and LSE and run attn_fwd_prefill (attn_fwd_prefill_f16 for fp16 inputs).
    scale None means 1/sqrt(d)."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    fn = attn_fwd_prefill_f16 if q.dtype == torch.float16 else attn_fwd_prefill
    fn(q, k, v, o, lse, causal, scale)
    return o, lse


def _prefill_paged_call(fn, dtype, q, kcache, vcache, block_table, kv_lens, o, lse, max_kv_len,
                        causal, scale, page_size, num_pages, stream, fp8_scales=None):
    lib = load_library()
    _check(q, "q", dtype, 4)
    dev = q.device
    _check(kcache, "kcache", dtype, 4, dev)
    _check(vcache, "vcache", dtype, 4, dev)
    _check(o, "o", torch.bfloat16 if fp8_scales else dtype, 4, dev)
    _check(block_table, "block_table", torch.int32, 2, dev)
    _check(kv_lens, "kv_lens", torch.int32, 1, dev)
    B, Hq, Nq, d = q.shape
    if tuple(vcache.shape) != tuple(kcache.shape) or tuple(o.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q/o or kcache/vcache")
    if kcache.shape[2] != page_size or kcache.shape[3] != d:
        raise ValueError("paged caches must be [num_pages, Hkv, page_size, d]")
    if block_table.shape[0] != B or kv_lens.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks] and kv_lens [B]")
    if lse is not None:
        _check(lse, "lse", torch.float32, 3, dev)
        if tuple(lse.shape) != (B, Hq, Nq):
            raise ValueError("lse must be [B, Hq, Nq]")
    if num_pages is None:
        num_pages = kcache.shape[0]
    st = getattr(lib, fn)(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(block_table),
                          _ptr(kv_lens), _ptr(o), _ptr(lse), B, Hq, kcache.shape[1], Nq,
                          d, int(max_kv_len), int(page_size), int(block_table.shape[1]),
                          int(num_pages), 1 if causal else 0, float(scale),
                          *([float(x) for x in fp8_scales] if fp8_scales else []),
                          _stream_handle(stream))
    if st != ATTN_OK:
        raise AttnError(st, fn)


def attn_fwd_prefill_paged_fp8(q, kcache, vcache, block_table, kv_lens, o, lse, max_kv_len: int,
                               causal: bool, scale: float, q_scale: float, k_scale: float,
                               v_scale: float, page_size: int = 16, num_pages: int | None = None,
                               stream=None) -> None:
    """attn_fwd_prefill_paged over FP8 inputs: q and the caches hold OCP E4M3 codes
    (torch.uint8 or torch.float8_e4m3fn) standing for q_scale * e4m3(code) (k_scale,
    v_scale); o is bf16."""
    _prefill_paged_call("attn_fwd_prefill_paged_fp8", (torch.uint8, torch.float8_e4m3fn), q,
                        kcache, vcache, block_table, kv_lens, o, lse, max_kv_len, causal, scale,
                        page_size, num_pages, stream, (q_scale, k_scale, v_scale))


def attn_fwd_prefill_paged(q, kcache, vcache, block_table, kv_lens, o, lse, max_kv_len: int,
                           causal: bool, scale: float, page_size: int = 16,
                           num_pages: int | None = None, stream=None) -> None:
    """Chunked prefill against a paged cache.  q/o [B,Hq,Nq,d] bf16; caches
    [num_pages,Hkv,16,d] bf16; block_table int32 [B, max_blocks] and kv_lens int32 [B]
    (device), each kv_lens[b] in [Nq, max_kv_len]; lse [B,Hq,Nq] fp32 or None."""
    _prefill_paged_call("attn_fwd_prefill_paged", torch.bfloat16, q, kcache, vcache, block_table,
                        kv_lens, o, lse, max_kv_len, causal, scale, page_size, num_pages, stream)


def attn_fwd_prefill_paged_f16(q, kcache, vcache, block_table, kv_lens, o, lse, max_kv_len: int,
                               causal: bool, scale: float, page_size: int = 16,
                               num_pages: int | None = None, stream=None) -> None:
    """attn_fwd_prefill_paged with fp16 q, caches and o."""
    _prefill_paged_call("attn_fwd_prefill_paged_f16", torch.float16, q, kcache, vcache,
                        block_table, kv_lens, o, lse, max_kv_len, causal, scale, page_size,
                        num_pages, stream)


def prefill_paged(q, kcache, vcache, block_table, kv_lens, max_kv_len: int, causal: bool = True,
                  scale: float | None = None):
    """Allocate O and LSE and run attn_fwd_prefill_paged.  scale None means 1/sqrt(d)."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    fn = attn_fwd_prefill_paged_f16 if q.dtype == torch.float16 else attn_fwd_prefill_paged
    fn(q, kcache, vcache, block_table, kv_lens, o, lse, max_kv_len, causal, scale)
    return o, lse


def _varlen_call(fn, dtype, q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                 max_seqlen_k, causal, scale, stream, fp8_scales=None):
    lib = load_library()
    _check(q, "q", dtype, 3)
    dev = q.device
    _check(k, "k", dtype, 3, dev)
    _check(v, "v", dtype, 3, dev)
    _check(o, "o", torch.bfloat16 if fp8_scales else dtype, 3, dev)
    _check(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1, dev)
    _check(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1, dev)
    total_q, Hq, d = q.shape
    total_k, Hkv, dk = k.shape
    B = cu_seqlens_q.shape[0] - 1
    if (dk != d or tuple(v.shape) != tuple(k.shape) or tuple(o.shape) != tuple(q.shape)
            or cu_seqlens_k.shape[0] != B + 1):
        raise ValueError("shape mismatch between q, k, v, o or the cumulative lengths")
    if lse is not None:
        _check(lse, "lse", torch.float32, 2, dev)
        if tuple(lse.shape) != (Hq, total_q):
            raise ValueError("lse must be [Hq, total_q]")
    st = getattr(lib, fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens_q),
                          _ptr(cu_seqlens_k), B, Hq, Hkv, total_q, total_k, int(max_seqlen_q),
                          int(max_seqlen_k), d, 1 if causal else 0, float(scale),
                          *([float(x) for x in fp8_scales] if fp8_scales else []),
                          _stream_handle(stream))
    if st != ATTN_OK:
        raise AttnError(st, fn)


def attn_fwd_prefill_varlen_fp8(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
                                max_seqlen_k: int, causal: bool, scale: float, q_scale: float,
                                k_scale: float, v_scale: float, stream=None) -> None:
    """attn_fwd_prefill_varlen over FP8 inputs: q, k, v hold OCP E4M3 codes (torch.uint8 or
    torch.float8_e4m3fn) standing for q_scale * e4m3(code) (k_scale, v_scale); o is bf16."""
    _varlen_call("attn_fwd_prefill_varlen_fp8", (torch.uint8, torch.float8_e4m3fn), q, k, v, o,
                 lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, causal, scale,
                 stream, (q_scale, k_scale, v_scale))


def attn_fwd_prefill_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
                            max_seqlen_k: int, causal: bool, scale: float, stream=None) -> None:
    """Ragged batch packed along tokens: q/o [total_q,Hq,d], k/v [total_k,Hkv,d] bf16;
    cu_seqlens_q/k int32 [B+1] (device); lse [Hq,total_q] fp32 or None."""
    _varlen_call("attn_fwd_prefill_varlen", torch.bfloat16, q, k, v, o, lse, cu_seqlens_q,
                 cu_seqlens_k, max_seqlen_q, max_seqlen_k, causal, scale, stream)


def attn_fwd_prefill_varlen_f16(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
                                max_seqlen_k: int, causal: bool, scale: float,
                                stream=None) -> None:
    """attn_fwd_prefill_varlen with fp16 q, k, v, o."""
    _varlen_call("attn_fwd_prefill_varlen_f16", torch.float16, q, k, v, o, lse, cu_seqlens_q,
                 cu_seqlens_k, max_seqlen_q, max_seqlen_k, causal, scale, stream)


def prefill_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                   causal: bool = True, scale: float | None = None):
    """Allocate O and LSE and run attn_fwd_prefill_varlen.  scale None means 1/sqrt(d)."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    o = torch.empty_like(q)
    lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    fn = attn_fwd_prefill_varlen_f16 if q.dtype == torch.float16 else attn_fwd_prefill_varlen
    fn(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, causal, scale)
    return o, lse


# -------------------------------------------------------------------------------- decode
def attn_decode_workspace_bytes(B, Hq, d, max_seqlen, num_splits=0) -> int:
    return int(load_library().attn_decode_workspace_bytes(B, Hq, d, max_seqlen, num_splits))


def attn_decode_num_splits(B, Hq, Hkv, d, max_seqlen, num_splits=0) -> int:
    return int(load_library().attn_decode_num_splits(B, Hq, Hkv, d, max_seqlen, num_splits))


def _decode_args(q, kcache, vcache, block_table, seqlens, o, lse, max_seqlen, workspace,
                 page_size, num_pages, cache_dtypes, qo_dtype=torch.bfloat16):
    """Checks shared by the decode entry points; returns the size arguments."""
    _check(q, "q", qo_dtype, 3)
    dev = q.device
    for name, t in (("kcache", kcache), ("vcache", vcache)):
        if isinstance(t, torch.Tensor) and t.dtype in cache_dtypes:
            _check(t, name, t.dtype, 4, dev)
        else:
            _check(t, name, cache_dtypes[0], 4, dev)
    _check(o, "o", qo_dtype, 3, dev)
    _check(seqlens, "seqlens", torch.int32, 1, dev)
    B, Hq, d = q.shape
    if tuple(vcache.shape) != tuple(kcache.shape) or tuple(o.shape) != tuple(q.shape):
        raise ValueError("shape mismatch between q/o or kcache/vcache")
    if seqlens.shape[0] != B:
        raise ValueError("seqlens must be [B]")
    Hkv = kcache.shape[1]
    if kcache.shape[3] != d:
        raise ValueError("cache head dimension differs from q")
    max_blocks = 0
    if block_table is None:
        if kcache.shape[0] != B or kcache.shape[2] != max_seqlen:
            raise ValueError("contiguous caches must be [B, Hkv, max_seqlen, d]")
        num_pages = 0
    else:
        _check(block_table, "block_table", torch.int32, 2, dev)
        if block_table.shape[0] != B:
            raise ValueError("block_table must be [B, max_blocks]")
        max_blocks = block_table.shape[1]
        if kcache.shape[2] != page_size:
            raise ValueError("paged caches must be [num_pages, Hkv, page_size, d]")
        if num_pages is None:
            num_pages = kcache.shape[0]
    if lse is not None:
        _check(lse, "lse", torch.float32, 2, dev)
        if tuple(lse.shape) != (B, Hq):
            raise ValueError("lse must be [B, Hq]")
    ws_bytes = 0
    if workspace is not None:
        if workspace.device != dev or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on q's device")
        ws_bytes = workspace.numel() * workspace.element_size()
    return B, Hq, Hkv, d, max_blocks, num_pages, ws_bytes


def _decode_call(fn, dtype, q, kcache, vcache, block_table, seqlens, o, lse, max_seqlen, scale,
                 num_splits, workspace, page_size, num_pages, stream):
    lib = load_library()
    B, Hq, Hkv, d, max_blocks, num_pages, ws_bytes = _decode_args(
        q, kcache, vcache, block_table, seqlens, o, lse, max_seqlen, workspace, page_size,
        num_pages, (dtype,), dtype)
    st = getattr(lib, fn)(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(block_table),
                          _ptr(seqlens), _ptr(o), _ptr(lse), B, Hq, Hkv, d, int(max_seqlen),
                          int(page_size), int(max_blocks), int(num_pages), float(scale),
                          int(num_splits), _ptr(workspace), ws_bytes, _stream_handle(stream))
    if st != ATTN_OK:
        raise AttnError(st, fn)


def attn_fwd_decode(q, kcache, vcache, block_table, seqlens, o, lse, max_seqlen: int,
                    scale: float, num_splits: int = 0, workspace=None, page_size: int = 16,
                    num_pages: int | None = None, stream=None) -> None:
    """q/o [B,Hq,d] bf16; lse [B,Hq] fp32 or None; seqlens int32 [B] (device).
    block_table None: caches [B,Hkv,max_seqlen,d]; else caches [num_pages,Hkv,16,d] and
    block_table int32 [B, max_blocks]."""
    _decode_call("attn_fwd_decode", torch.bfloat16, q, kcache, vcache, block_table, seqlens, o,
                 lse, max_seqlen, scale, num_splits, workspace, page_size, num_pages, stream)


ATTN_DECODE_NOALLOC_MAX_BYTES = 32 << 20


def attn_fwd_decode_noalloc(q, kcache, vcache, block_table, seqlens, o, lse, max_seqlen: int,
                            scale: float, num_splits: int = 0, page_size: int = 16,
                            num_pages: int | None = None, stream=None) -> None:
    """attn_fwd_decode with its split partials in the library's per-GPU static array
    (ATTN_DECODE_NOALLOC_MAX_BYTES) instead of a workspace: allocates nothing.  Calls
    that may overlap on one GPU race."""
    lib = load_library()
    B, Hq, Hkv, d, max_blocks, num_pages, _ = _decode_args(
        q, kcache, vcache, block_table, seqlens, o, lse, max_seqlen, None, page_size,
        num_pages, (torch.bfloat16,), torch.bfloat16)
    st = lib.attn_fwd_decode_noalloc(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(block_table),
                                     _ptr(seqlens), _ptr(o), _ptr(lse), B, Hq, Hkv, d,
                                     int(max_seqlen), int(page_size), int(max_blocks),
                                     int(num_pages), float(scale), int(num_splits),
                                     _stream_handle(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_decode_noalloc")


def attn_fwd_decode_f16(q, kcache, vcache, block_table, seqlens, o, lse, max_seqlen: int,
                        scale: float, num_splits: int = 0, workspace=None, page_size: int = 16,
                        num_pages: int | None = None, stream=None) -> None:
    """attn_fwd_decode with fp16 q, caches and o."""
    _decode_call("attn_fwd_decode_f16", torch.float16, q, kcache, vcache, block_table, seqlens, o,
                 lse, max_seqlen, scale, num_splits, workspace, page_size, num_pages, stream)


def attn_fwd_decode_fp8(q, kcache, vcache, block_table, seqlens, o, lse, max_seqlen: int,
                        scale: float, k_scale: float, v_scale: float, num_splits: int = 0,
                        workspace=None, page_size: int = 16, num_pages: int | None = None,
                        stream=None) -> None:
    """attn_fwd_decode over an FP8 cache: kcache/vcache hold OCP E4M3 codes (torch.uint8
    or torch.float8_e4m3fn) standing for k_scale * e4m3(code) and v_scale * e4m3(code)."""
    lib = load_library()
    B, Hq, Hkv, d, max_blocks, num_pages, ws_bytes = _decode_args(
        q, kcache, vcache, block_table, seqlens, o, lse, max_seqlen, workspace, page_size,
        num_pages, (torch.uint8, torch.float8_e4m3fn))
    st = lib.attn_fwd_decode_fp8(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(block_table),
                                 _ptr(seqlens), _ptr(o), _ptr(lse), B, Hq, Hkv, d,
                                 int(max_seqlen), int(page_size), int(max_blocks),
                                 int(num_pages), float(scale), float(k_scale), float(v_scale),
                                 int(num_splits), _ptr(workspace), ws_bytes,
                                 _stream_handle(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_decode_fp8")


def decode_workspace(B, Hq, d, max_seqlen, num_splits=0, device="cuda"):
    """A workspace tensor of the size attn_fwd_decode needs (None when it needs none)."""
    n = attn_decode_workspace_bytes(B, Hq, d, max_seqlen, num_splits)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def decode(q, kcache, vcache, seqlens, max_seqlen: int, block_table=None,
           scale: float | None = None, num_splits: int = 0, workspace=None):
    """Allocate O, LSE (and the workspace when not given) and run attn_fwd_decode."""
    B, Hq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = decode_workspace(B, Hq, d, max_seqlen, num_splits, q.device)
    fn = attn_fwd_decode_f16 if q.dtype == torch.float16 else attn_fwd_decode
    fn(q, kcache, vcache, block_table, seqlens, o, lse, max_seqlen, scale, num_splits, workspace)
    return o, lse


def decode_fp8(q, kcache, vcache, seqlens, max_seqlen: int, k_scale: float, v_scale: float,
               block_table=None, scale: float | None = None, num_splits: int = 0,
               workspace=None):
    """Allocate O, LSE (and the workspace when not given) and run attn_fwd_decode_fp8."""
    B, Hq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = decode_workspace(B, Hq, d, max_seqlen, num_splits, q.device)
    attn_fwd_decode_fp8(q, kcache, vcache, block_table, seqlens, o, lse, max_seqlen, scale,
                        k_scale, v_scale, num_splits, workspace)
    return o, lse


# -------------------------------------------------------------------------------- backward
def attn_bwd_workspace_bytes(B, Hq, Nq) -> int:
    return int(load_library().attn_bwd_workspace_bytes(B, Hq, Nq))


def _bwd_call(fn, dtype, q, k, v, o, lse, dout, dq, dk, dv, causal, scale, workspace, stream):
    lib = load_library()
    _check(q, "q", dtype, 4)
    dev = q.device
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk),
                    ("dv", dv)):
        _check(t, name, dtype, 4, dev)
    _check(lse, "lse", torch.float32, 3, dev)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if (tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape)
            or tuple(dq.shape) != tuple(q.shape) or tuple(v.shape) != tuple(k.shape)
            or tuple(dk.shape) != tuple(k.shape) or tuple(dv.shape) != tuple(k.shape)
            or k.shape[0] != B or k.shape[3] != d or tuple(lse.shape) != (B, Hq, Nq)):
        raise ValueError("shape mismatch between the backward's tensors")
    if workspace is None:
        workspace = torch.empty(attn_bwd_workspace_bytes(B, Hq, Nq), dtype=torch.uint8,
                                device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = getattr(lib, fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                          _ptr(dk), _ptr(dv), B, Hq, Hkv, Nq, Nk, d, 1 if causal else 0,
                          float(scale), _ptr(workspace), ws_bytes, _stream_handle(stream))
    if st != ATTN_OK:
        raise AttnError(st, fn)


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, causal: bool, scale: float, workspace=None,
             stream=None) -> None:
    """Gradients of attn_fwd_prefill.  q, o, dout, dq [B,Hq,Nq,d] bf16; k, v, dk, dv
    [B,Hkv,Nk,d] bf16; lse [B,Hq,Nq] fp32 (the forward's); workspace of at least
    attn_bwd_workspace_bytes(B, Hq, Nq) bytes (allocated here when None)."""
    _bwd_call("attn_bwd", torch.bfloat16, q, k, v, o, lse, dout, dq, dk, dv, causal, scale,
              workspace, stream)


def attn_bwd_f16(q, k, v, o, lse, dout, dq, dk, dv, causal: bool, scale: float, workspace=None,
                 stream=None) -> None:
    """attn_bwd with fp16 q, k, v, o, dout, dq, dk, dv."""
    _bwd_call("attn_bwd_f16", torch.float16, q, k, v, o, lse, dout, dq, dk, dv, causal, scale,
              workspace, stream)


def backward(q, k, v, o, lse, dout, causal: bool = True, scale: float | None = None):
    """Allocate dq, dk, dv and run attn_bwd (attn_bwd_f16 for fp16 tensors).  scale None
    means 1/sqrt(d)."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fn = attn_bwd_f16 if q.dtype == torch.float16 else attn_bwd
    fn(q, k, v, o, lse, dout, dq, dk, dv, causal, scale)
    return dq, dk, dv


__all__ = ["attn_bwd", "attn_bwd_f16", "attn_bwd_workspace_bytes", "backward", "attn_fwd_prefill_varlen",
           "attn_fwd_prefill_varlen_f16", "attn_fwd_prefill_varlen_fp8",
           "prefill_varlen",
           "attn_fwd_prefill", "attn_fwd_prefill_f16", "attn_fwd_prefill_fp8", "prefill_fp8",
           "attn_fwd_prefill_paged_f16", "attn_fwd_prefill_paged_fp8",
           "attn_fwd_decode", "attn_fwd_decode_f16", "attn_fwd_decode_fp8",
           "attn_decode_workspace_bytes", "decode_fp8",
           "attn_decode_num_splits", "attn_status_string", "prefill", "decode",
           "attn_fwd_prefill_paged", "prefill_paged",
           "decode_workspace", "load_library", "AttnError", "LIB_PATH",
           "attn_fwd_decode_noalloc", "ATTN_DECODE_NOALLOC_MAX_BYTES"]
