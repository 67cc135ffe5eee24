"""ctypes binding of libssa.so: argument marshalling only.

Each function here hands torch tensors' device pointers, strides and the
current HIP stream to the C entry point of the same name; every step of the
computation runs in the library's HIP kernels. There is no fallback: if the
library is missing or a tensor is not on the GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libssa.so")

SSA_F32 = 0
SSA_BF16 = 1

# Exported symbols, in the order include/ssa.h declares them.
EXPORTS = ("ssa_prefill", "ssa_prefill_dual", "ssa_prefill_backward", "ssa_prefill_backward_workspace_size",
           "ssa_decode", "ssa_decode_noalloc", "full_attn_decode", "ssa_decode_workspace_size", "ssa_extend",
           "ssa_extend_workspace_size", "hybrid_decode", "hybrid_decode_workspace_size",
           "ssa_status_string")


class SSAError(RuntimeError):
    """A non-zero ssa_status returned by the library."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class Pattern(ctypes.Structure):
    """ssa_pattern: block size b, sink blocks s, local blocks l."""
    _fields_ = [("block", ctypes.c_int32), ("sink", ctypes.c_int32), ("local", ctypes.c_int32)]


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libssa.so (built in-tree by ``__graft_entry__.build()``), or the
    build SSA_LIB names (the host-sanitized build of tests/sanitize.py)."""
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("SSA_LIB") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(hipcc --offload-arch=gfx950); there is no fallback path")
    lib = ctypes.CDLL(path)
    p, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                            ctypes.c_size_t)
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.ssa_prefill.restype = ctypes.c_int
    lib.ssa_prefill.argtypes = [ctypes.c_int, p, p, p, p, p, i32, i32, i32, i32, i32, i32,
                                i64p, i64p, i64p, i64p, Pattern, f32, p]
    lib.ssa_prefill_dual.restype = ctypes.c_int
    lib.ssa_prefill_dual.argtypes = [ctypes.c_int, p, p, p, p, p, p, p, p, f32, i32, i32, i32, i32,
                                     i32, i32, i64p, i64p, i64p, i64p, Pattern, f32, p]
    lib.ssa_prefill_backward.restype = ctypes.c_int
    lib.ssa_prefill_backward.argtypes = [ctypes.c_int, p, p, p, p, p, p, p, p, p, i32, i32, i32, i32,
                                         i32, i32, i64p, i64p, i64p, i64p, i64p, i64p, i64p, i64p,
                                         p, sz, Pattern, f32, p]
    lib.ssa_prefill_backward_workspace_size.restype = sz
    lib.ssa_prefill_backward_workspace_size.argtypes = [ctypes.c_int, i32, i32, i32, i32, i32, i32,
                                                        Pattern]
    lib.ssa_decode.restype = ctypes.c_int
    lib.ssa_decode.argtypes = [ctypes.c_int, p, p, p, i64p, i64p, p, i32, p, i32, i32, i32, i32, i32,
                               i32, p, p, p, sz, Pattern, f32, p]
    lib.full_attn_decode.restype = ctypes.c_int
    lib.full_attn_decode.argtypes = [ctypes.c_int, p, p, p, i64p, i64p, p, i32, p, i32, i32, i32,
                                     i32, i32, i32, p, p, p, sz, f32, p]
    lib.ssa_decode_noalloc.restype = ctypes.c_int
    lib.ssa_decode_noalloc.argtypes = [ctypes.c_int, p, p, p, i64p, i64p, p, i32, p, i32, i32, i32, i32,
                                       i32, i32, p, p, Pattern, f32, p]
    lib.ssa_decode_workspace_size.restype = sz
    lib.ssa_decode_workspace_size.argtypes = [ctypes.c_int, i32, i32, i32, i32, i32, i32, i32,
                                              Pattern, ctypes.c_int]
    lib.ssa_extend.restype = ctypes.c_int
    lib.ssa_extend.argtypes = [ctypes.c_int, p, p, p, i64p, i64p, p, i32, p, p, i32, i32, i32, i32, i32,
                               i32, i32, i32, p, p, p, sz, Pattern, f32, p]
    lib.ssa_extend_workspace_size.restype = sz
    lib.ssa_extend_workspace_size.argtypes = [ctypes.c_int, i32, i32, i32, i32, i32, i32, i32, i32,
                                              i32, Pattern]
    lib.hybrid_decode.restype = ctypes.c_int
    lib.hybrid_decode.argtypes = [ctypes.c_int, p, p, p, i64p, i64p, p, i32, p, p, i32, i32, i32, i32,
                                  i32, i32, i32, p, p, p, sz, Pattern, f32, p]
    lib.hybrid_decode_workspace_size.restype = sz
    lib.hybrid_decode_workspace_size.argtypes = [ctypes.c_int, i32, i32, i32, i32, i32, i32, i32, i32,
                                                 Pattern]
    lib.ssa_status_string.restype = ctypes.c_char_p
    lib.ssa_status_string.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().ssa_status_string(int(status)).decode()


def _check(status: int) -> None:
    if status != 0:
        raise SSAError(status, status_string(status))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SSA_BF16
    if t.dtype == torch.float32:
        return SSA_F32
    raise TypeError(f"SSA kernels take bfloat16 or float32 tensors, got {t.dtype}")


def _on_gpu(*tensors: torch.Tensor) -> None:
    for t in tensors:
        if not t.is_cuda:
            raise ValueError("SSA kernels run on the GPU only; got a tensor on " + str(t.device))


def _strides3(t: torch.Tensor):
    if t.stride(-1) != 1:
        raise ValueError("the head-dim axis must have unit stride")
    return (ctypes.c_int64 * 3)(*t.stride()[:3])


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, block: int = 128, sink: int = 1,
            local: int = 7, scale: float | None = None, out: torch.Tensor | None = None,
            return_lse: bool = False):
    """ssa_prefill: q [B, N, Hq, d_qk], k [B, N, Hkv, d_qk], v [B, N, Hkv, d_v].

    Returns o [B, N, Hq, d_v] (and lse [B, Hq, N] fp32 when ``return_lse``).
    The default scale is 1/sqrt(d_qk).
    """
    lib = load_library()
    _on_gpu(q, k, v)
    dt = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    B, N, Hq, d_qk = q.shape
    Hkv, d_v = k.shape[2], v.shape[3]
    if k.shape != (B, N, Hkv, d_qk) or v.shape != (B, N, Hkv, d_v):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if out is None:
        out = torch.empty((B, N, Hq, d_v), dtype=q.dtype, device=q.device)
    elif out.shape != (B, N, Hq, d_v) or out.dtype != q.dtype:
        raise ValueError("out has the wrong shape or dtype")
    _on_gpu(out)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device) if return_lse else None
    if scale is None:
        scale = 1.0 / math.sqrt(d_qk)
    _check(lib.ssa_prefill(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, N, Hq, Hkv, d_qk,
                           d_v, _strides3(q), _strides3(k), _strides3(v), _strides3(out),
                           Pattern(block, sink, local), float(scale), _stream(q.device)))
    return (out, lse) if return_lse else out


def prefill_dual(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, block: int = 128,
                 sink: int = 1, local: int = 7, scale: float | None = None,
                 alpha: float | None = None, return_lse: bool = False, out=None):
    """ssa_prefill_dual: SSA and full causal attention of the same inputs in
    one pass. Returns (o_ssa, o_full) and, when ``alpha`` is given, o_mix =
    alpha * o_full + (1 - alpha) * o_ssa after them; with ``return_lse`` the
    two lse tensors [B, Hq, N] follow. ``out`` may hold preallocated
    (o_ssa, o_full, o_mix) tensors of one layout (o_mix may be None)."""
    lib = load_library()
    _on_gpu(q, k, v)
    dt = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    B, N, Hq, d_qk = q.shape
    Hkv, d_v = k.shape[2], v.shape[3]
    if k.shape != (B, N, Hkv, d_qk) or v.shape != (B, N, Hkv, d_v):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if out is None:
        mk = lambda: torch.empty((B, N, Hq, d_v), dtype=q.dtype, device=q.device)  # noqa: E731
        o_ssa, o_full = mk(), mk()
        o_mix = mk() if alpha is not None else None
    else:
        o_ssa, o_full, o_mix = out
        for t in (o_ssa, o_full) + ((o_mix,) if o_mix is not None else ()):
            _on_gpu(t)
            if t.shape != (B, N, Hq, d_v) or t.dtype != q.dtype or t.stride() != o_ssa.stride():
                raise ValueError("outputs must be [B, N, Hq, d_v] of q's dtype with one layout")
        if (o_mix is None) != (alpha is None):
            raise ValueError("give alpha exactly when an o_mix buffer is given")
    lse = [torch.empty((B, Hq, N), dtype=torch.float32, device=q.device) if return_lse else None
           for _ in range(2)]
    if scale is None:
        scale = 1.0 / math.sqrt(d_qk)
    _check(lib.ssa_prefill_dual(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(o_ssa), _ptr(lse[0]),
                                _ptr(o_full), _ptr(lse[1]), _ptr(o_mix),
                                float(alpha if alpha is not None else 0.0), B, N, Hq, Hkv, d_qk,
                                d_v, _strides3(q), _strides3(k), _strides3(v), _strides3(o_ssa),
                                Pattern(block, sink, local), float(scale), _stream(q.device)))
    res = (o_ssa, o_full) + ((o_mix,) if o_mix is not None else ())
    return res + tuple(lse) if return_lse else res


def backward_workspace_size(dtype: torch.dtype, batch: int, seq_len: int, heads_q: int,
                            heads_kv: int, d_qk: int, d_v: int, *, block: int = 128, sink: int = 1,
                            local: int = 7) -> int:
    """Bytes of workspace ssa_prefill_backward needs (0 if it rejects the shape)."""
    code = SSA_BF16 if dtype == torch.bfloat16 else SSA_F32
    return int(load_library().ssa_prefill_backward_workspace_size(
        code, batch, seq_len, heads_q, heads_kv, d_qk, d_v, Pattern(block, sink, local)))


def prefill_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                     lse: torch.Tensor, dout: torch.Tensor, *, block: int = 128, sink: int = 1,
                     local: int = 7, scale: float | None = None, dq=None, dk=None, dv=None,
                     workspace=None):
    """ssa_prefill_backward: gradients (dq, dk, dv) of ``prefill`` for the
    upstream gradient ``dout``, given the forward's output ``o`` and its
    ``lse`` [B, Hq, N] (``prefill(..., return_lse=True)``)."""
    lib = load_library()
    _on_gpu(q, k, v, o, lse, dout)
    dt = _dtype_code(q)
    for t in (k, v, o, dout):
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, o, dout must share one dtype")
    B, N, Hq, d_qk = q.shape
    Hkv, d_v = k.shape[2], v.shape[3]
    if k.shape != (B, N, Hkv, d_qk) or v.shape != (B, N, Hkv, d_v):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if o.shape != (B, N, Hq, d_v) or dout.shape != (B, N, Hq, d_v):
        raise ValueError("o and dout must be [B, N, Hq, d_v]")
    if lse.dtype != torch.float32 or lse.shape != (B, Hq, N) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, Hq, N] tensor")
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
    dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
    for got, want in ((dq, q), (dk, k), (dv, v)):
        if got.shape != want.shape or got.dtype != want.dtype:
            raise ValueError("gradient outputs must match their inputs' shape and dtype")
    _on_gpu(dq, dk, dv)
    need = backward_workspace_size(q.dtype, B, N, Hq, Hkv, d_qk, d_v, block=block, sink=sink,
                                   local=local)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _on_gpu(workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(d_qk)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.ssa_prefill_backward(
        dt, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        B, N, Hq, Hkv, d_qk, d_v, _strides3(q), _strides3(k), _strides3(v), _strides3(o),
        _strides3(dout), _strides3(dq), _strides3(dk), _strides3(dv), _ptr(workspace), ws_bytes,
        Pattern(block, sink, local), float(scale), _stream(q.device)))
    return dq, dk, dv


def decode_workspace_size(dtype: torch.dtype, batch: int, heads_q: int, heads_kv: int, d_qk: int,
                          d_v: int, page_size: int, max_pages: int, *, block: int = 128,
                          sink: int = 1, local: int = 7, full: bool = False) -> int:
    """Bytes of workspace ssa_decode (or full_attn_decode, ``full=True``) needs."""
    code = SSA_BF16 if dtype == torch.bfloat16 else SSA_F32
    return int(load_library().ssa_decode_workspace_size(code, batch, heads_q, heads_kv, d_qk, d_v,
                                                        page_size, max_pages,
                                                        Pattern(block, sink, local), int(full)))


def _decode(full: bool, q, k_cache, v_cache, page_table, ctx_lens, *, block, sink, local, scale,
            out, workspace, return_lse, noalloc: bool = False):
    lib = load_library()
    _on_gpu(q, k_cache, v_cache, page_table, ctx_lens)
    dt = _dtype_code(q)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and the caches must share one dtype")
    if page_table.dtype != torch.int32 or ctx_lens.dtype != torch.int32:
        raise TypeError("page_table and ctx_lens must be int32")
    if not (q.is_contiguous() and page_table.is_contiguous() and ctx_lens.is_contiguous()):
        raise ValueError("q, page_table and ctx_lens must be contiguous")
    B, Hq, d_qk = q.shape
    _, page_size, Hkv, d_qk2 = k_cache.shape
    d_v = v_cache.shape[3]
    if d_qk2 != d_qk or v_cache.shape[:3] != k_cache.shape[:3]:
        raise ValueError("cache shape mismatch")
    if page_table.dim() != 2 or page_table.shape[0] != B or ctx_lens.shape != (B,):
        raise ValueError("page_table must be [B, max_pages] and ctx_lens [B]")
    max_pages = page_table.shape[1]
    if out is None:
        out = torch.empty((B, Hq, d_v), dtype=q.dtype, device=q.device)
    elif out.shape != (B, Hq, d_v) or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, Hq, d_v] tensor of q's dtype")
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if return_lse else None
    if scale is None:
        scale = 1.0 / math.sqrt(d_qk)
    if noalloc:
        _check(lib.ssa_decode_noalloc(dt, _ptr(q), _ptr(k_cache), _ptr(v_cache), _strides3(k_cache),
                                      _strides3(v_cache), _ptr(page_table), max_pages, _ptr(ctx_lens), B,
                                      Hq, Hkv, d_qk, d_v, page_size, _ptr(out), _ptr(lse),
                                      Pattern(block, sink, local), float(scale), _stream(q.device)))
        return (out, lse) if return_lse else out
    need = decode_workspace_size(q.dtype, B, Hq, Hkv, d_qk, d_v, page_size, max_pages, block=block,
                                 sink=sink, local=local, full=full)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _on_gpu(workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    common = (dt, _ptr(q), _ptr(k_cache), _ptr(v_cache), _strides3(k_cache), _strides3(v_cache),
              _ptr(page_table), max_pages, _ptr(ctx_lens), B, Hq, Hkv, d_qk, d_v, page_size,
              _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes)
    if full:
        _check(lib.full_attn_decode(*common, float(scale), _stream(q.device)))
    else:
        _check(lib.ssa_decode(*common, Pattern(block, sink, local), float(scale), _stream(q.device)))
    return (out, lse) if return_lse else out


def decode(q, k_cache, v_cache, page_table, ctx_lens, *, block: int = 128, sink: int = 1,
           local: int = 7, scale: float | None = None, out=None, workspace=None,
           return_lse: bool = False):
    """ssa_decode: q [B, Hq, d_qk]; caches [pages, page_size, Hkv, d]; page_table
    [B, max_pages] int32; ctx_lens [B] int32 (the new token included)."""
    return _decode(False, q, k_cache, v_cache, page_table, ctx_lens, block=block, sink=sink,
                   local=local, scale=scale, out=out, workspace=workspace, return_lse=return_lse)


def decode_noalloc(q, k_cache, v_cache, page_table, ctx_lens, *, block: int = 128, sink: int = 1,
                   local: int = 7, scale: float | None = None, out=None, return_lse: bool = False):
    """ssa_decode_noalloc: ``decode`` in the library's fixed per-GPU scratch
    (no workspace argument; the library allocates nothing)."""
    return _decode(False, q, k_cache, v_cache, page_table, ctx_lens, block=block, sink=sink,
                   local=local, scale=scale, out=out, workspace=None, return_lse=return_lse, noalloc=True)


def full_decode(q, k_cache, v_cache, page_table, ctx_lens, *, scale: float | None = None, out=None,
                workspace=None, return_lse: bool = False):
    """full_attn_decode: as ``decode`` but attending to the whole context."""
    return _decode(True, q, k_cache, v_cache, page_table, ctx_lens, block=1, sink=0, local=1,
                   scale=scale, out=out, workspace=workspace, return_lse=return_lse)


def extend_workspace_size(dtype: torch.dtype, batch: int, total_q: int, max_q_len: int, heads_q: int,
                          heads_kv: int, d_qk: int, d_v: int, page_size: int, max_pages: int, *,
                          block: int = 128, sink: int = 1, local: int = 7) -> int:
    """Bytes of workspace ssa_extend needs (0 for the tile kernel)."""
    code = SSA_BF16 if dtype == torch.bfloat16 else SSA_F32
    return int(load_library().ssa_extend_workspace_size(code, batch, total_q, max_q_len, heads_q,
                                                        heads_kv, d_qk, d_v, page_size, max_pages,
                                                        Pattern(block, sink, local)))


def extend(q, k_cache, v_cache, page_table, ctx_lens, cu_q, max_q_len: int, *, block: int = 128,
           sink: int = 1, local: int = 7, scale: float | None = None, out=None, workspace=None,
           return_lse: bool = False):
    """ssa_extend: q [total_q, Hq, d_qk] packed rows of the new tokens;
    caches [pages, page_size, Hkv, d]; page_table [B, max_pages] int32;
    ctx_lens [B] int32 (new tokens included); cu_q [B + 1] int32 prefix sums
    of the chunk lengths; max_q_len bounds every chunk length."""
    lib = load_library()
    _on_gpu(q, k_cache, v_cache, page_table, ctx_lens, cu_q)
    dt = _dtype_code(q)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and the caches must share one dtype")
    for t in (page_table, ctx_lens, cu_q):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise TypeError("page_table, ctx_lens and cu_q must be contiguous int32")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    total_q, Hq, d_qk = q.shape
    _, page_size, Hkv, d_qk2 = k_cache.shape
    d_v = v_cache.shape[3]
    B = ctx_lens.shape[0]
    if d_qk2 != d_qk or v_cache.shape[:3] != k_cache.shape[:3]:
        raise ValueError("cache shape mismatch")
    if page_table.dim() != 2 or page_table.shape[0] != B or cu_q.shape != (B + 1,):
        raise ValueError("page_table must be [B, max_pages] and cu_q [B + 1]")
    max_pages = page_table.shape[1]
    if out is None:
        out = torch.empty((total_q, Hq, d_v), dtype=q.dtype, device=q.device)
    elif out.shape != (total_q, Hq, d_v) or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [total_q, Hq, d_v] tensor of q's dtype")
    lse = torch.empty((total_q, Hq), dtype=torch.float32, device=q.device) if return_lse else None
    need = extend_workspace_size(q.dtype, B, total_q, max_q_len, Hq, Hkv, d_qk, d_v, page_size,
                                 max_pages, block=block, sink=sink, local=local)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _on_gpu(workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(d_qk)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.ssa_extend(dt, _ptr(q), _ptr(k_cache), _ptr(v_cache), _strides3(k_cache),
                          _strides3(v_cache), _ptr(page_table), max_pages, _ptr(ctx_lens), _ptr(cu_q),
                          B, total_q, int(max_q_len), Hq, Hkv, d_qk, d_v, page_size, _ptr(out),
                          _ptr(lse), _ptr(workspace), ws_bytes, Pattern(block, sink, local),
                          float(scale), _stream(q.device)))
    return (out, lse) if return_lse else out


def hybrid_decode_workspace_size(dtype: torch.dtype, batch: int, heads_q: int, heads_kv: int,
                                 d_qk: int, d_v: int, page_size: int, max_pages: int, topk_k: int, *,
                                 block: int = 1, sink: int = 16, local: int = 1024) -> int:
    """Bytes of workspace hybrid_decode needs."""
    code = SSA_BF16 if dtype == torch.bfloat16 else SSA_F32
    return int(load_library().hybrid_decode_workspace_size(code, batch, heads_q, heads_kv, d_qk, d_v,
                                                           page_size, max_pages, topk_k,
                                                           Pattern(block, sink, local)))


def hybrid_decode(q, k_cache, v_cache, page_table, ctx_lens, topk, *, block: int = 1, sink: int = 16,
                  local: int = 1024, scale: float | None = None, out=None, workspace=None,
                  return_lse: bool = False):
    """hybrid_decode: ``decode`` over the SSA window (by default 16 sink
    tokens and a 1,024-token window) plus the listed tokens topk [B, K] int32
    (entries inside the window, past the context or negative are skipped)."""
    lib = load_library()
    _on_gpu(q, k_cache, v_cache, page_table, ctx_lens, topk)
    dt = _dtype_code(q)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and the caches must share one dtype")
    for t in (page_table, ctx_lens, topk):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise TypeError("page_table, ctx_lens and topk must be contiguous int32")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    B, Hq, d_qk = q.shape
    _, page_size, Hkv, d_qk2 = k_cache.shape
    d_v = v_cache.shape[3]
    if d_qk2 != d_qk or v_cache.shape[:3] != k_cache.shape[:3]:
        raise ValueError("cache shape mismatch")
    if page_table.dim() != 2 or page_table.shape[0] != B or ctx_lens.shape != (B,):
        raise ValueError("page_table must be [B, max_pages] and ctx_lens [B]")
    if topk.dim() != 2 or topk.shape[0] != B:
        raise ValueError("topk must be [B, K]")
    K = topk.shape[1]
    max_pages = page_table.shape[1]
    if out is None:
        out = torch.empty((B, Hq, d_v), dtype=q.dtype, device=q.device)
    elif out.shape != (B, Hq, d_v) or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, Hq, d_v] tensor of q's dtype")
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if return_lse else None
    need = hybrid_decode_workspace_size(q.dtype, B, Hq, Hkv, d_qk, d_v, page_size, max_pages, K,
                                        block=block, sink=sink, local=local)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _on_gpu(workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(d_qk)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.hybrid_decode(dt, _ptr(q), _ptr(k_cache), _ptr(v_cache), _strides3(k_cache),
                             _strides3(v_cache), _ptr(page_table), max_pages, _ptr(ctx_lens),
                             _ptr(topk), K, B, Hq, Hkv, d_qk, d_v, page_size, _ptr(out), _ptr(lse),
                             _ptr(workspace), ws_bytes, Pattern(block, sink, local), float(scale),
                             _stream(q.device)))
    return (out, lse) if return_lse else out
