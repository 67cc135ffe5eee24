"""CPU oracle for streaming sparse attention: test infrastructure only.

This package wraps ``ssa_oracle.c`` (plain C, double precision) with ctypes.
Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import it; the product library never does, and the two share no code.

What the oracle computes, and the readings it takes where the pages are
silent, is stated at the top of ``ssa_oracle.c``. In short (LongCat ZigZag
Attention digest, section 01 part (1), the SSA paragraph, and part (2), the
deployed configuration b=128, s=1, l=7): query i attends to key j iff
``j <= i`` and ``j // b < s or j // b > i // b - l``, with scaled-dot-product
softmax over those keys.

Arrays are numpy: float32, or uint16 holding bfloat16 bit patterns (both are
exact in double). Any strides are accepted as long as the last (head-dim)
axis is contiguous.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssa_oracle.c")
_LIB = os.path.join(_HERE, "libssa_oracle.so")
# The same source built with AddressSanitizer and UBSan (tests/sanitize.py);
# SSA_ORACLE_LIB names the build to load.
_LIB_SANITIZED = os.path.join(_HERE, "libssa_oracle_asan.so")
_lib = None

ELEM_F32 = 0
ELEM_BF16 = 1


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no hand vectorisation); with
    sanitize, a separate AddressSanitizer + UBSan build (-O1, aborting on the
    first report), loaded only when SSA_ORACLE_LIB names it."""
    out = _LIB_SANITIZED if sanitize else _LIB
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(_SRC):
        tmp = out + ".tmp"
        flags = (["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=undefined"] if sanitize else ["-O2"])
        subprocess.check_call(["gcc", *flags, "-fopenmp", "-shared", "-fPIC", "-std=c11",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, out)
    return out


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get("SSA_ORACLE_LIB") or _LIB
        if path == _LIB and not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(path)
        p, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.oracle_ssa_prefill.restype = i32
        lib.oracle_ssa_prefill.argtypes = [i32, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32,
                                           i32, i32, i32, i32, dbl, p, i64, p, p, p]
        lib.oracle_decode_paged.restype = i32
        lib.oracle_decode_paged.argtypes = [i32, p, p, p, p, p, i64, p, i64, p, i32, i32, i32,
                                            i32, i32, i32, i32, i32, i32, i32, dbl, p, p]
        lib.oracle_ssa_backward.restype = i32
        lib.oracle_ssa_backward.argtypes = [i32, p, p, p, p, p, p, p, p, i32, i32, i32, i32, i32,
                                            i32, i32, i32, i32, i32, dbl, p, i64, p, p, p]
        lib.oracle_max_threads.restype = i32
        lib.oracle_set_threads.argtypes = [i32]
        _lib = lib
    return _lib


def _elem(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return ELEM_F32
    if a.dtype == np.uint16:
        return ELEM_BF16
    raise TypeError(f"oracle takes float32 or bfloat16 bits (uint16), got {a.dtype}")


def _strides(a: np.ndarray, axes: int) -> np.ndarray:
    if a.strides[-1] != a.itemsize:
        raise ValueError("last axis must be contiguous")
    return np.array([s // a.itemsize for s in a.strides[:axes]], dtype=np.int64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def prefill(q, k, v, *, block=128, sink=1, local=7, scale, full=False, rows=None,
            weights=False):
    """Attention of every (or every listed) query row of [B, N, H, d] inputs.

    Returns ``(o, lse, w)``: o [B, R, Hq, d_v] float64, lse [B, Hq, R] float64,
    w [B, Hq, R, N] float64 dense weights (only when ``weights``; else None).
    ``full=True`` gives plain causal attention (the pattern is ignored).
    """
    lib = _load()
    elem = _elem(q)
    if _elem(k) != elem or _elem(v) != elem:
        raise TypeError("q, k, v must share one element type")
    B, N, Hq, d_qk = q.shape
    Bk, Nk, Hkv, d_qk2 = k.shape
    Bv, Nv, Hkv2, d_v = v.shape
    if (Bk, Nk, d_qk2) != (B, N, d_qk) or (Bv, Nv, Hkv2) != (B, N, Hkv):
        raise ValueError("shape mismatch")
    rows_arr = None
    if rows is not None:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    R = N if rows_arr is None else rows_arr.size
    o = np.empty((B, R, Hq, d_v), dtype=np.float64)
    lse = np.empty((B, Hq, R), dtype=np.float64)
    w = np.empty((B, Hq, R, N), dtype=np.float64) if weights else None
    qs, ks, vs = _strides(q, 3), _strides(k, 3), _strides(v, 3)
    rc = lib.oracle_ssa_prefill(elem, _ptr(q), _ptr(k), _ptr(v), _ptr(qs), _ptr(ks), _ptr(vs),
                                B, N, Hq, Hkv, d_qk, d_v, block, sink, local, int(full),
                                float(scale), _ptr(rows_arr), R, _ptr(o), _ptr(lse), _ptr(w))
    if rc != 0:
        raise ValueError("oracle_ssa_prefill rejected its arguments")
    return o, lse, w


def prefill_dual(q, k, v, *, block=128, sink=1, local=7, scale, alpha=None, rows=None):
    """The calibration forward (LongCat ZigZag Attention digest, section 01
    part (1), the calibration paragraph): SSA attention, full causal attention
    and their mix, read as ``alpha * o_full + (1 - alpha) * o_ssa`` (the mix
    equation is lost from the page).

    Returns ``(o_ssa, lse_ssa, o_full, lse_full, o_mix)`` in float64, shapes as
    ``prefill``; o_mix is None when ``alpha`` is None.
    """
    kw = dict(block=block, sink=sink, local=local, scale=scale, rows=rows)
    o_ssa, lse_ssa, _ = prefill(q, k, v, **kw)
    o_full, lse_full, _ = prefill(q, k, v, full=True, **kw)
    o_mix = None
    if alpha is not None:
        if not 0.0 <= alpha <= 1.0:
            raise ValueError("alpha must lie in [0, 1]")
        o_mix = alpha * o_full + (1.0 - alpha) * o_ssa
    return o_ssa, lse_ssa, o_full, lse_full, o_mix


def decode_paged(q, k_cache, v_cache, page_table, ctx_lens, *, block=128, sink=1, local=7,
                 scale, full=False):
    """One new query per sequence against a paged cache.

    q [B, Hq, d_qk]; k_cache [pages, page_size, Hkv, d_qk]; v_cache
    [pages, page_size, Hkv, d_v] (may be a view of k_cache); page_table
    [B, max_pages] int32; ctx_lens [B] int32. Returns ``(o, lse)`` in float64.
    """
    lib = _load()
    elem = _elem(q)
    if _elem(k_cache) != elem or _elem(v_cache) != elem:
        raise TypeError("q and caches must share one element type")
    q = np.ascontiguousarray(q)
    B, Hq, d_qk = q.shape
    num_pages, page_size, Hkv, d_qk2 = k_cache.shape
    num_pages2, page_size2, Hkv2, d_v = v_cache.shape
    if d_qk2 != d_qk or (num_pages2, page_size2, Hkv2) != (num_pages, page_size, Hkv):
        raise ValueError("cache shape mismatch")
    page_table = np.ascontiguousarray(page_table, dtype=np.int32)
    ctx_lens = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    if page_table.shape[0] != B or ctx_lens.shape != (B,):
        raise ValueError("page_table / ctx_lens shape mismatch")
    max_pages = page_table.shape[1]
    o = np.empty((B, Hq, d_v), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64)
    ks, vs = _strides(k_cache, 3), _strides(v_cache, 3)
    rc = lib.oracle_decode_paged(elem, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(ks),
                                 _ptr(vs), num_pages, _ptr(page_table), max_pages,
                                 _ptr(ctx_lens), page_size, B, Hq, Hkv, d_qk, d_v, block, sink,
                                 local, int(full), float(scale), _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_decode_paged rejected its arguments")
    return o, lse


def extend(q, k_cache, v_cache, page_table, ctx_lens, cu_q, *, block=128, sink=1, local=7, scale):
    """New tokens of each sequence against the paged cache (chunked prefill,
    multi-token decode). Sequence b's rows cu_q[b] .. cu_q[b+1]-1 sit at the
    last q_len_b positions of its ctx_lens[b] tokens; a row at position p
    attends exactly as one decode step at context length p + 1 (the SSA
    paragraph defines the window per query position; decode puts the query at
    the last position of its context). Each row is handed to ``decode_paged``
    with its own context length and its sequence's page-table row.

    q [total_q, Hq, d_qk]. Returns ``(o, lse)``: [total_q, Hq, d_v] and
    [total_q, Hq] in float64.
    """
    cu_q = np.asarray(cu_q, dtype=np.int64)
    ctx_lens = np.asarray(ctx_lens, dtype=np.int64)
    page_table = np.asarray(page_table, dtype=np.int32)
    B = ctx_lens.shape[0]
    if cu_q.shape != (B + 1,) or cu_q[0] != 0 or np.any(np.diff(cu_q) < 0) or cu_q[-1] != q.shape[0]:
        raise ValueError("cu_q must be non-decreasing prefix sums from 0 to total_q")
    q_len = np.diff(cu_q)
    if np.any(q_len > ctx_lens):
        raise ValueError("a chunk is longer than its context")
    seq = np.repeat(np.arange(B), q_len)
    r = np.arange(q.shape[0]) - cu_q[seq]
    row_ctx = (ctx_lens[seq] - q_len[seq] + r + 1).astype(np.int32)
    return decode_paged(q, k_cache, v_cache, page_table[seq], row_ctx, block=block, sink=sink,
                        local=local, scale=scale)


def _bf16_or_f32_to_f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def hybrid_decode(q, k_cache, v_cache, page_table, ctx_lens, topk, *, block=1, sink=16, local=1024,
                  scale):
    """One decode step over the SSA window plus listed tokens (the streaming-
    aware indexing of "LongCat Sparse Attention": fixed sink and window
    tokens, and tokens an indexer chose). For the query at position L - 1 the
    attended set is the window of the block rule (j <= L - 1 with j // b < s
    or j // b > (L - 1) // b - l) united with the listed positions that lie in
    [0, L); negative entries are padding. One softmax over that set.

    q [B, Hq, d_qk], caches [pages, page_size, Hkv, d], page_table [B,
    max_pages], ctx_lens [B], topk [B, K]. Returns ``(o, lse)`` in float64;
    L <= 0 gives zeros and -inf.
    """
    q64 = _bf16_or_f32_to_f64(q)
    kc, vc = _bf16_or_f32_to_f64(k_cache), _bf16_or_f32_to_f64(v_cache)
    page_table = np.asarray(page_table)
    ctx_lens = np.asarray(ctx_lens)
    topk = np.asarray(topk)
    B, Hq, _ = q64.shape
    P, Hkv = kc.shape[1], kc.shape[2]
    group = Hq // Hkv
    d_v = vc.shape[3]
    o = np.zeros((B, Hq, d_v))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        L = int(ctx_lens[b])
        if L <= 0:
            continue
        j = np.arange(L)
        qb = (L - 1) // block
        window = (j // block < sink) | (j // block > qb - local)
        listed = np.zeros(L, dtype=bool)
        t = topk[b]
        listed[t[(t >= 0) & (t < L)]] = True
        toks = j[window | listed]
        pages = page_table[b, toks // P]
        slots = toks % P
        for g in range(Hkv):
            kr = kc[pages, slots, g]                       # [T, d_qk]
            vr = vc[pages, slots, g]                       # [T, d_v]
            heads = slice(g * group, (g + 1) * group)
            sc = scale * (kr @ q64[b, heads].T)            # [T, group]
            m = sc.max(axis=0)
            w = np.exp(sc - m)
            o[b, heads] = (w.T @ vr) / w.sum(axis=0)[:, None]
            lse[b, heads] = m + np.log(w.sum(axis=0))
    return o, lse


def backward(q, k, v, dout, *, block=128, sink=1, local=7, scale, full=False, rows=None):
    """Gradients of the prefill operator for the upstream gradient ``dout``.

    q [B, N, Hq, d_qk], k [B, N, Hkv, d_qk], v [B, N, Hkv, d_v], dout
    [B, N, Hq, d_v], all of one element type. Returns ``(dq, dk, dv)`` in
    float64: dq [B, R, Hq, d_qk] for the evaluated rows, dk / dv [B, N, Hkv, d]
    holding the contributions of those rows (all rows when ``rows`` is None).
    """
    lib = _load()
    elem = _elem(q)
    if _elem(k) != elem or _elem(v) != elem or _elem(dout) != elem:
        raise TypeError("q, k, v, dout must share one element type")
    B, N, Hq, d_qk = q.shape
    Bk, Nk, Hkv, d_qk2 = k.shape
    Bv, Nv, Hkv2, d_v = v.shape
    if (Bk, Nk, d_qk2) != (B, N, d_qk) or (Bv, Nv, Hkv2) != (B, N, Hkv):
        raise ValueError("shape mismatch")
    if dout.shape != (B, N, Hq, d_v):
        raise ValueError("dout shape mismatch")
    rows_arr = None
    if rows is not None:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    R = N if rows_arr is None else rows_arr.size
    dq = np.empty((B, R, Hq, d_qk), dtype=np.float64)
    dk = np.empty((B, N, Hkv, d_qk), dtype=np.float64)
    dv = np.empty((B, N, Hkv, d_v), dtype=np.float64)
    qs, ks, vs, ds = _strides(q, 3), _strides(k, 3), _strides(v, 3), _strides(dout, 3)
    rc = lib.oracle_ssa_backward(elem, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(qs), _ptr(ks),
                                 _ptr(vs), _ptr(ds), B, N, Hq, Hkv, d_qk, d_v, block, sink, local,
                                 int(full), float(scale), _ptr(rows_arr), R, _ptr(dq), _ptr(dk),
                                 _ptr(dv))
    if rc != 0:
        raise ValueError("oracle_ssa_backward rejected its arguments")
    return dq, dk, dv


def backward_keys(q, k, v, dout, keys, *, block=128, sink=1, local=7, scale):
    """dk and dv of the listed key positions, from every query row that
    attends them, without evaluating dq: the exact gradient of the prefill
    operator (softmax attention over the SSA window) restricted to those keys.

    With ``P_ij = exp(scale q_i.k_j - lse_i)`` over the attended set,
    ``D_i = dout_i . o_i`` (the forward output: ``sum_j P_ij dout_i.v_j``),
    ``dS_ij = P_ij (dout_i.v_j - D_i)``: ``dk_j = scale sum_i dS_ij q_i`` and
    ``dv_j = sum_i P_ij dout_i``, summed over the query heads of a kv head.
    lse and o come from ``prefill`` (double); the rows of a key are the
    ``i >= j`` whose window holds it (the block rule of ``prefill``).

    Returns ``(dk, dv)``: [B, len(keys), Hkv, d_qk] and [B, len(keys), Hkv,
    d_v] in float64.
    """
    keys = np.asarray(keys, dtype=np.int64)
    B, N, Hq, d_qk = q.shape
    Hkv, d_v = k.shape[2], v.shape[3]
    group = Hq // Hkv
    if keys.size and (keys.min() < 0 or keys.max() >= N):
        raise ValueError("key positions must lie in [0, N)")
    i0 = int(keys.min()) if keys.size else N
    rows = np.arange(i0, N)
    o, lse, _ = prefill(q, k, v, block=block, sink=sink, local=local, scale=scale, rows=rows)
    i = rows[:, None]
    j = keys[None, :]
    mask = (j <= i) & ((j // block < sink) | (j // block > i // block - local))
    dk = np.zeros((B, keys.size, Hkv, d_qk))
    dv = np.zeros((B, keys.size, Hkv, d_v))
    for b in range(B):
        for g in range(Hkv):
            kj = _bf16_or_f32_to_f64(k[b, keys, g])                 # [K, d_qk]
            vj = _bf16_or_f32_to_f64(v[b, keys, g])                 # [K, d_v]
            for h in range(g * group, (g + 1) * group):
                qi = _bf16_or_f32_to_f64(q[b, rows, h])             # [R, d_qk]
                doi = _bf16_or_f32_to_f64(dout[b, rows, h])         # [R, d_v]
                p = np.where(mask, np.exp(scale * (qi @ kj.T) - lse[b, h][:, None]), 0.0)
                dd = np.einsum("rd,rd->r", doi, o[b, :, h])
                ds = p * (doi @ vj.T - dd[:, None])
                dk[b, :, g] += scale * (ds.T @ qi)
                dv[b, :, g] += p.T @ doi
    return dk, dv
