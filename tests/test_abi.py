"""The C ABI on the host: the library loads, exports what include/ssa.h
declares, and rejects bad arguments before launching anything (every call
here fails validation or is a no-op, so no GPU is needed)."""
import ctypes
import math
import os
import re

import pytest
import torch

import block_sparse_streaming_amd as ssa

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "ssa.h")
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = 0x10000  # aligned, never dereferenced: validation fails before any launch


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(?:ssa_status|size_t|const char \*)\s*\*?\s*(\w+)\s*\(", text))


def test_exports_match_header():
    lib = ssa.load_library()
    declared = declared_functions()
    assert declared == set(ssa.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    for code, prefix in [(0, "SSA_OK"), (1, "SSA_ERR_INVALID_ARG"), (2, "SSA_ERR_UNSUPPORTED"),
                         (3, "SSA_ERR_WORKSPACE"), (4, "SSA_ERR_HIP")]:
        assert ssa.status_string(code).startswith(prefix)
    assert "unknown" in ssa.status_string(99)


def strides(*s):
    return (ctypes.c_int64 * 3)(*s)


def prefill_call(dtype=1, B=1, N=256, Hq=4, Hkv=4, dqk=128, dv=128, pattern=(128, 1, 7),
                 scale=0.1, ptr=FAKE, qs=None, lse=None):
    lib = ssa.load_library()
    st = qs or strides(N * Hq * dqk, Hq * dqk, dqk)
    p = ctypes.c_void_p(ptr) if ptr is not None else None
    return lib.ssa_prefill(dtype, p, p, p, p, lse, B, N, Hq, Hkv, dqk, dv, st, st, st, st,
                           ssa.Pattern(*pattern), scale, None)


def test_prefill_validation():
    assert prefill_call(dtype=7) == INVALID
    assert prefill_call(B=-1) == INVALID
    assert prefill_call(Hq=4, Hkv=3) == INVALID
    assert prefill_call(pattern=(128, 1, 0)) == INVALID     # l = 0 leaves rows empty
    assert prefill_call(pattern=(0, 1, 7)) == INVALID
    assert prefill_call(pattern=(128, -1, 7)) == INVALID
    assert prefill_call(scale=math.nan) == INVALID
    assert prefill_call(scale=math.inf) == INVALID
    assert prefill_call(scale=0.0) == INVALID
    assert prefill_call(scale=-0.1) == INVALID
    assert prefill_call(ptr=None) == INVALID
    assert prefill_call(ptr=FAKE + 2) == INVALID             # misaligned rows
    assert prefill_call(qs=strides(1024, 3, 1)) == INVALID  # stride not 16-byte aligned
    assert prefill_call(qs=strides(-8, 8, 8)) == INVALID
    assert prefill_call(dqk=96, dv=96) == UNSUPPORTED
    assert prefill_call(dtype=0, dqk=192, dv=128) == UNSUPPORTED
    # empty problems are no-ops and launch nothing
    assert prefill_call(B=0, ptr=None) == OK
    assert prefill_call(N=0, ptr=None) == OK


def decode_call(full=False, dtype=1, B=2, Hq=4, Hkv=4, dqk=128, dv=128, ps=128, max_pages=8,
                pattern=(128, 1, 7), ws_bytes=1 << 30, ptr=FAKE, vptr=None, vs=None):
    lib = ssa.load_library()
    ks = strides(ps * Hkv * dqk, Hkv * dqk, dqk)
    vst = vs or ks
    p = ctypes.c_void_p(ptr) if ptr is not None else None
    vp = ctypes.c_void_p(vptr) if vptr is not None else p
    args = [dtype, p, p, vp, ks, vst, p, max_pages, p, B, Hq, Hkv, dqk, dv, ps, p, None, p, ws_bytes]
    if full:
        return lib.full_attn_decode(*args, 0.1, None)
    return lib.ssa_decode(*args, ssa.Pattern(*pattern), 0.1, None)


def noalloc_call(dtype=1, B=2, Hq=4, Hkv=4, dqk=128, dv=128, ps=128, max_pages=8, pattern=(128, 1, 7),
                 ptr=FAKE):
    lib = ssa.load_library()
    ks = strides(ps * Hkv * dqk, Hkv * dqk, dqk)
    p = ctypes.c_void_p(ptr) if ptr is not None else None
    return lib.ssa_decode_noalloc(dtype, p, p, p, ks, ks, p, max_pages, p, B, Hq, Hkv, dqk, dv, ps, p, None,
                                  ssa.Pattern(*pattern), 0.1, None)


def test_decode_noalloc_validation():
    """The no-allocation decode checks its arguments like ssa_decode, on the
    host, before any HIP call (these run without a GPU), and rejects a call
    whose workspace would not fit its fixed 32 MiB scratch."""
    assert noalloc_call(dtype=3) == INVALID
    assert noalloc_call(Hq=6, Hkv=4) == INVALID
    assert noalloc_call(ptr=None) == INVALID
    assert noalloc_call(pattern=(128, 1, 0)) == INVALID
    assert noalloc_call(dqk=96, dv=96) == UNSUPPORTED
    assert noalloc_call(B=0, ptr=None) == OK
    # 200 sequences x 64 heads, d = 128: 8 splits of fp32 partials, 52 MB
    assert ssa.decode_workspace_size(torch.bfloat16, 200, 64, 64, 128, 128, 128, 8) > 32 << 20
    assert noalloc_call(B=200, Hq=64, Hkv=64) == WORKSPACE
    # 8,192-token window, 2 kv heads: 64 splits, 105 MB
    big = dict(B=200, Hq=16, Hkv=2, max_pages=64, pattern=(128, 1, 63))
    assert ssa.decode_workspace_size(torch.bfloat16, 200, 16, 2, 128, 128, 128, 64, block=128, sink=1,
                                     local=63) > 32 << 20
    assert noalloc_call(**big) == WORKSPACE


@pytest.mark.parametrize("full", [False, True])
def test_decode_validation(full):
    assert decode_call(full, dtype=3) == INVALID
    assert decode_call(full, Hq=6, Hkv=4) == INVALID
    assert decode_call(full, ps=0) == INVALID
    assert decode_call(full, max_pages=0) == INVALID
    assert decode_call(full, ptr=None) == INVALID
    assert decode_call(full, ptr=FAKE + 4) == INVALID
    assert decode_call(full, dqk=96, dv=96) == UNSUPPORTED
    assert decode_call(full, Hq=48, Hkv=4) == UNSUPPORTED     # group of 12
    assert decode_call(full, dtype=0, dqk=576, dv=512, Hq=64, Hkv=1) == UNSUPPORTED
    # the latent kernel needs v_cache to alias k_cache
    assert decode_call(full, dqk=576, dv=512, Hq=64, Hkv=1, vptr=FAKE + 4096) == UNSUPPORTED
    assert decode_call(full, ws_bytes=16) == WORKSPACE
    assert decode_call(full, B=0, ptr=None) == OK
    if not full:
        assert decode_call(pattern=(128, 1, 0)) == INVALID


def test_workspace_sizes():
    import torch
    ws = ssa.decode_workspace_size
    # windowed latent decode: (s + l) * b / 128 tokens per split = 8 splits,
    # each a bf16 partial output of d_v values and an fp32 lse
    slots = 32 * 64 * 8
    need = ws(torch.bfloat16, 32, 64, 1, 576, 512, 128, 1024)
    lse_off = -(-slots * 512 * 2 // 256) * 256
    assert need == lse_off + slots * 4
    # short caches bound the window: max_pages * page_size = 256 tokens -> 2 splits
    assert ws(torch.bfloat16, 1, 16, 16, 128, 128, 128, 2) == -(-16 * 2 * 128 * 4 // 256) * 256 + 16 * 2 * 4
    # full decode grows with the context
    assert ws(torch.bfloat16, 32, 64, 1, 576, 512, 128, 1024, full=True) > need
    # latent full decode with 2-token pages: the split is capped at 480 tokens
    # (at most (480 - 2) // 2 + 4 = 243 pages), so 262144 tokens need 547 splits
    slots = 4 * 64 * 547
    assert ws(torch.bfloat16, 4, 64, 1, 576, 512, 2, 131072, full=True) == \
        -(-slots * 512 * 2 // 256) * 256 + slots * 4
    # full decode with many (sequence, head) rows: splits stay at most 8,192
    # tokens, so a 1M-token context is cut into 128 splits per row instead of
    # one work-group walking all of it
    slots = 65 * 16 * 128
    assert ws(torch.bfloat16, 65, 16, 16, 128, 128, 128, 8192, full=True) == \
        -(-slots * 128 * 4 // 256) * 256 + slots * 4
    assert ws(torch.bfloat16, 1, 4, 3, 128, 128, 128, 8) == 0          # invalid heads
    assert ws(torch.bfloat16, 1, 4, 4, 128, 128, 128, 8, local=0) == 0


def backward_call(dtype=1, B=1, N=256, Hq=4, Hkv=4, dqk=128, dv=128, pattern=(128, 1, 7),
                  scale=0.1, ptr=FAKE, lse=FAKE, ws_bytes=1 << 30, st=None):
    lib = ssa.load_library()
    s = st or strides(N * Hq * dqk, Hq * dqk, dqk)
    p = ctypes.c_void_p(ptr) if ptr is not None else None
    lp = ctypes.c_void_p(lse) if lse is not None else None
    return lib.ssa_prefill_backward(dtype, p, p, p, p, lp, p, p, p, p, B, N, Hq, Hkv, dqk, dv,
                                    s, s, s, s, s, s, s, s, p, ws_bytes,
                                    ssa.Pattern(*pattern), scale, None)


def test_backward_validation():
    assert backward_call(dtype=5) == INVALID
    assert backward_call(Hq=4, Hkv=3) == INVALID
    assert backward_call(pattern=(128, 1, 0)) == INVALID
    assert backward_call(scale=math.nan) == INVALID
    assert backward_call(ptr=None) == INVALID
    assert backward_call(lse=None) == INVALID                 # the forward's lse is required
    assert backward_call(ptr=FAKE + 2) == INVALID
    assert backward_call(st=strides(1024, 3, 1)) == INVALID
    assert backward_call(dtype=0) == UNSUPPORTED              # fp32 backward is not compiled
    assert backward_call(dqk=96, dv=96) == UNSUPPORTED
    assert backward_call(ws_bytes=64) == WORKSPACE
    assert backward_call(B=0, ptr=None, lse=None) == OK
    assert backward_call(N=0, ptr=None, lse=None) == OK


def test_backward_workspace_sizes():
    import torch
    ws = ssa.backward_workspace_size
    # 32K tokens, 16 heads, b=128 s=1 l=7: row statistics (2 floats per row and
    # head) + partial sums of the 128 sink keys over ceil(32768 / 3584) = 10
    # chunks of 4 * 7 * 128 rows.
    rowstat = 16 * 32768 * 2 * 4
    part = 10 * 16 * 128 * (128 + 128) * 4
    assert ws(torch.bfloat16, 1, 32768, 16, 16, 128, 128) == rowstat + part
    # no sink: row statistics only, rows padded to 128
    assert ws(torch.bfloat16, 2, 1000, 4, 2, 64, 64, sink=0, local=3) == 2 * 4 * 1024 * 2 * 4
    # short sequence: one chunk (rows padded to 128), sink keys clamped to N
    assert ws(torch.bfloat16, 1, 100, 2, 2, 192, 128) == -(-2 * 128 * 2 * 4 // 256) * 256 + \
        1 * 2 * 100 * 320 * 4
    assert ws(torch.float32, 1, 100, 2, 2, 128, 128) == 0    # not compiled
    assert ws(torch.bfloat16, 1, 100, 3, 2, 128, 128) == 0   # invalid heads


def dual_call(dtype=1, B=1, N=256, Hq=4, Hkv=4, dqk=128, dv=128, pattern=(128, 1, 7), scale=0.1,
              alpha=0.5, o_ssa=FAKE, o_full=FAKE + 0x1000, o_mix=FAKE + 0x2000):
    lib = ssa.load_library()
    st = strides(N * Hq * dqk, Hq * dqk, dqk)
    p = ctypes.c_void_p(FAKE)
    vp = lambda x: ctypes.c_void_p(x) if x is not None else None  # noqa: E731
    return lib.ssa_prefill_dual(dtype, p, p, p, vp(o_ssa), None, vp(o_full), None, vp(o_mix), alpha,
                                B, N, Hq, Hkv, dqk, dv, st, st, st, st, ssa.Pattern(*pattern),
                                scale, None)


def test_dual_validation():
    assert dual_call(alpha=-0.01) == INVALID
    assert dual_call(alpha=1.01) == INVALID
    assert dual_call(alpha=math.nan) == INVALID
    assert dual_call(pattern=(128, 1, 0)) == INVALID
    assert dual_call(scale=-1.0) == INVALID
    assert dual_call(o_full=None) == INVALID               # the full output is required
    assert dual_call(o_full=FAKE) == INVALID               # same buffer as o_ssa
    assert dual_call(o_mix=FAKE + 0x1000) == INVALID       # same buffer as o_full
    assert dual_call(o_full=FAKE + 0x1008) == INVALID      # misaligned
    assert dual_call(dtype=0) == UNSUPPORTED                # fp32 has no dual kernel
    assert dual_call(dqk=96, dv=96) == UNSUPPORTED
    assert dual_call(N=0) == OK and dual_call(B=0) == OK   # no-op


def extend_call(dtype=1, B=2, total_q=2, max_q=1, Hq=4, Hkv=4, dqk=128, dv=128, ps=128, max_pages=8,
                pattern=(128, 1, 7), ws_bytes=1 << 30, ptr=FAKE, scale=0.1):
    lib = ssa.load_library()
    ks = strides(ps * Hkv * dqk, Hkv * dqk, dqk)
    p = ctypes.c_void_p(ptr) if ptr is not None else None
    return lib.ssa_extend(dtype, p, p, p, ks, ks, p, max_pages, p, p, B, total_q, max_q, Hq, Hkv, dqk,
                          dv, ps, p, None, p, ws_bytes, ssa.Pattern(*pattern), scale, None)


def test_extend_validation():
    assert extend_call(dtype=5) == INVALID
    assert extend_call(B=-1) == INVALID
    assert extend_call(total_q=-1) == INVALID
    assert extend_call(max_q=0) == INVALID                  # rows exist, so some chunk is >= 1
    assert extend_call(Hq=4, Hkv=3) == INVALID
    assert extend_call(pattern=(128, 1, 0)) == INVALID
    assert extend_call(ps=0) == INVALID
    assert extend_call(scale=0.0) == INVALID
    assert extend_call(ptr=None) == INVALID
    assert extend_call(ptr=FAKE + 4) == INVALID
    assert extend_call(dqk=96, dv=96) == UNSUPPORTED
    assert extend_call(ws_bytes=0) == WORKSPACE             # one-row chunks: decode kernels need scratch
    assert extend_call(B=0, ptr=None) == OK and extend_call(total_q=0, max_q=0, ptr=None) == OK


def test_extend_workspace_sizes():
    lib = ssa.load_library()
    pat = ssa.Pattern(128, 1, 7)
    # one-row chunks on a decode shape: row map + decode partials
    short = lib.ssa_extend_workspace_size(1, 6, 6, 1, 4, 4, 128, 128, 128, 8, pat)
    dec = lib.ssa_decode_workspace_size(1, 6, 4, 4, 128, 128, 128, 8, pat, 0)
    assert short == 256 + dec
    # two or more rows take the tile kernel: no workspace
    assert lib.ssa_extend_workspace_size(1, 2, 4, 2, 4, 4, 128, 128, 128, 8, pat) == 0
    assert lib.ssa_extend_workspace_size(1, 2, 600, 500, 4, 4, 128, 128, 128, 8, pat) == 0
    # d_qk = 192 has no decode kernel: tiles even for one-row chunks
    assert lib.ssa_extend_workspace_size(1, 2, 2, 1, 4, 4, 192, 128, 128, 8, pat) == 0
    # d = 256 has no tile kernel: decode kernels for any chunk
    assert lib.ssa_extend_workspace_size(1, 2, 8, 4, 4, 4, 256, 256, 128, 8, pat) > 0
    # fp32 has no tile kernel: decode kernels even for long chunks
    assert lib.ssa_extend_workspace_size(0, 2, 600, 500, 4, 4, 128, 128, 128, 8, pat) > 0
    assert lib.ssa_extend_workspace_size(1, 0, 6, 4, 4, 4, 128, 128, 128, 8, pat) == 0
