"""Streaming sparse attention (SSA) for AMD Instinct MI355X (gfx950).

The compute lives in ``libssa.so`` (hand-written HIP kernels behind the C ABI
declared in ``include/ssa.h``); this package is its thin ctypes binding plus
the seeded input generators used by the tests and the benchmark.

    prefill(q, k, v, block=128, sink=1, local=7)      -> ssa_prefill
    prefill_dual(q, k, v, alpha=...)                   -> ssa_prefill_dual
    prefill_backward(q, k, v, o, lse, dout)            -> ssa_prefill_backward
    decode(q, k_cache, v_cache, page_table, ctx_lens)  -> ssa_decode
    decode_noalloc(q, k_cache, v_cache, page_table, ctx_lens)  -> ssa_decode_noalloc
    extend(q, k_cache, v_cache, page_table, ctx_lens, cu_q, max_q_len) -> ssa_extend
    hybrid_decode(q, k_cache, v_cache, page_table, ctx_lens, topk)     -> hybrid_decode
    full_decode(...)                                   -> full_attn_decode
"""
from ._binding import (EXPORTS, LIB_PATH, SSA_BF16, SSA_F32, Pattern, SSAError,
                       backward_workspace_size, decode, decode_noalloc, decode_workspace_size, extend,
                       extend_workspace_size, full_decode, hybrid_decode,
                       hybrid_decode_workspace_size,
                       load_library, prefill, prefill_backward, prefill_dual, status_string)

__all__ = ["prefill", "prefill_dual", "prefill_backward", "backward_workspace_size", "decode", "decode_noalloc",
           "full_decode", "decode_workspace_size", "extend", "extend_workspace_size",
           "hybrid_decode", "hybrid_decode_workspace_size", "load_library", "status_string", "SSAError",
           "Pattern", "EXPORTS", "LIB_PATH", "SSA_F32", "SSA_BF16"]
