#!/usr/bin/env python3
"""Benchmark of the streaming sparse attention hot path on one MI355X.

Headline (one JSON line on stdout): ssa_prefill throughput in TFLOP/s on the
32K-token bf16 workload (B=1, N=32768, 16 heads, d=128, b=128, s=1, l=7),
counted as algorithmic flops 2*(d_qk + d_v) per attended (query, key) pair.
The same line carries the other workloads of the metric: prefill at 2K (fp32)
and 256K tokens, SSA and full-attention decode on the 128K-context latent
workload and SSA decode on the ragged 4K-1M workload (HBM GB/s of algorithmic
bytes), the prefill backward at 32K and 256K tokens (TFLOP/s), the dual
forward (SSA, full causal attention and their alpha-mix in one pass) at 32K
(TFLOP/s of full causal attention), chunked prefill and multi-token decode
against the paged cache (TFLOP/s; GB/s), hybrid decode over the window and
a list of 1,024 tokens (GB/s), each against its roofline, and the CPU oracle
timed on the prefill.

Inputs are synthetic (seeded N(0,1)) and resident in HBM before timing.
Timing uses HIP events recorded on the stream the kernels are launched on
(torch's current stream, which the binding passes to the library).

--profile {prefill,prefill_fp32,prefill_256k,decode,backward,backward_256k,dual,extend,hybrid,copy}
runs one short workload and prints nothing
else, for rocprofv3 counter collection (copy: a plain 1 GiB device copy whose
counter readings calibrate FETCH_SIZE / WRITE_SIZE).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SSA prefill TFLOP/s + decode HBM GB/s (b=128,s=1,l=7) at 32K–256K ctx"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3      # MI355X fp32 matrix / vector
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def attended_pairs(N: int, block: int, sink: int, local: int) -> int:
    """Number of (query, key) pairs of one head: sum over rows of |A(i)|."""
    i = np.arange(N, dtype=np.int64)
    sb = sink * block
    a1 = np.minimum(sb, i + 1)
    lo = np.maximum(sb, (i // block - local + 1) * block)
    return int((a1 + np.maximum(0, i + 1 - lo)).sum())


def decode_selected_tokens(L: int, block: int, sink: int, local: int) -> int:
    if L <= 0:
        return 0
    sb = sink * block
    lo = max(sb, ((L - 1) // block - local + 1) * block)
    return min(sb, L) + max(0, L - lo)


SETTLE_S = [0.5]   # seconds of untimed back-to-back calls before each timed region (--settle)


def settle(fn, seconds: float) -> None:
    """Run fn() back to back, untimed, for about `seconds` of wall-clock time.
    After an idle or a lighter phase the GPU's clocks take tens of milliseconds
    of sustained load to reach their steady state (the 32K prefill runs its
    first ~30 launches at ~0.35 ms, then ~0.29 ms); a timed region that starts
    earlier measures that ramp instead of the kernel."""
    import torch
    if seconds <= 0:
        return
    t0 = time.perf_counter()
    n = 1
    while True:
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return
        n = min(2 * n, 64)


def time_events(fn, iters: int) -> float:
    """Average milliseconds of fn() over iters back-to-back calls, by HIP events
    on the current stream, synchronised before and after; the calls are timed
    after settle(fn)."""
    import torch
    settle(fn, SETTLE_S[0])
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(iters):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / iters


def recorded_traffic(keys: list[str]):
    """HBM bytes per launch measured by rocprofv3 FETCH_SIZE / WRITE_SIZE runs
    (copy-calibrated) and stored in profiles/traffic.json, summed over `keys`;
    None when a kernel has no record or its sources changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    total = 0.0
    for key in keys:
        entry = data.get(key)
        if entry is None:
            return None
        h = hashlib.sha256()
        for name in entry["sources"]:
            with open(os.path.join(ROOT, "block_sparse_streaming_amd", "csrc", name), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != entry["source_sha256"]:
            return None
        total += entry["bytes_per_launch"]
    return total


MEASURED = {}   # attainable ceilings measured on this GPU at start-up (see measure_ceilings)


def measure_ceilings():
    """What this GPU sustains right now through vendor libraries, as a second
    reference beside the published peaks: a 16384^3 bf16 GEMM (hipBLASLt) for
    the matrix cores, and a memory-bound skinny GEMM reading a 4 GiB operand
    for HBM (2 * 4 GiB / time counts the operand only)."""
    import torch
    dev = "cuda:0"
    n = 16384
    a = torch.randn(n, n, device=dev).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev).to(torch.bfloat16)
    for _ in range(2):
        torch.mm(a, b)
    ms = time_events(lambda: torch.mm(a, b), 5)
    gemm = 2 * n ** 3 / (ms * 1e-3) / 1e12
    del a, b
    x = torch.ones((1 << 18, 1 << 13), dtype=torch.bfloat16, device=dev)   # 4 GiB
    w = torch.ones((1 << 13, 16), dtype=torch.bfloat16, device=dev)
    for _ in range(2):
        torch.mm(x, w)
    ms = time_events(lambda: torch.mm(x, w), 10)
    hbm = x.numel() * 2 / (ms * 1e-3) / 1e9
    del x, w
    free_gpu()
    MEASURED.update({"bf16_gemm_tflops": gemm, "hbm_read_gbs": hbm,
                     "how": "torch.mm bf16 16384^3 (hipBLASLt); torch.mm [262144x8192]x[8192x16] bf16, "
                            "operand bytes / time"})
    return MEASURED


TRAFFIC_SOURCE = ("recorded, not measured in this run: profiles/traffic.json, HBM bytes per launch from "
                  "rocprofv3 FETCH_SIZE and WRITE_SIZE runs (copy-calibrated), kept only while the "
                  "kernel's sources hash to the recorded SHA-256")


def with_measured(roof: dict) -> dict:
    roof["traffic_source"] = TRAFFIC_SOURCE if roof.get("traffic") is not None else None
    key = "bf16_gemm_tflops" if roof["unit"] == "TFLOP/s" else "hbm_read_gbs"
    if key in MEASURED and not (roof["unit"] == "TFLOP/s" and roof["peak"] != PEAK_BF16_TFLOPS):
        roof["measured_peak"] = MEASURED[key]
        roof["frac_of_measured"] = roof["achieved"] / MEASURED[key]
    return roof


def free_gpu():
    import gc
    import torch
    gc.collect()
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# Prefill
# ---------------------------------------------------------------------------
def prefill_setup(cfg):
    import torch
    import block_sparse_streaming_amd as ssa
    from block_sparse_streaming_amd import inputs

    q, k, v = inputs.prefill_inputs(cfg, "cuda:0")
    out = torch.empty((cfg.B, cfg.N, cfg.Hq, cfg.d_v), dtype=cfg.dtype, device="cuda:0")

    def step():
        ssa.prefill(q, k, v, **inputs.PATTERN, scale=cfg.scale, out=out)

    return cfg, step


def bench_prefill(cfg, steps: int, warmup: int):
    import torch
    from block_sparse_streaming_amd import inputs

    cfg, step = prefill_setup(cfg)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ms = time_events(step, steps)
    pairs = attended_pairs(cfg.N, **inputs.PATTERN) * cfg.Hq * cfg.B
    flops = pairs * 2 * (cfg.d_qk + cfg.d_v)
    tflops = flops / (ms * 1e-3) / 1e12
    bf16 = cfg.dtype == torch.bfloat16
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_FP32_TFLOPS
    kernel = (f"ssa_prefill_bf16<{cfg.d_qk}, {cfg.d_v}, 0>" if bf16 else
              f"ssa_prefill_f32<{cfg.d_qk}, {cfg.d_v}>")
    if bf16:
        grid = -(-cfg.N // 128) * cfg.Hq * cfg.B * 256      # 128-row tiles, 4 waves
    else:
        grid = -(-cfg.N // 32) * cfg.Hq * cfg.B * 64 * (8 if cfg.d_qk <= 64 else 4)   # 32-row tiles
    res = {"workload": cfg.name, "ms": ms, "steps": steps, "algorithmic_flops": flops,
           "TFLOP/s": tflops,
           "roofline": with_measured({"bound": "mfma", "achieved": tflops, "peak": peak, "unit": "TFLOP/s",
                                      "frac": tflops / peak,
                                      "traffic": recorded_traffic([f"{kernel} grid={grid}"])})}
    del step
    free_gpu()
    return cfg, res


# ---------------------------------------------------------------------------
# Dual forward (SSA + full causal attention + alpha-mix, one pass)
# ---------------------------------------------------------------------------
DUAL_ALPHA = 0.5


def dual_setup(cfg):
    import torch
    import block_sparse_streaming_amd as ssa
    from block_sparse_streaming_amd import inputs

    q, k, v = inputs.prefill_inputs(cfg, "cuda:0")
    outs = tuple(torch.empty((cfg.B, cfg.N, cfg.Hq, cfg.d_v), dtype=cfg.dtype, device="cuda:0")
                 for _ in range(3))

    def step():
        ssa.prefill_dual(q, k, v, **inputs.PATTERN, scale=cfg.scale, alpha=DUAL_ALPHA, out=outs)

    return cfg, step


def bench_dual(cfg, steps: int, warmup: int):
    """ssa_prefill_dual: the SSA output, the full causal output and their mix
    in one launch. Its work is that of full causal attention: N(N+1)/2 pairs
    per head at 2 (d_qk + d_v) flops each."""
    import torch
    cfg, step = dual_setup(cfg)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ms = time_events(step, steps)
    flops = cfg.N * (cfg.N + 1) // 2 * cfg.Hq * cfg.B * 2 * (cfg.d_qk + cfg.d_v)
    tflops = flops / (ms * 1e-3) / 1e12
    grid = -(-cfg.N // 128) * cfg.Hq * cfg.B * 256
    kernel = f"ssa_prefill_bf16<{cfg.d_qk}, {cfg.d_v}, 1>"
    name = cfg.name.replace("prefill", "prefill_dual", 1)
    res = {"workload": name, "ms": ms, "steps": steps, "algorithmic_flops": flops, "TFLOP/s": tflops,
           "alpha": DUAL_ALPHA,
           "roofline": with_measured({"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS,
                                      "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_TFLOPS,
                                      "traffic": recorded_traffic([f"{kernel} grid={grid}"])})}
    del step
    free_gpu()
    return name, res


# ---------------------------------------------------------------------------
# Extend: new tokens against the paged cache (chunked prefill, multi-token decode)
# ---------------------------------------------------------------------------
def extend_row_counts(lens, qlens, block: int, sink: int, local: int) -> np.ndarray:
    """|A(p)| of every new row (position p = L - q_len + r), concatenated."""
    out = []
    sb = sink * block
    for L, n in zip(lens, qlens):
        p = np.arange(L - n, L, dtype=np.int64)
        lo = np.maximum(sb, (p // block - local + 1) * block)
        out.append(np.minimum(sb, p + 1) + np.maximum(0, p + 1 - lo))
    return np.concatenate(out) if out else np.zeros(0, np.int64)


def extend_union_tokens(L: int, n: int, block: int, sink: int, local: int) -> int:
    """Cache rows some new row of a sequence attends: the sink blocks and
    [lo(first new position), L)."""
    sb = sink * block
    p0 = L - n
    lo = max(sb, (p0 // block - local + 1) * block)
    return min(sb, L) + max(0, L - lo)


def extend_chunk_setup():
    import torch
    import block_sparse_streaming_amd as ssa
    from block_sparse_streaming_amd import inputs

    lens, qlens = inputs.EXTEND_CHUNK_LENS, inputs.EXTEND_CHUNK_QLENS
    inp = inputs.extend_inputs(lens, qlens, 16, 16, 128, 128, torch.bfloat16, "cuda:0",
                               inputs.EXTEND_SEED)
    out = torch.empty((sum(qlens), 16, 128), dtype=torch.bfloat16, device="cuda:0")
    mq = max(qlens)

    def step():
        ssa.extend(inp.q, inp.k_cache, inp.v_cache, inp.page_table, inp.ctx_lens, inp.cu_q, mq,
                   **inputs.PATTERN, out=out)

    return inp, step


def bench_extend_chunk(steps: int, warmup: int):
    """ssa_extend on the chunked-prefill workload (paged tile kernel): four
    sequences at 32K-128K tokens of context, each appending 8,192 tokens."""
    import torch
    from block_sparse_streaming_amd import inputs
    inp, step = extend_chunk_setup()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ms = time_events(step, steps)
    H, d = 16, 128
    pairs = int(extend_row_counts(inp.lens, inp.qlens, **inputs.PATTERN).sum()) * H
    flops = pairs * 2 * (d + d)
    tflops = flops / (ms * 1e-3) / 1e12
    grid = -(-max(inp.qlens) // 128) * H * len(inp.lens) * 256
    name = "extend_chunk_bf16_b4_ctx32k-128k_q8192_h16_d128"
    res = {"workload": name, "ms": ms, "steps": steps, "algorithmic_flops": flops, "TFLOP/s": tflops,
           "roofline": with_measured({"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS,
                                      "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_TFLOPS,
                                      "traffic": recorded_traffic(
                                          [f"ssa_prefill_bf16<128, 128, 2> grid={grid}"])})}
    del inp, step
    free_gpu()
    return name, res


def extend_mtp_setup(n_inst: int):
    """The multi-token decode workload, with n_inst page-table / query
    instances over one cache (their selected pages together exceed the
    Infinity Cache)."""
    import torch
    from block_sparse_streaming_amd import inputs
    B, T = 32, inputs.EXTEND_MTP_Q
    lens, qlens = (inputs.EXTEND_MTP_LEN,) * B, (T,) * B
    base = inputs.extend_inputs(lens, qlens, 64, 1, 576, 512, torch.bfloat16, "cuda:0",
                                inputs.EXTEND_MTP_SEED, latent=True)
    insts = []
    for r in range(n_inst):
        table, _ = inputs.page_table_for(lens, inputs.PAGE_SIZE, seed=inputs.EXTEND_MTP_SEED + 100 + r)
        g = inputs.generator("cuda:0", inputs.EXTEND_MTP_SEED + 200 + r)
        qr = inputs.randn(tuple(base.q.shape), torch.bfloat16, "cuda:0", g)
        insts.append((qr, torch.from_numpy(table).to("cuda:0")))
    return base, insts


def bench_extend_mtp(iters: int):
    """ssa_extend on the multi-token decode workload (decode kernels over
    query rows): 32 sequences at 128K tokens, four new tokens each, 64 query
    heads on one 576-wide latent head. Rotates over 8 instances and replays a
    HIP graph, as the latent decode measurement does."""
    import torch
    import block_sparse_streaming_amd as ssa
    from block_sparse_streaming_amd import inputs
    n_inst = 8
    base, insts = extend_mtp_setup(n_inst)
    B, T, Hq = len(base.lens), inputs.EXTEND_MTP_Q, 64
    rows = B * T
    max_pages = base.page_table.shape[1]
    ws = torch.empty(max(16, ssa.extend_workspace_size(torch.bfloat16, B, rows, T, Hq, 1, 576, 512,
                                                       inputs.PAGE_SIZE, max_pages, **inputs.PATTERN)),
                     dtype=torch.uint8, device="cuda:0")
    outs = [torch.empty((rows, Hq, 512), dtype=torch.bfloat16, device="cuda:0") for _ in range(n_inst)]

    def call(r):
        qr, tr = insts[r]
        ssa.extend(qr, base.k_cache, base.v_cache, tr, base.ctx_lens, base.cu_q, T, **inputs.PATTERN,
                   scale=576 ** -0.5, out=outs[r], workspace=ws)

    for r in range(n_inst):
        call(r)
    torch.cuda.synchronize()
    reps = 4
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            for _ in range(reps):
                for r in range(n_inst):
                    call(r)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    ms = time_events(graph.replay, max(1, iters // (reps * n_inst))) / (reps * n_inst)
    # Algorithmic bytes: the union of the rows' attended latent rows (each read
    # once), q and o, the page ids of those rows and the lengths.
    union = [extend_union_tokens(L, T, **inputs.PATTERN) for L in base.lens]
    nbytes = (sum(union) * 576 * 2 + rows * Hq * (576 + 512) * 2 +
              sum(-(-u // inputs.PAGE_SIZE) for u in union) * 4 + (2 * B + 1) * 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    name = "extend_mtp_bf16_latent_b32_q4_h64_d576_L131072"
    res = {"workload": name, "us": ms * 1e3, "bytes": nbytes, "GB/s": gbs,
           "rows_per_call": rows,
           "roofline": decode_roofline(gbs, ["extend_rows mtp", "decode_split_latent mtp",
                                             "decode_merge<true, 512> mtp"]),
           "timing": f"HIP graph of {reps * n_inst} calls rotating over {n_inst} instances"}
    del graph, insts, outs, base, ws
    free_gpu()
    return name, res


# ---------------------------------------------------------------------------
# Hybrid decode: SSA window plus listed tokens
# ---------------------------------------------------------------------------
def hybrid_setup(n_inst: int):
    """The hybrid decode workload: the latent decode shape (32 sequences at
    128K, 64 heads) with 16 sink tokens, a 1,024-token window and 1,024 listed
    tokens; n_inst page-table / query / list instances over one cache."""
    import torch
    from block_sparse_streaming_amd import inputs
    B = 32
    lens = (inputs.EXTEND_MTP_LEN,) * B
    base = inputs.extend_inputs(lens, (1,) * B, 64, 1, 576, 512, torch.bfloat16, "cuda:0",
                                inputs.HYBRID_SEED, latent=True)
    insts = []
    for r in range(n_inst):
        table, _ = inputs.page_table_for(lens, inputs.PAGE_SIZE, seed=inputs.HYBRID_SEED + 100 + r)
        g = inputs.generator("cuda:0", inputs.HYBRID_SEED + 200 + r)
        qr = inputs.randn(tuple(base.q.shape), torch.bfloat16, "cuda:0", g)
        lst = inputs.token_lists(lens, inputs.HYBRID_K, inputs.HYBRID_SEED + 300 + r)
        insts.append((qr, torch.from_numpy(table).to("cuda:0"), torch.from_numpy(lst).to("cuda:0"), lst))
    return base, insts


def hybrid_bytes(lens, lists, block: int, sink: int, local: int, page_size: int, Hq: int) -> int:
    """Algorithmic bytes of one hybrid call: the latent rows of the window and
    of the listed tokens outside it (each once), q, o, the page ids of the
    window's pages and of the listed rows, the lists and the lengths."""
    rows = 0
    pids = 0
    for L, lst in zip(lens, lists):
        j = np.arange(L)
        win = (j // block < sink) | (j // block > (L - 1) // block - local)
        extra = np.setdiff1d(lst[(lst >= 0) & (lst < L)], j[win])
        rows += int(win.sum()) + extra.size
        pids += np.unique(j[win] // page_size).size + extra.size
    B = len(lens)
    return (rows * 576 * 2 + B * Hq * (576 + 512) * 2 + pids * 4 + sum(len(x) for x in lists) * 4 +
            B * 4)


def bench_hybrid(iters: int):
    """hybrid_decode on the hybrid workload, rotating over 8 instances and
    replayed from a HIP graph, as the latent decode measurement does."""
    import torch
    import block_sparse_streaming_amd as ssa
    from block_sparse_streaming_amd import inputs
    n_inst = 8
    base, insts = hybrid_setup(n_inst)
    B, Hq = len(base.lens), 64
    pat = inputs.HYBRID_PATTERN
    max_pages = base.page_table.shape[1]
    ws = torch.empty(ssa.hybrid_decode_workspace_size(torch.bfloat16, B, Hq, 1, 576, 512, inputs.PAGE_SIZE,
                                                      max_pages, inputs.HYBRID_K, **pat),
                     dtype=torch.uint8, device="cuda:0")
    outs = [torch.empty((B, Hq, 512), dtype=torch.bfloat16, device="cuda:0") for _ in range(n_inst)]

    def call(r):
        qr, tr, lt, _ = insts[r]
        ssa.hybrid_decode(qr, base.k_cache, base.v_cache, tr, base.ctx_lens, lt, **pat, scale=576 ** -0.5,
                          out=outs[r], workspace=ws)

    for r in range(n_inst):
        call(r)
    torch.cuda.synchronize()
    reps = 4
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            for _ in range(reps):
                for r in range(n_inst):
                    call(r)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    ms = time_events(graph.replay, max(1, iters // (reps * n_inst))) / (reps * n_inst)
    nbytes = int(np.mean([hybrid_bytes(base.lens, inst[3], **pat, page_size=inputs.PAGE_SIZE, Hq=Hq)
                          for inst in insts]))
    gbs = nbytes / (ms * 1e-3) / 1e9
    name = "hybrid_decode_bf16_latent_b32_h64_d576_L131072_sink16_win1024_top1024"
    res = {"workload": name, "us": ms * 1e3, "bytes": nbytes, "GB/s": gbs,
           "roofline": decode_roofline(gbs, ["decode_split_latent hybrid",
                                             "decode_merge<true, 512> hybrid"]),
           "timing": f"HIP graph of {reps * n_inst} calls rotating over {n_inst} instances"}
    del graph, insts, outs, base, ws
    free_gpu()
    return name, res


# ---------------------------------------------------------------------------
# Backward of prefill
# ---------------------------------------------------------------------------
def backward_flops(cfg) -> int:
    """Algorithmic flops of the backward: per attended pair and head, the
    recomputed scores (2 d_qk), dP = dout.v (2 d_v), dv (2 d_v), dk (2 d_qk)
    and dq (2 d_qk)."""
    from block_sparse_streaming_amd import inputs
    pairs = attended_pairs(cfg.N, **inputs.PATTERN) * cfg.Hq * cfg.B
    return pairs * 2 * (3 * cfg.d_qk + 2 * cfg.d_v)


def backward_kernel_keys(cfg) -> list[str]:
    """Trace keys (kernel, grid in work-items) of the three backward launches
    for the deployed pattern, as the library plans them."""
    from block_sparse_streaming_amd import inputs
    b, s, l = (inputs.PATTERN[k] for k in ("block", "sink", "local"))
    n_pad = -(-cfg.N // 128) * 128
    tiles = n_pad // 128
    sink_keys = min(s * b, cfg.N)
    sink_tiles = -(-sink_keys // 128)
    sink_rows = min(sink_tiles * 128, cfg.N)
    span = -(-min(l * b, n_pad) // 128) * 128
    chunk = min(4 * max(span, 128), n_pad)
    n_chunks = -(-cfg.N // chunk) if sink_tiles else 0
    dq = tiles * cfg.Hq * cfg.B
    dkv = (sink_tiles * n_chunks + tiles - sink_tiles) * cfg.Hkv * cfg.B
    fin = -(-(cfg.B * cfg.Hkv * sink_rows * (cfg.d_qk + cfg.d_v) // 4) // 256)
    d = f"<{cfg.d_qk}, {cfg.d_v}>"
    return [f"ssa_bwd_dq_bf16{d} grid={dq * 256}", f"ssa_bwd_dkv_bf16{d} grid={dkv * 256}",
            f"ssa_bwd_sink_finalize{d} grid={fin * 256}"]


def backward_setup(cfg):
    import torch
    import block_sparse_streaming_amd as ssa
    from block_sparse_streaming_amd import inputs

    q, k, v = inputs.prefill_inputs(cfg, "cuda:0")
    do = inputs.prefill_grad(cfg, "cuda:0")
    o, lse = ssa.prefill(q, k, v, **inputs.PATTERN, scale=cfg.scale, return_lse=True)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    need = ssa.backward_workspace_size(cfg.dtype, cfg.B, cfg.N, cfg.Hq, cfg.Hkv, cfg.d_qk, cfg.d_v,
                                       **inputs.PATTERN)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")

    def step():
        ssa.prefill_backward(q, k, v, o, lse, do, **inputs.PATTERN, scale=cfg.scale, dq=dq, dk=dk,
                             dv=dv, workspace=ws)

    return cfg, step


def bench_backward(cfg, steps: int, warmup: int):
    """ssa_prefill_backward (three launches: dq, dk/dv, sink finalize) on a
    prefill workload, given the forward's o and lse."""
    import torch
    cfg, step = backward_setup(cfg)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ms = time_events(step, steps)
    flops = backward_flops(cfg)
    tflops = flops / (ms * 1e-3) / 1e12
    name = cfg.name.replace("prefill", "backward", 1)
    res = {"workload": name, "ms": ms, "steps": steps, "algorithmic_flops": flops, "TFLOP/s": tflops,
           "roofline": with_measured({"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS,
                                      "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_TFLOPS,
                                      "traffic": recorded_traffic(backward_kernel_keys(cfg))})}
    del step
    free_gpu()
    return name, res


# ---------------------------------------------------------------------------
# Decode
# ---------------------------------------------------------------------------
def decode_bytes(cfg, lens, selected, page_size: int) -> int:
    """Algorithmic bytes of one decode call: the attended cache rows (a value
    that aliases the key row counts once), q, o, the page-table entries of the
    attended pages and the context lengths."""
    esz = 2
    tok_bytes = cfg.Hkv * cfg.d_qk * esz if cfg.latent else cfg.Hkv * (cfg.d_qk + cfg.d_v) * esz
    qo = len(lens) * cfg.Hq * (cfg.d_qk + cfg.d_v) * esz
    return sum(selected) * tok_bytes + qo + sum(-(-t // page_size) for t in selected) * 4 + len(lens) * 4


def decode_roofline(gbs: float, traffic_keys=None) -> dict:
    return with_measured({"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": gbs / PEAK_HBM_GBS,
                          "traffic": recorded_traffic(traffic_keys) if traffic_keys else None})


def bench_decode_latent(iters: int):
    """ssa_decode and full_attn_decode on the 128K latent workload. The SSA
    call rotates over 8 page-table/query instances, whose selected pages
    (8 x 42 MB) exceed the 256 MB Infinity Cache, and is replayed from a HIP
    graph so that host launch overhead does not pad the short kernels."""
    import torch
    import block_sparse_streaming_amd as ssa
    from block_sparse_streaming_amd import inputs

    cfg = inputs.DECODE_LATENT_128K
    pat = inputs.PATTERN
    dev = "cuda:0"
    base = inputs.decode_inputs(cfg, dev)
    n_inst = 8
    insts = []
    for r in range(n_inst):
        table, _ = inputs.page_table_for(base.lens, inputs.PAGE_SIZE, seed=cfg.seed + 100 + r)
        g = inputs.generator(dev, cfg.seed + 200 + r)
        qr = inputs.randn(tuple(base.q.shape), cfg.dtype, dev, g)
        insts.append((qr, torch.from_numpy(table).to(dev)))
    B, Hq, dv = cfg.B, cfg.Hq, cfg.d_v
    outs = [torch.empty((B, Hq, dv), dtype=cfg.dtype, device=dev) for _ in range(n_inst)]
    max_pages = base.page_table.shape[1]
    ws_ssa = torch.empty(ssa.decode_workspace_size(cfg.dtype, B, Hq, cfg.Hkv, cfg.d_qk, dv,
                                                   inputs.PAGE_SIZE, max_pages),
                         dtype=torch.uint8, device=dev)
    ws_full = torch.empty(ssa.decode_workspace_size(cfg.dtype, B, Hq, cfg.Hkv, cfg.d_qk, dv,
                                                    inputs.PAGE_SIZE, max_pages, full=True),
                          dtype=torch.uint8, device=dev)

    def ssa_call(r):
        qr, tr = insts[r]
        ssa.decode(qr, base.k_cache, base.v_cache, tr, base.ctx_lens, **pat, scale=cfg.scale,
                   out=outs[r], workspace=ws_ssa)

    def full_call():
        ssa.full_decode(base.q, base.k_cache, base.v_cache, base.page_table, base.ctx_lens,
                        scale=cfg.scale, out=outs[0], workspace=ws_full)

    for r in range(n_inst):
        ssa_call(r)
    full_call()
    torch.cuda.synchronize()

    reps = 4
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            for _ in range(reps):
                for r in range(n_inst):
                    ssa_call(r)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    n_graph = max(1, iters // (reps * n_inst))
    ssa_ms = time_events(graph.replay, n_graph) / (reps * n_inst)
    full_ms = time_events(full_call, max(3, iters // 16))

    sel = [decode_selected_tokens(L, **pat) for L in base.lens]
    ssa_bytes = decode_bytes(cfg, base.lens, sel, inputs.PAGE_SIZE)
    full_bytes = decode_bytes(cfg, base.lens, list(base.lens), inputs.PAGE_SIZE)
    ssa_gbs = ssa_bytes / (ssa_ms * 1e-3) / 1e9
    full_gbs = full_bytes / (full_ms * 1e-3) / 1e9
    res = {
        "workload": cfg.name,
        "ssa_decode": {"us": ssa_ms * 1e3, "bytes": ssa_bytes, "GB/s": ssa_gbs,
                       "roofline": decode_roofline(ssa_gbs, ["decode_split_latent ssa",
                                                             "decode_merge<true, 512> ssa"]),
                       "timing": f"HIP graph of {reps * n_inst} calls rotating over {n_inst} instances"},
        "full_attn_decode": {"us": full_ms * 1e3, "bytes": full_bytes, "GB/s": full_gbs,
                             "roofline": decode_roofline(full_gbs, ["decode_split_latent full",
                                                                    "decode_merge<true, 512> full"])},
        "ssa_over_full_time": ssa_ms / full_ms,
    }
    del graph, insts, outs, base, ws_ssa, ws_full
    free_gpu()
    return res


def bench_decode_ragged(iters: int):
    """ssa_decode on the ragged workload (65 sequences, 4K-1M tokens, 16 heads,
    d=128). Its selected pages (~0.5 GB) exceed the Infinity Cache, so back-to-
    back calls read HBM."""
    import torch
    import block_sparse_streaming_amd as ssa
    from block_sparse_streaming_amd import inputs

    cfg = inputs.DECODE_RAGGED
    pat = inputs.PATTERN
    dev = "cuda:0"
    inp = inputs.decode_inputs(cfg, dev)
    out = torch.empty((cfg.B, cfg.Hq, cfg.d_v), dtype=cfg.dtype, device=dev)
    ws = torch.empty(ssa.decode_workspace_size(cfg.dtype, cfg.B, cfg.Hq, cfg.Hkv, cfg.d_qk, cfg.d_v,
                                               inputs.PAGE_SIZE, inp.page_table.shape[1]),
                     dtype=torch.uint8, device=dev)

    def call():
        ssa.decode(inp.q, inp.k_cache, inp.v_cache, inp.page_table, inp.ctx_lens, **pat,
                   scale=cfg.scale, out=out, workspace=ws)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    ms = time_events(call, iters)
    sel = [decode_selected_tokens(L, **pat) for L in inp.lens]
    nbytes = decode_bytes(cfg, inp.lens, sel, inputs.PAGE_SIZE)
    gbs = nbytes / (ms * 1e-3) / 1e9
    res = {"workload": cfg.name, "ssa_decode": {"us": ms * 1e3, "bytes": nbytes, "GB/s": gbs,
                                                "roofline": decode_roofline(
                                                    gbs, ["decode_split_valu<true, 128, 1, false> ragged",
                                                          "decode_merge<true, 128> ragged"])}}
    del inp, out, ws
    free_gpu()
    return res


# ---------------------------------------------------------------------------
# CPU oracle
# ---------------------------------------------------------------------------
def cpu_info() -> dict:
    """The host the oracle runs on: CPU model (from /proc/cpuinfo) and the
    number of CPUs this process may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count()
    return {"cpu_model": model, "nproc": nproc}


def _bits(t):
    """Host array for the oracle: bf16 bit patterns as uint16, or float32."""
    import torch
    t = t.contiguous()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def _cpu_randn(shape, dtype, gen):
    import torch
    return torch.randn(shape, generator=gen).to(dtype)


_ORACLE_THREADS = []   # the oracle's thread count before any change (all cores)


def _oracle_seconds(threads: int, fn) -> float:
    """Seconds of fn() with the oracle on `threads` threads (0: all). fn may
    be a list of callables (pieces of one workload): their times add up, and
    a progress line goes to stderr after each."""
    import oracle
    if not _ORACLE_THREADS:
        _ORACLE_THREADS.append(oracle.max_threads())
    oracle.set_threads(threads if threads > 0 else _ORACLE_THREADS[0])
    try:
        total = 0.0
        for f in (fn if isinstance(fn, list) else [fn]):
            t0 = time.perf_counter()
            f()
            total += time.perf_counter() - t0
            print(f"# oracle: {total:.1f} s on {threads or _ORACLE_THREADS[0]} thread(s)", file=sys.stderr,
                  flush=True)
        return total
    finally:
        oracle.set_threads(_ORACLE_THREADS[0])


def _prefill_oracle(cfg, heads: int, rows, gen, pieces: int = 1):
    """A callable running the oracle on `rows` of `heads` query heads of the
    workload's shape (inputs drawn on the CPU, same distribution and dtype),
    and the attended (query, key) pairs it evaluates. With pieces > 1, a list
    of callables over consecutive parts of the rows (one set of inputs)."""
    import oracle
    from block_sparse_streaming_amd import inputs
    q = _bits(_cpu_randn((cfg.B, cfg.N, heads, cfg.d_qk), cfg.dtype, gen))
    k = _bits(_cpu_randn((cfg.B, cfg.N, heads, cfg.d_qk), cfg.dtype, gen))
    v = _bits(_cpu_randn((cfg.B, cfg.N, heads, cfg.d_v), cfg.dtype, gen))
    pat = inputs.PATTERN
    b, s, l = pat["block"], pat["sink"], pat["local"]
    r = np.arange(cfg.N) if rows is None else np.asarray(rows)
    lo = np.maximum(s * b, (r // b - l + 1) * b)
    pairs = int((np.minimum(s * b, r + 1) + np.maximum(0, r + 1 - lo)).sum()) * heads * cfg.B
    if pieces == 1:
        return (lambda: oracle.prefill(q, k, v, **pat, scale=cfg.scale, rows=rows)), pairs
    parts = np.array_split(r, pieces)
    return [(lambda p=p: oracle.prefill(q, k, v, **pat, scale=cfg.scale, rows=p)) for p in parts], pairs


def _decode_oracle(cfg, lens, full: bool, gen):
    """A callable running the paged decode oracle on sequences of context
    lengths `lens` (the workload's heads and dims; a host cache holding only
    the pages the call reads, in shuffled order), and the attended tokens."""
    import oracle
    from block_sparse_streaming_amd import inputs
    pat = inputs.PATTERN
    P = inputs.PAGE_SIZE
    b, s, l = pat["block"], pat["sink"], pat["local"]
    need, toks = [], 0
    for L in lens:
        j = np.arange(L)
        keep = np.ones(L, bool) if full else (j // b < s) | (j // b > (L - 1) // b - l)
        need.append(np.unique(j[keep] // P))
        toks += int(keep.sum())
    n = sum(x.size for x in need)
    perm = np.random.default_rng(cfg.seed).permutation(n).astype(np.int32)
    max_pages = max(-(-L // P) for L in lens)
    table = np.full((len(lens), max_pages), 0, np.int32)
    off = 0
    for i, x in enumerate(need):
        table[i, x] = perm[off:off + x.size]
        off += x.size
    q = _bits(_cpu_randn((len(lens), cfg.Hq, cfg.d_qk), cfg.dtype, gen))
    kc = _bits(_cpu_randn((n, P, cfg.Hkv, cfg.d_qk), cfg.dtype, gen))
    vc = kc[..., :cfg.d_v] if cfg.latent else _bits(_cpu_randn((n, P, cfg.Hkv, cfg.d_v), cfg.dtype, gen))
    kw = dict(block=1, sink=0, local=1) if full else pat
    lens_np = np.asarray(lens, np.int32)
    return (lambda: oracle.decode_paged(q, kc, vc, table, lens_np, **kw, scale=cfg.scale, full=full)), toks


def _entry(what, sample, scale_to_full, seconds_all, seconds_one, work_full, unit, per_unit, threads,
           scale_one=None):
    """One workload's oracle timing: the sample's seconds on all cores and on
    one core, the time for the whole workload they imply (linear in work) and
    the rate in the metric's unit. scale_one: the one-core sample's own
    factor, when it is another sample."""
    full_all = seconds_all * scale_to_full
    full_one = seconds_one * (scale_to_full if scale_one is None else scale_one)
    return {"what": what, "sample": sample, "work_full": work_full,
            "all_cores": {"threads": threads, "sample_s": seconds_all, "full_s": full_all,
                          unit: work_full * per_unit / full_all},
            "one_core": {"threads": 1, "sample_s": seconds_one, "full_s": full_one,
                         unit: work_full * per_unit / full_one},
            "unit": unit}


def cpu_baseline(full_runs: bool = False):
    """The CPU oracle, as it stands, timed on this host with all cores and
    with one core, for each workload of the metric. The headline value is the
    32K prefill on all cores over the whole workload (a few seconds). The
    other figures come from bounded samples of each workload (rows of some
    query heads for prefill, sequences for decode; the oracle's cost is linear
    in attended pairs or tokens, so a sample scales to the workload exactly),
    except with full_runs, where prefill at 2K and 32K and decode on the latent
    and ragged workloads run whole (the 256K prefill is always sampled)."""
    import torch
    import oracle
    from block_sparse_streaming_amd import inputs

    gen = torch.Generator().manual_seed(4040)
    if not _ORACLE_THREADS:
        _ORACLE_THREADS.append(oracle.max_threads())
    threads = _ORACLE_THREADS[0]
    table = {}

    def flops(cfg):
        return 2 * (cfg.d_qk + cfg.d_v)

    # prefill fp32 2K: the whole workload both ways
    cfg = inputs.PREFILL_FP32_2K
    fn, pairs = _prefill_oracle(cfg, cfg.Hq, None, gen)
    table[cfg.name] = _entry("ssa_prefill", "whole workload", 1.0, _oracle_seconds(0, fn),
                             _oracle_seconds(1, fn), pairs, "TFLOP/s", flops(cfg) * 1e-12, threads)

    # prefill bf16 32K: whole on all cores; one core on every 16th query tile
    # (whole with full_runs)
    cfg = inputs.PREFILL_BF16_32K
    fn_all, pairs = _prefill_oracle(cfg, cfg.Hq, None, gen)
    t_all = _oracle_seconds(0, fn_all)
    if full_runs:
        parts, _ = _prefill_oracle(cfg, cfg.Hq, None, gen, pieces=16)   # progress lines
        t_one, scale_one, sample = _oracle_seconds(1, parts), 1.0, "whole workload"
    else:
        rows = np.concatenate([np.arange(t * 128, t * 128 + 128) for t in range(0, cfg.N // 128, 16)])
        fn1, pairs1 = _prefill_oracle(cfg, cfg.Hq, rows, gen)
        t_one, scale_one = _oracle_seconds(1, fn1), pairs / pairs1
        sample = "all cores: whole workload; one core: every 16th 128-row query tile, all heads"
    headline = _entry("ssa_prefill", sample, 1.0, t_all, t_one, pairs, "TFLOP/s",
                      flops(cfg) * 1e-12, threads, scale_one=scale_one)
    table[cfg.name] = headline

    # prefill bf16 256K: stratified rows (query tiles 0..8, 1023, 1024, 2047
    # and 4 seeded random tiles) of 2 of the 64 heads
    cfg = inputs.PREFILL_BF16_256K
    rng = np.random.default_rng(7)
    tiles = sorted(set(list(range(9)) + [1023, 1024, 2047] +
                       [int(x) for x in rng.choice(np.arange(9, 2047), 4, replace=False)]))
    rows = np.concatenate([np.arange(t * 128, t * 128 + 128) for t in tiles])
    fn, pairs_s = _prefill_oracle(cfg, 2, rows, gen)
    pairs_full = attended_pairs(cfg.N, **inputs.PATTERN) * cfg.Hq * cfg.B
    t_all, t_one = _oracle_seconds(0, fn), _oracle_seconds(1, fn)
    table[cfg.name] = _entry("ssa_prefill", f"{len(tiles)} query tiles x 2 of 64 heads "
                             f"({pairs_s} of {pairs_full} pairs), extrapolated by pair count",
                             pairs_full / pairs_s, t_all, t_one, pairs_full, "TFLOP/s",
                             flops(cfg) * 1e-12, threads)

    # latent decode at 128K: SSA on all 32 sequences both ways; full
    # attention on one sequence (all 32 with full_runs)
    cfg = inputs.DECODE_LATENT_128K
    lens = cfg.lens
    fn, toks = _decode_oracle(cfg, lens, False, gen)
    nbytes = toks * cfg.d_qk * 2
    table[cfg.name + ":ssa_decode"] = _entry(
        "ssa_decode", "whole workload", 1.0, _oracle_seconds(0, fn), _oracle_seconds(1, fn), nbytes,
        "GB/s", 1e-9, threads)
    sub = lens if full_runs else lens[:1]
    pieces = [_decode_oracle(cfg, sub[k:k + 2], True, gen) for k in range(0, len(sub), 2)]
    fn, toks_s = [p[0] for p in pieces], sum(p[1] for p in pieces)
    toks_full = sum(lens)
    table[cfg.name + ":full_attn_decode"] = _entry(
        "full_attn_decode", "whole workload" if full_runs else
        f"1 of {len(lens)} sequences, extrapolated by token count", toks_full / toks_s,
        _oracle_seconds(0, fn), _oracle_seconds(1, fn), toks_full * cfg.d_qk * 2, "GB/s", 1e-9, threads)

    # ragged decode: SSA on all 65 sequences both ways
    cfg = inputs.DECODE_RAGGED
    fn, toks = _decode_oracle(cfg, cfg.lens, False, gen)
    table[cfg.name + ":ssa_decode"] = _entry(
        "ssa_decode", "whole workload", 1.0, _oracle_seconds(0, fn), _oracle_seconds(1, fn),
        toks * cfg.Hkv * (cfg.d_qk + cfg.d_v) * 2, "GB/s", 1e-9, threads)

    info = cpu_info()
    h = headline["all_cores"]
    return {"value": h["TFLOP/s"], "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole 32K prefill workload ({h['full_s']:.1f} s of fp64 oracle work on "
                      f"{threads} threads); per-workload figures, all cores and one core, in 'workloads'",
            "cpu_model": info["cpu_model"], "nproc": info["nproc"], "workloads": table}


def print_cpu_oracle_table():
    """Markdown table of the oracle's times on this host (full runs)."""
    t0 = time.perf_counter()
    cpu = cpu_baseline(full_runs=True)
    print(f"Host: {cpu['cpu_model']}, nproc {cpu['nproc']}, oracle threads {cpu['cores']} "
          f"(all cores) and 1; {time.perf_counter() - t0:.0f} s in all.\n")
    print("| workload | call | sample | all cores: s | all cores: rate | one core: s | one core: rate |")
    print("|---|---|---|---|---|---|---|")
    for name, e in cpu["workloads"].items():
        u = e["unit"]
        a, o = e["all_cores"], e["one_core"]
        print(f"| {name.split(':')[0]} | {e['what']} | {e['sample']} | {a['full_s']:.2f} | "
              f"{a[u] * (1e3 if u == 'TFLOP/s' else 1):.3f} {'GFLOP/s' if u == 'TFLOP/s' else u} | "
              f"{o['full_s']:.2f} | {o[u] * (1e3 if u == 'TFLOP/s' else 1):.3f} "
              f"{'GFLOP/s' if u == 'TFLOP/s' else u} |", flush=True)


# ---------------------------------------------------------------------------
# Counter-collection runs
# ---------------------------------------------------------------------------
def profile_run(what: str):
    import torch
    from block_sparse_streaming_amd import inputs
    if what in ("prefill", "prefill_fp32", "prefill_256k"):
        cfg = {"prefill": inputs.PREFILL_BF16_32K, "prefill_fp32": inputs.PREFILL_FP32_2K,
               "prefill_256k": inputs.PREFILL_BF16_256K}[what]
        _, step = prefill_setup(cfg)
        for _ in range(3):
            step()
    elif what == "backward_256k":
        _, step = backward_setup(inputs.PREFILL_BF16_256K)
        for _ in range(2):
            step()
    elif what == "decode":
        bench_decode_latent(64)
        bench_decode_ragged(8)
    elif what == "backward":
        _, step = backward_setup(inputs.PREFILL_BF16_32K)
        for _ in range(3):
            step()
    elif what == "dual":
        _, step = dual_setup(inputs.PREFILL_BF16_32K)
        for _ in range(3):
            step()
    elif what == "hybrid":
        bench_hybrid(32)
    elif what == "extend":
        _, step = extend_chunk_setup()
        for _ in range(3):
            step()
        bench_extend_mtp(32)
    elif what == "copy":
        n = 1 << 28                                   # 1 GiB of fp32 each way
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
    torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of untimed back-to-back calls after the warmup steps, before each "
                         "timed region (clock ramp); 0 disables")
    ap.add_argument("--profile", choices=["prefill", "prefill_fp32", "prefill_256k", "decode", "backward",
                                          "backward_256k", "dual", "extend", "hybrid", "copy"], default=None)
    ap.add_argument("--cpu-oracle-table", action="store_true",
                    help="time the CPU oracle on every workload (all cores and one core, whole "
                         "workloads where that is feasible) and print a markdown table; no GPU work")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the 32K prefill (and the CPU oracle)")
    args = ap.parse_args()
    SETTLE_S[0] = max(0.0, args.settle)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the path "
              "shards by head or by sequence with no communication, so one GPU's share is the "
              "measured workload", file=sys.stderr)
        sys.exit(2)

    if args.cpu_oracle_table:
        print_cpu_oracle_table()
        return
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.profile:
        profile_run(args.profile)
        return

    def note(msg):
        print("# " + msg, file=sys.stderr, flush=True)

    if not args.headline_only:
        m = measure_ceilings()
        note(f"measured ceilings: bf16 GEMM {m['bf16_gemm_tflops']:.0f} TFLOP/s, "
             f"HBM read {m['hbm_read_gbs']:.0f} GB/s")
    from block_sparse_streaming_amd import inputs
    cfg, head = bench_prefill(inputs.PREFILL_BF16_32K, args.steps, args.warmup)
    note(f"prefill {cfg.name}: {head['ms']:.4f} ms/launch, {head['TFLOP/s']:.1f} TFLOP/s")
    workloads = {}
    if not args.headline_only:
        for wl, steps in ((inputs.PREFILL_FP32_2K, 50), (inputs.PREFILL_BF16_256K, 5)):
            c, r = bench_prefill(wl, steps, 2)
            workloads[c.name] = r
            note(f"prefill {c.name}: {r['ms']:.4f} ms/launch, {r['TFLOP/s']:.1f} TFLOP/s")
        dec = bench_decode_latent(256)
        workloads[dec["workload"]] = dec
        note(f"decode {dec['workload']}: ssa {dec['ssa_decode']['us']:.2f} us "
             f"({dec['ssa_decode']['GB/s']:.0f} GB/s), full {dec['full_attn_decode']['us']:.1f} us "
             f"({dec['full_attn_decode']['GB/s']:.0f} GB/s)")
        rag = bench_decode_ragged(50)
        workloads[rag["workload"]] = rag
        note(f"decode {rag['workload']}: ssa {rag['ssa_decode']['us']:.2f} us "
             f"({rag['ssa_decode']['GB/s']:.0f} GB/s)")
        for wl, steps in ((inputs.PREFILL_BF16_32K, 20), (inputs.PREFILL_BF16_256K, 3)):
            name, r = bench_backward(wl, steps, 2)
            workloads[name] = r
            note(f"backward {name}: {r['ms']:.4f} ms/call, {r['TFLOP/s']:.1f} TFLOP/s")
        name, r = bench_dual(inputs.PREFILL_BF16_32K, 10, 2)
        workloads[name] = r
        note(f"dual {name}: {r['ms']:.4f} ms/launch, {r['TFLOP/s']:.1f} TFLOP/s")
        name, r = bench_extend_chunk(10, 2)
        workloads[name] = r
        note(f"extend {name}: {r['ms']:.4f} ms/call, {r['TFLOP/s']:.1f} TFLOP/s")
        name, r = bench_extend_mtp(256)
        workloads[name] = r
        note(f"extend {name}: {r['us']:.2f} us/call ({r['GB/s']:.0f} GB/s)")
        name, r = bench_hybrid(256)
        workloads[name] = r
        note(f"hybrid {name}: {r['us']:.2f} us/call ({r['GB/s']:.0f} GB/s)")
    cpu = cpu_baseline()
    note(f"cpu oracle: {cpu['value'] * 1e3:.3f} GFLOP/s on {cpu['cores']} threads "
         f"({cpu['cpu_model']}, nproc {cpu['nproc']})")
    from block_sparse_streaming_amd import inputs
    line = {
        "metric": METRIC,
        "value": head["TFLOP/s"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": SETTLE_S[0],
        "ms_per_step": head["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.B, "seq_len": cfg.N, "heads": cfg.Hq,
                   "d_qk": cfg.d_qk, "d_v": cfg.d_v, "pattern": dict(inputs.PATTERN),
                   "algorithmic_flops_per_step": head["algorithmic_flops"]},
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "measured_ceilings": dict(MEASURED),
        "workloads": workloads,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
