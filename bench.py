#!/usr/bin/env python3
"""Benchmark of the streaming sparse attention hot path on one MI355X.

Headline (one JSON line on stdout): ssa_prefill throughput in TFLOP/s on the
32K-token bf16 workload (B=1, N=32768, 16 heads, d=128, b=128, s=1, l=7),
counted as algorithmic flops 2*(d_qk + d_v) per attended (query, key) pair.
The same line carries the decode half of the metric (ssa_decode and
full_attn_decode HBM GB/s on the 128K-context latent workload), the roofline
of each kernel and the CPU oracle timed on a bounded sample of the prefill.

Inputs are synthetic (seeded N(0,1)) and resident in HBM before timing.
Timing uses HIP events on the stream the kernels run on.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SSA prefill TFLOP/s + decode HBM GB/s (b=128,s=1,l=7) at 32K–256K ctx"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
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


def time_events(fn, iters: int) -> float:
    """Average milliseconds of fn() over iters back-to-back calls, by HIP events."""
    import torch
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(iters):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / iters


def bench_prefill(steps: int, warmup: int):
    import torch
    import block_sparse_streaming_amd as ssa
    from block_sparse_streaming_amd import inputs

    cfg = inputs.CONFIGS[2]
    pat = inputs.PATTERN
    q, k, v = inputs.prefill_inputs(cfg, "cuda:0")
    out = torch.empty((cfg.B, cfg.N, cfg.Hq, cfg.d_v), dtype=cfg.dtype, device="cuda:0")

    def step():
        ssa.prefill(q, k, v, **pat, scale=cfg.scale, out=out)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = time_events(step, steps)
    wall = time.perf_counter() - t0
    pairs = attended_pairs(cfg.N, **pat) * cfg.Hq * cfg.B
    flops = pairs * 2 * (cfg.d_qk + cfg.d_v)
    tflops = flops / (ms * 1e-3) / 1e12
    return cfg, ms, wall, flops, tflops


def bench_decode(iters: int):
    """ssa_decode and full_attn_decode on the 128K latent workload. The SSA
    call rotates over 8 page-table/query instances (8 x 42 MB > the 256 MB
    Infinity Cache) and is replayed from a HIP graph so that host launch
    overhead does not pad the 10-us kernels."""
    import torch
    import block_sparse_streaming_amd as ssa
    from block_sparse_streaming_amd import inputs

    cfg = inputs.CONFIGS[3]
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
    ws_ssa = torch.empty(ssa.decode_workspace_size(cfg.dtype, B, Hq, cfg.Hkv, cfg.d_qk, dv,
                                                   inputs.PAGE_SIZE, base.page_table.shape[1]),
                         dtype=torch.uint8, device=dev)
    ws_full = torch.empty(ssa.decode_workspace_size(cfg.dtype, B, Hq, cfg.Hkv, cfg.d_qk, dv,
                                                    inputs.PAGE_SIZE, base.page_table.shape[1],
                                                    full=True), dtype=torch.uint8, device=dev)

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

    tok_bytes = cfg.d_qk * 2                          # latent row; the value aliases it
    sel = sum(decode_selected_tokens(L, **pat) for L in base.lens)
    sel_pages = sum(-(-decode_selected_tokens(L, **pat) // inputs.PAGE_SIZE) for L in base.lens)
    qo = B * Hq * (cfg.d_qk + dv) * 2
    ssa_bytes = sel * tok_bytes + qo + sel_pages * 4 + B * 4
    full_tokens = sum(base.lens)
    full_bytes = full_tokens * tok_bytes + qo + sum(-(-L // inputs.PAGE_SIZE) for L in base.lens) * 4 + B * 4
    ssa_gbs = ssa_bytes / (ssa_ms * 1e-3) / 1e9
    full_gbs = full_bytes / (full_ms * 1e-3) / 1e9
    return {
        "workload": cfg.name,
        "ssa_decode": {"us": ssa_ms * 1e3, "bytes": ssa_bytes, "GB/s": ssa_gbs,
                       "roofline": {"bound": "hbm", "achieved": ssa_gbs, "peak": PEAK_HBM_GBS,
                                    "unit": "GB/s", "frac": ssa_gbs / PEAK_HBM_GBS, "traffic": None},
                       "timing": f"HIP graph of {reps * n_inst} calls rotating over {n_inst} instances"},
        "full_attn_decode": {"us": full_ms * 1e3, "bytes": full_bytes, "GB/s": full_gbs,
                             "roofline": {"bound": "hbm", "achieved": full_gbs, "peak": PEAK_HBM_GBS,
                                          "unit": "GB/s", "frac": full_gbs / PEAK_HBM_GBS,
                                          "traffic": None}},
        "ssa_over_full_time": ssa_ms / full_ms,
    }


def cpu_baseline():
    """The CPU oracle, as it stands, on the prefill workload: every query tile
    of every head (the whole workload is a few seconds of fp64 work on the
    host cores, inside the bounded budget), drawn on the CPU with the same
    distribution and dtype."""
    import torch
    import oracle
    from block_sparse_streaming_amd import inputs

    cfg = inputs.CONFIGS[2]
    pat = inputs.PATTERN
    gen = torch.Generator().manual_seed(cfg.seed)
    q = torch.randn((1, cfg.N, cfg.Hq, cfg.d_qk), generator=gen).to(cfg.dtype)
    k = torch.randn((1, cfg.N, cfg.Hkv, cfg.d_qk), generator=gen).to(cfg.dtype)
    v = torch.randn((1, cfg.N, cfg.Hkv, cfg.d_v), generator=gen).to(cfg.dtype)
    qh, kh, vh = (t.view(torch.int16).numpy().view(np.uint16) for t in (q, k, v))
    t0 = time.perf_counter()
    oracle.prefill(qh, kh, vh, **pat, scale=cfg.scale)
    elapsed = time.perf_counter() - t0
    flops = attended_pairs(cfg.N, **pat) * cfg.Hq * cfg.B * 2 * (cfg.d_qk + cfg.d_v)
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"the whole prefill workload ({cfg.N // 128} query tiles x {cfg.Hq} heads), "
                      f"{elapsed:.1f} s of fp64 oracle work"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards with no communication; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    cfg, ms, wall, flops, tflops = bench_prefill(args.steps, args.warmup)
    print(f"# prefill {cfg.name}: {ms:.4f} ms/launch, {tflops:.1f} TFLOP/s", file=sys.stderr,
          flush=True)
    dec = bench_decode(200)
    print(f"# decode: ssa {dec['ssa_decode']['us']:.2f} us ({dec['ssa_decode']['GB/s']:.0f} GB/s), "
          f"full {dec['full_attn_decode']['us']:.1f} us ({dec['full_attn_decode']['GB/s']:.0f} GB/s)",
          file=sys.stderr, flush=True)
    cpu = cpu_baseline()
    print(f"# cpu oracle: {cpu['value'] * 1e3:.3f} GFLOP/s on {cpu['cores']} threads", file=sys.stderr,
          flush=True)
    line = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.B, "seq_len": cfg.N, "heads": cfg.Hq,
                   "d_qk": cfg.d_qk, "d_v": cfg.d_v, "pattern": dict(inputs_pattern()),
                   "algorithmic_flops_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / PEAK_BF16_TFLOPS, "traffic": None},
        "cpu_baseline": cpu,
        "decode": dec,
    }
    print(json.dumps(line), flush=True)


def inputs_pattern():
    from block_sparse_streaming_amd import inputs
    return inputs.PATTERN


if __name__ == "__main__":
    main()
