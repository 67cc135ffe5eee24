"""Calls captured in a HIP graph and replayed give the eager results, bit for
bit: the benchmark times the decode-family calls that way. Each graph is
replayed several times with eager work and synchronisations between the
replays, and every replay is checked (a captured call must not rely on state
that only the first replay sees)."""
import numpy as np
import pytest
import torch

import block_sparse_streaming_amd as ssa
from block_sparse_streaming_amd import inputs
from tests.gpu_util import say

DEV = "cuda:0"
LAT_SCALE = 576 ** -0.5


def _latent(lens, qlens, seed):
    return inputs.extend_inputs(lens, qlens, 64, 1, 576, 512, torch.bfloat16, DEV, seed, latent=True)


def _instances(inp, n, seed, lists_k=0):
    out = []
    for r in range(n):
        table, _ = inputs.page_table_for(inp.lens, inputs.PAGE_SIZE, seed=seed + 100 + r)
        q = inputs.randn(tuple(inp.q.shape), inp.q.dtype, DEV, inputs.generator(DEV, seed + 200 + r))
        lst = None
        if lists_k:
            lst = torch.from_numpy(inputs.token_lists(inp.lens, lists_k, seed + 300 + r)).to(DEV)
        out.append((q, torch.from_numpy(table).to(DEV), lst))
    return out


def _calls(kind):
    """(calls over instances writing outs[r], outs, noise) for one workload."""
    seed = 4100
    if kind in ("ssa", "full"):
        inp = _latent((5000, 130, 2049, 777), (1, 1, 1, 1), seed)
        full = kind == "full"
        ws = torch.zeros(ssa.decode_workspace_size(torch.bfloat16, 4, 64, 1, 576, 512, inputs.PAGE_SIZE,
                                                   inp.page_table.shape[1], full=full),
                         dtype=torch.uint8, device=DEV)
        insts = _instances(inp, 3, seed)
        outs = [torch.empty((4, 64, 512), dtype=torch.bfloat16, device=DEV) for _ in insts]

        def call(r):
            q, table, _ = insts[r]
            if full:
                ssa.full_decode(q, inp.k_cache, inp.v_cache, table, inp.ctx_lens, scale=LAT_SCALE,
                                out=outs[r], workspace=ws)
            else:
                ssa.decode(q, inp.k_cache, inp.v_cache, table, inp.ctx_lens, **inputs.PATTERN,
                           scale=LAT_SCALE, out=outs[r], workspace=ws)
    elif kind == "valu":
        # MHA / GQA shapes: the split kernel merges each row itself, through
        # arrival counters in the workspace that every call leaves at zero.
        inp = inputs.extend_inputs((5000, 130, 2049, 777), (1, 1, 1, 1), 8, 4, 128, 128, torch.bfloat16, DEV,
                                   seed)
        ws = torch.zeros(ssa.decode_workspace_size(torch.bfloat16, 4, 8, 4, 128, 128, inputs.PAGE_SIZE,
                                                   inp.page_table.shape[1]),
                         dtype=torch.uint8, device=DEV)
        insts = _instances(inp, 3, seed)
        outs = [torch.empty((4, 8, 128), dtype=torch.bfloat16, device=DEV) for _ in insts]

        def call(r):
            q, table, _ = insts[r]
            ssa.decode(q, inp.k_cache, inp.v_cache, table, inp.ctx_lens, **inputs.PATTERN,
                       scale=128 ** -0.5, out=outs[r], workspace=ws)
    elif kind == "hybrid":
        inp = _latent((5000, 3000, 2049, 1500), (1, 1, 1, 1), seed)
        pat = dict(block=1, sink=16, local=1024)
        K = 256
        ws = torch.zeros(ssa.hybrid_decode_workspace_size(torch.bfloat16, 4, 64, 1, 576, 512, inputs.PAGE_SIZE,
                                                          inp.page_table.shape[1], K, **pat),
                         dtype=torch.uint8, device=DEV)
        insts = _instances(inp, 3, seed, lists_k=K)
        outs = [torch.empty((4, 64, 512), dtype=torch.bfloat16, device=DEV) for _ in insts]

        def call(r):
            q, table, lst = insts[r]
            ssa.hybrid_decode(q, inp.k_cache, inp.v_cache, table, inp.ctx_lens, lst, **pat,
                              scale=LAT_SCALE, out=outs[r], workspace=ws)
    else:  # "mtp": multi-token latent decode (decode kernels over rows) and "chunk": the paged tile kernel
        if kind == "mtp":
            inp = _latent((5000, 2049, 777), (4, 4, 4), seed)
            max_q = 4
        else:
            inp = inputs.extend_inputs((3000, 1300), (700, 300), 4, 2, 128, 128, torch.bfloat16, DEV, seed)
            max_q = 700
        total_q = inp.q.shape[0]
        Hq, Hkv, dqk, dv = inp.q.shape[1], inp.k_cache.shape[2], inp.q.shape[2], inp.v_cache.shape[3]
        ws_bytes = ssa.extend_workspace_size(torch.bfloat16, len(inp.lens), total_q, max_q, Hq, Hkv, dqk, dv,
                                             inputs.PAGE_SIZE, inp.page_table.shape[1])
        ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=DEV)
        insts = _instances(inp, 3, seed)
        outs = [torch.empty((total_q, Hq, dv), dtype=torch.bfloat16, device=DEV) for _ in insts]
        scale = LAT_SCALE if kind == "mtp" else dqk ** -0.5

        def call(r):
            q, table, _ = insts[r]
            ssa.extend(q, inp.k_cache, inp.v_cache, table, inp.ctx_lens, inp.cu_q, max_q, **inputs.PATTERN,
                       scale=scale, out=outs[r], workspace=ws)
    return call, outs, len(outs)


@pytest.mark.gpu
@pytest.mark.parametrize("kind", ["ssa", "full", "valu", "hybrid", "mtp", "chunk"])
def test_graph_replays_match_eager(kind):
    call, outs, n = _calls(kind)
    say("graph", kind)
    for r in range(n):
        call(r)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    assert all(bool(torch.isfinite(o.float()).all()) for o in ref)

    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            for _ in range(2):
                for r in range(n):
                    call(r)
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))          # eager work between replays; stale results would show
        call(0)                            # an eager call sharing the workspace
        torch.cuda.synchronize()
        assert torch.equal(outs[0], ref[0]), (kind, "eager", rep)
        outs[0].fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for r in range(n):
            assert torch.equal(outs[r], ref[r]), (kind, rep, r)
