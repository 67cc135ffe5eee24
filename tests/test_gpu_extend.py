"""GPU parity of ssa_extend (new tokens of each sequence against the paged
cache: multi-token decode and chunked prefill) against the CPU oracle,
through the C ABI.

Both kernels are covered: one-row chunks, and every chunk on shapes only
the decode kernels compile (fp32, d = 256, the latent shape), run as decode
steps over query rows; longer chunks on bf16 d = 64 / 128 / 192 take the
paged tile kernel, short multi-token chunks included. Every row of every case is
compared with the oracle, which evaluates each row as one decode step at its
own context length. The oracle reads only the pages the rows attend (the rest
are NaN), so a wrong page read by either side would show.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_streaming_amd as ssa
import oracle
from block_sparse_streaming_amd import inputs
from tests.gpu_util import assert_lse, assert_parity, compact_pages, host, rows_logical_pages, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
PAT = dict(block=128, sink=1, local=7)


def _oracle_rows(inp, pattern, scale, rows=None, latent_dv=None, page_size=inputs.PAGE_SIZE):
    """Oracle output of the given packed rows (all rows by default), each as a
    one-row chunk at its own context length."""
    cu = np.concatenate([[0], np.cumsum(inp.qlens)])
    seq = np.repeat(np.arange(len(inp.lens)), inp.qlens)
    total = int(cu[-1])
    rows = np.arange(total) if rows is None else np.asarray(rows)
    seq_r = seq[rows]
    pos = np.array(inp.lens)[seq_r] - np.array(inp.qlens)[seq_r] + (rows - cu[seq_r])
    need = [rows_logical_pages(inp.lens[b], pos[seq_r == b], page_size, pattern["block"],
                               pattern["sink"], pattern["local"]) for b in range(len(inp.lens))]
    kc, vc, table = compact_pages(inp.k_cache, inp.v_cache, inp.table_np, need, latent_dv)
    idx = torch.as_tensor(rows, device=DEV)
    q_rows = host(inp.q[idx])
    one = np.arange(rows.size + 1, dtype=np.int32)
    return oracle.extend(q_rows, kc, vc, table[seq_r], (pos + 1).astype(np.int32), one, **pattern,
                         scale=scale)


def _run(inp, pattern, scale, what, latent_dv=None, rows=None, page_size=inputs.PAGE_SIZE):
    say("extend", what, "rows", tuple(inp.q.shape), "lens", inp.lens[:6], "qlens", inp.qlens[:6],
        "...", len(inp.lens), pattern, inp.q.dtype)
    o, lse = ssa.extend(inp.q, inp.k_cache, inp.v_cache, inp.page_table, inp.ctx_lens, inp.cu_q,
                        max(inp.qlens), **pattern, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = _oracle_rows(inp, pattern, scale, rows, latent_dv, page_size)
    if rows is not None:
        idx = torch.as_tensor(rows, device=DEV)
        o, lse = o[idx], lse[idx]
    assert_parity(o, ro, inp.q.dtype, what)
    assert_lse(lse, rl, inp.q.dtype, what)
    return o, lse


def _inp(lens, qlens, Hq, Hkv, dqk, dv, dtype=torch.bfloat16, seed=0, **kw):
    return inputs.extend_inputs(lens, qlens, Hq, Hkv, dqk, dv, dtype, DEV, seed, **kw)


# Multi-token decode (chunks of 1-8 rows): decode kernels for fp32, d = 256 and
# the latent shape, the tile kernel for bf16 d = 64 / 128.
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_multi_token_decode_mha(dtype):
    lens = (1, 4, 127, 128, 129, 1023, 1024, 1025, 5000, 3)
    qlens = (1, 4, 3, 8, 2, 4, 1, 4, 4, 0)
    _run(_inp(lens, qlens, 4, 4, 128, 128, dtype, seed=700, spare_pages=3), PAT, 128 ** -0.5,
         f"mtp mha {dtype}")


@pytest.mark.parametrize("group,d", [(2, 64), (4, 128), (8, 64), (2, 256)])
def test_multi_token_decode_gqa(group, d):
    lens, qlens = (333, 2048, 4100), (4, 2, 3)
    _run(_inp(lens, qlens, 2 * group, 2, d, d, seed=710 + d + group), PAT, d ** -0.5,
         f"mtp gqa{group} d{d}")


@pytest.mark.parametrize("group", [64, 16])
def test_multi_token_decode_latent(group):
    """The absorbed-MLA latent shape: 576-wide rows whose first 512 entries are
    the value; three draft tokens plus the current one per sequence."""
    lens, qlens = (131, 1024, 1025, 7000, 40000), (4, 4, 4, 4, 2)
    inp = _inp(lens, qlens, group, 1, 576, 512, seed=720 + group, latent=True)
    _run(inp, PAT, 576 ** -0.5, f"mtp latent g{group}", latent_dv=512)


@pytest.mark.parametrize("pattern", [dict(block=64, sink=2, local=3), dict(block=16, sink=3, local=9),
                                     dict(block=100, sink=0, local=2)],
                         ids=lambda p: f"b{p['block']}s{p['sink']}l{p['local']}")
def test_multi_token_decode_patterns(pattern):
    _run(_inp((1, 100, 700, 3000, 9999), (1, 5, 8, 3, 6), 2, 2, 128, 128, seed=730), pattern,
         128 ** -0.5, f"mtp {pattern}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_multi_token_decode_single_split_windows(dtype):
    """Windows of at most 128 tokens fit one split, so the decode kernels over
    query rows write each packed row's output themselves, without a merge
    (fp32 and d = 256 take the decode kernels at any chunk length)."""
    d = 128 if dtype == torch.float32 else 256
    for pattern in (dict(block=32, sink=1, local=3), dict(block=128, sink=0, local=1)):
        _run(_inp((1, 60, 129, 700, 3000), (1, 7, 8, 3, 6), 4, 2, d, d, dtype=dtype, seed=735), pattern,
             d ** -0.5, f"mtp single split {dtype} {pattern}")


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2)])
def test_one_row_chunks_equal_decode_bitwise(Hq, Hkv):
    """bf16 one-row chunks take the decode kernels over query rows: each row
    equals ssa_decode of the same sequence bit for bit, and the oracle."""
    lens = (1, 127, 128, 129, 1025, 5000, 40000)
    inp = _inp(lens, (1,) * len(lens), Hq, Hkv, 128, 128, seed=735 + Hq, spare_pages=2)
    o, lse = _run(inp, PAT, 128 ** -0.5, f"one-row chunks g{Hq // Hkv}")
    od, ld = ssa.decode(inp.q, inp.k_cache, inp.v_cache, inp.page_table, inp.ctx_lens, **PAT,
                        scale=128 ** -0.5, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), od.view(torch.int16)) and torch.equal(lse, ld)


# Chunked prefill (chunks longer than one row): the paged tile kernel.
@pytest.mark.parametrize("dqk,dv,Hq,Hkv", [(128, 128, 2, 2), (128, 128, 4, 1), (64, 64, 4, 2),
                                           (192, 128, 2, 1)])
def test_chunked_prefill_shapes(dqk, dv, Hq, Hkv):
    lens = (2000, 300, 4097, 129, 1500, 12)
    qlens = (700, 300, 9, 129, 1, 12)       # tails, whole sequences, a 1-row chunk among long ones
    _run(_inp(lens, qlens, Hq, Hkv, dqk, dv, seed=740 + dqk + Hq), PAT, dqk ** -0.5,
         f"chunk d{dqk}/{dv} g{Hq // Hkv}")


@pytest.mark.parametrize("pattern", [dict(block=128, sink=0, local=1), dict(block=64, sink=2, local=3),
                                     dict(block=16, sink=1, local=4), dict(block=100, sink=1, local=2),
                                     dict(block=50, sink=3, local=5), dict(block=300, sink=1, local=2),
                                     dict(block=7, sink=5, local=1), dict(block=128, sink=1, local=64),
                                     dict(block=64, sink=1, local=16)],  # waves of a tile: both loop copies
                         ids=lambda p: f"b{p['block']}s{p['sink']}l{p['local']}")
def test_chunked_prefill_patterns(pattern):
    _run(_inp((1300, 2500, 777), (400, 1000, 777), 2, 2, 128, 128, seed=750), pattern, 128 ** -0.5,
         f"chunk {pattern}")


@pytest.mark.parametrize("page_size", [1, 16, 64, 256])
def test_chunked_prefill_page_sizes(page_size):
    _run(_inp((1300, 900), (300, 130), 2, 2, 128, 128, seed=760 + page_size, page_size=page_size,
              spare_pages=5), PAT, 128 ** -0.5, f"chunk page {page_size}", page_size=page_size)


def test_whole_sequence_chunk_equals_prefill_bitwise():
    """One chunk holding a whole sequence visits the same sub-tiles with the
    same arithmetic as ssa_prefill: the rows agree bit for bit."""
    N, H, d = 3000, 2, 128
    inp = _inp((N,), (N,), H, H, d, d, seed=770, spare_pages=2)
    say("extend whole sequence vs prefill", N)
    o = ssa.extend(inp.q, inp.k_cache, inp.v_cache, inp.page_table, inp.ctx_lens, inp.cu_q, N, **PAT)
    # the same keys laid out contiguously
    P = inputs.PAGE_SIZE
    tab = torch.as_tensor(inp.table_np[0], device=DEV, dtype=torch.long)
    k = inp.k_cache[tab].reshape(-1, H, d)[:N][None]
    v = inp.v_cache[tab].reshape(-1, H, d)[:N][None]
    ref = ssa.prefill(inp.q[None], k.contiguous(), v.contiguous(), **PAT)
    torch.cuda.synchronize()
    assert P * tab.numel() >= N
    assert torch.equal(o.view(torch.int16), ref[0].view(torch.int16))


def test_chunked_prefill_full_size_sampled():
    """The chunked-prefill workload the benchmark times: 4 sequences at 32K to
    128K tokens of context, each with a new 8,192-token chunk, 16 heads,
    d = 128, shuffled 128-token pages. Sampled rows of two heads' worth of
    query heads (every head is computed; the oracle checks a sample)."""
    lens, qlens = inputs.EXTEND_CHUNK_LENS, inputs.EXTEND_CHUNK_QLENS
    inp = _inp(lens, qlens, 16, 16, 128, 128, seed=inputs.EXTEND_SEED)
    total = sum(qlens)
    rng = np.random.default_rng(780)
    cu = np.concatenate([[0], np.cumsum(qlens)])
    rows = np.unique(np.concatenate([cu[:-1], cu[1:] - 1, cu[:-1] + 127, cu[:-1] + 128,
                                     rng.choice(total, 200, replace=False)]))
    _run(inp, PAT, 128 ** -0.5, "chunk full size", rows=rows)


def test_multi_token_decode_full_size_sampled():
    """The multi-token decode workload the benchmark times: 32 sequences at
    131,072 tokens, four new rows each, on the latent shape (64 query heads on
    one 576-wide latent head), shuffled 128-token pages. Every row is computed;
    the rows of eight sequences are checked against the oracle."""
    B, T = 32, inputs.EXTEND_MTP_Q
    inp = _inp((inputs.EXTEND_MTP_LEN,) * B, (T,) * B, 64, 1, 576, 512, seed=inputs.EXTEND_MTP_SEED, latent=True)
    rows = np.concatenate([np.arange(b * T, (b + 1) * T) for b in (0, 3, 7, 12, 18, 23, 29, 31)])
    _run(inp, PAT, 576 ** -0.5, "mtp full size", latent_dv=512, rows=rows)


def test_rejects_small_workspace():
    """One-row chunks run on the decode kernels, which need the workspace."""
    inp = _inp((500, 600), (1, 1), 4, 4, 128, 128, seed=790)
    need = ssa.extend_workspace_size(torch.bfloat16, 2, 2, 1, 4, 4, 128, 128, inputs.PAGE_SIZE,
                                     inp.page_table.shape[1])
    assert need > 0
    ws = torch.empty(need - 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(ssa.SSAError) as e:
        ssa.extend(inp.q, inp.k_cache, inp.v_cache, inp.page_table, inp.ctx_lens, inp.cu_q, 1,
                   workspace=ws)
    assert e.value.status == 3
