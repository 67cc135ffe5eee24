"""GPU parity of ssa_decode and full_attn_decode against the CPU oracle, through
the C ABI, plus the decode invariants (page order, poisoned pages, SSA == full
attention for short contexts, decode == last prefill row)."""
import math

import numpy as np
import pytest
import torch

import block_sparse_streaming_amd as ssa
import oracle
from block_sparse_streaming_amd import inputs
from tests.gpu_util import assert_lse, assert_parity, compact_paged, host, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
PAT = dict(block=128, sink=1, local=7)


def _cfg(dtype, Hq, Hkv, d_qk, d_v, latent=False, seed=0):
    return inputs.DecodeConfig("case", dtype, Hq, Hkv, d_qk, d_v, latent, seed)


def _check(cfg, inp, pattern, full=False, what="", page_size=inputs.PAGE_SIZE):
    say("decode", what, "full" if full else "ssa", cfg.dtype, cfg.Hq, cfg.Hkv, cfg.d_qk, cfg.d_v,
        "lens", inp.lens[:8], "...", len(inp.lens), pattern)
    if full:
        o, lse = ssa.full_decode(inp.q, inp.k_cache, inp.v_cache, inp.page_table, inp.ctx_lens,
                                 scale=cfg.scale, return_lse=True)
    else:
        o, lse = ssa.decode(inp.q, inp.k_cache, inp.v_cache, inp.page_table, inp.ctx_lens,
                            **pattern, scale=cfg.scale, return_lse=True)
    torch.cuda.synchronize()
    kc, vc, table = compact_paged(inp.k_cache, inp.v_cache, inp.table_np, inp.lens, page_size,
                                  pattern["block"], pattern["sink"], pattern["local"], full,
                                  latent_dv=cfg.d_v if cfg.latent else None)
    ro, rl = oracle.decode_paged(host(inp.q), kc, vc, table, np.array(inp.lens, np.int32),
                                 **(dict(block=1, sink=0, local=1) if full else pattern),
                                 scale=cfg.scale, full=full)
    assert_parity(o, ro, cfg.dtype, what)
    assert_lse(lse, rl, cfg.dtype, what)
    return o, lse


EDGE_LENS = (1, 127, 128, 129, 1023, 1024, 1025, 5000)


@pytest.mark.parametrize("full", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_edge_lengths_mha(dtype, full):
    cfg = _cfg(dtype, 4, 4, 128, 128, seed=21)
    inp = inputs.decode_inputs(cfg, DEV, lens=EDGE_LENS + (0,), spare_pages=3)
    _check(cfg, inp, PAT, full, what=f"edge {dtype}")


@pytest.mark.parametrize("pattern", [dict(block=128, sink=0, local=1), dict(block=64, sink=2, local=3),
                                     dict(block=100, sink=1, local=4), dict(block=128, sink=1, local=40),
                                     dict(block=16, sink=3, local=9)],
                         ids=lambda p: f"b{p['block']}s{p['sink']}l{p['local']}")
def test_patterns(pattern):
    cfg = _cfg(torch.bfloat16, 2, 2, 128, 128, seed=22)
    inp = inputs.decode_inputs(cfg, DEV, lens=(1, 100, 700, 3000, 9999))
    _check(cfg, inp, pattern, what=str(pattern))


@pytest.mark.parametrize("group", [2, 4, 8])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_gqa_and_head_dims(group, d):
    if group * d > 1024:
        pytest.skip("no compiled variant (group * d_v > 1024)")
    cfg = _cfg(torch.bfloat16, 2 * group, 2, d, d, seed=23 + d + group)
    inp = inputs.decode_inputs(cfg, DEV, lens=(333, 2048, 4100))
    _check(cfg, inp, PAT, what=f"gqa{group} d{d}")
    _check(cfg, inp, PAT, full=True, what=f"gqa{group} d{d} full")


@pytest.mark.parametrize("page_size", [16, 64, 256])
def test_page_sizes(page_size):
    cfg = _cfg(torch.bfloat16, 4, 4, 128, 128, seed=24)
    inp = inputs.decode_inputs(cfg, DEV, lens=(1, 1000, 1025, 3333), page_size=page_size)
    _check(cfg, inp, PAT, what=f"page {page_size}", page_size=page_size)
    _check(cfg, inp, PAT, full=True, what=f"page {page_size} full", page_size=page_size)


@pytest.mark.parametrize("group", [16, 32, 64, 128])
def test_latent_small(group):
    cfg = _cfg(torch.bfloat16, group, 1, 576, 512, latent=True, seed=25 + group)
    inp = inputs.decode_inputs(cfg, DEV, lens=(1, 130, 1024, 1500, 4097))
    _check(cfg, inp, PAT, what=f"latent g{group}")
    _check(cfg, inp, PAT, full=True, what=f"latent g{group} full")


def test_latent_two_kv_heads():
    cfg = _cfg(torch.bfloat16, 32, 2, 576, 512, latent=True, seed=26)
    inp = inputs.decode_inputs(cfg, DEV, lens=(777, 2000))
    _check(cfg, inp, PAT, what="latent 2 kv heads")


@pytest.mark.parametrize("page_size", [1, 2])
def test_latent_tiny_pages_wide_table(page_size):
    """Pages of 1-2 tokens under a page table 131072 columns wide: the full
    decode plan's split is then bounded by how many page ids one work-group
    keeps (the split would otherwise cover more than 256 pages)."""
    cfg = _cfg(torch.bfloat16, 64, 1, 576, 512, latent=True, seed=27 + page_size)
    lens = (3000, 1, 2500, 4097)
    inp = inputs.decode_inputs(cfg, DEV, lens=lens, page_size=page_size)
    wide = np.zeros((len(lens), 131072), np.int32)
    wide[:, :inp.table_np.shape[1]] = inp.table_np
    inp = inputs.DecodeInputs(inp.q, inp.k_cache, inp.v_cache, torch.from_numpy(wide).to(DEV),
                              inp.ctx_lens, wide, lens)
    _check(cfg, inp, PAT, what=f"latent P{page_size}", page_size=page_size)
    _check(cfg, inp, PAT, full=True, what=f"latent P{page_size} full", page_size=page_size)


def test_latent_128k_full_size():
    """32 sequences x 131072 tokens, shuffled pages: SSA decode on every
    sequence; full decode called on all 32 (the split plan the benchmark
    times: 8,192-token splits, 16 per row) and checked on two of them (the
    oracle's cost is the limit)."""
    cfg = inputs.DECODE_LATENT_128K
    inp = inputs.decode_inputs(cfg, DEV)
    _check(cfg, inp, PAT, what=cfg.name)
    say("decode", cfg.name, "full, all 32 sequences")
    o, lse = ssa.full_decode(inp.q, inp.k_cache, inp.v_cache, inp.page_table, inp.ctx_lens,
                             scale=cfg.scale, return_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    sub = [0, 17]
    kc, vc, table = compact_paged(inp.k_cache, inp.v_cache, inp.table_np[sub],
                                  tuple(inp.lens[i] for i in sub), inputs.PAGE_SIZE, 1, 0, 1, True,
                                  latent_dv=cfg.d_v)
    q_sub = host(inp.q[torch.tensor(sub, device=DEV)].contiguous())
    ro, rl = oracle.decode_paged(q_sub, kc, vc, table, np.array([inp.lens[i] for i in sub], np.int32),
                                 block=1, sink=0, local=1, scale=cfg.scale, full=True)
    idx = torch.tensor(sub, device=DEV)
    assert_parity(o[idx], ro, cfg.dtype, cfg.name + " full (rows 0, 17 of 32)")
    assert_lse(lse[idx], rl, cfg.dtype, cfg.name + " full (rows 0, 17 of 32)")


def test_ragged_full_size():
    cfg = inputs.DECODE_RAGGED
    inp = inputs.decode_inputs(cfg, DEV)
    assert min(inp.lens) < 1024
    _check(cfg, inp, PAT, what=cfg.name)


@pytest.mark.parametrize("dtype,group,page_size,pattern,full", [
    (torch.bfloat16, 1, 128, PAT, False),
    (torch.float32, 1, 16, dict(block=64, sink=1, local=1), False),      # 128-token window: one split
    (torch.bfloat16, 4, 64, dict(block=32, sink=2, local=2), False),     # 128-token window: one split
    (torch.bfloat16, 8, 128, dict(block=16, sink=1, local=3), False),    # 64-token window: one split
    (torch.bfloat16, 2, 16, PAT, True),                                   # full, 256-token table: one split
])
def test_many_rows(dtype, group, page_size, pattern, full):
    """Calls with hundreds of (sequence, kv head) rows and lengths from 0 up,
    GQA groups, page sizes, fp32 and bf16; the windows of at most 128 tokens
    (and the full decode over a 256-token table) fit one split, whose result
    the split kernel writes without a merge."""
    hkv = 16 if group == 1 else 8
    B = -(-560 // hkv)
    rng = np.random.default_rng(300 + group)
    top = 256 if full else 3000
    lens = [0, 1, 127, 128, 129, 255, 256] + [int(x) for x in rng.integers(0, top + 1, B - 7)]
    lens = [min(x, top) for x in lens]
    cfg = _cfg(dtype, hkv * group, hkv, 128, 128, seed=31 + group)
    inp = inputs.decode_inputs(cfg, DEV, lens=tuple(lens), spare_pages=2, page_size=page_size)
    _check(cfg, inp, pattern, full, what=f"many rows {dtype} G{group} page{page_size} {pattern} full={full}",
           page_size=page_size)


def test_page_order_and_poison_invariance():
    """Two physical page orders give bit-identical output; NaN in every page
    slot outside the window leaves the output finite and bit-identical."""
    cfg = _cfg(torch.bfloat16, 4, 4, 128, 128, seed=27)
    lens = (1, 900, 1025, 5000, 20000)
    a = inputs.decode_inputs(cfg, DEV, lens=lens, seed=27)
    o1 = ssa.decode(a.q, a.k_cache, a.v_cache, a.page_table, a.ctx_lens, **PAT)
    # same logical contents under another page permutation
    table2, n2 = inputs.page_table_for(lens, 128, seed=999, spare_pages=5)
    k2 = torch.full((n2,) + tuple(a.k_cache.shape[1:]), float("nan"), dtype=cfg.dtype, device=DEV)
    v2 = torch.full((n2,) + tuple(a.v_cache.shape[1:]), float("nan"), dtype=cfg.dtype, device=DEV)
    for b, L in enumerate(lens):
        npg = -(-L // 128)
        src = torch.from_numpy(a.table_np[b, :npg].astype(np.int64)).to(DEV)
        dst = torch.from_numpy(table2[b, :npg].astype(np.int64)).to(DEV)
        k2[dst] = a.k_cache[src]
        v2[dst] = a.v_cache[src]
    o2 = ssa.decode(a.q, k2, v2, torch.from_numpy(table2).to(DEV), a.ctx_lens, **PAT)
    assert torch.equal(o1, o2)
    # poison everything outside each sequence's window
    k3, v3 = k2.clone(), v2.clone()
    for b, L in enumerate(lens):
        j = np.arange(-(-L // 128) * 128)
        keep = (j < L) & ((j // 128 < 1) | (j // 128 > (L - 1) // 128 - 7))
        pages = torch.from_numpy(table2[b, j[~keep] // 128].astype(np.int64)).to(DEV)
        slots = torch.from_numpy((j[~keep] % 128).astype(np.int64)).to(DEV)
        k3[pages, slots] = float("nan")
        v3[pages, slots] = float("nan")
    o3 = ssa.decode(a.q, k3, v3, torch.from_numpy(table2).to(DEV), a.ctx_lens, **PAT)
    assert torch.isfinite(o3.float()).all()
    assert torch.equal(o1, o3)


def test_ssa_equals_full_for_short_contexts():
    """L <= (s+l)*b: the window is the whole context (bf16 outputs equal up to
    the split order of the two calls, so compare at the parity tolerance)."""
    for latent in (False, True):
        cfg = (_cfg(torch.bfloat16, 64, 1, 576, 512, latent=True, seed=28) if latent
               else _cfg(torch.bfloat16, 8, 8, 128, 128, seed=28))
        inp = inputs.decode_inputs(cfg, DEV, lens=(1, 64, 512, 1000, 1024))
        o_s = ssa.decode(inp.q, inp.k_cache, inp.v_cache, inp.page_table, inp.ctx_lens, **PAT)
        o_f = ssa.full_decode(inp.q, inp.k_cache, inp.v_cache, inp.page_table, inp.ctx_lens)
        diff = (o_s.float() - o_f.float()).abs().max().item()
        assert diff <= 2e-2, diff


def test_decode_matches_last_prefill_row():
    """Decode at context L equals row L-1 of a prefill over the same keys."""
    H, d = 4, 128
    for L in (1, 129, 1024, 1500, 4000):
        g = inputs.generator(DEV, 30 + L)
        q = inputs.randn((1, L, H, d), torch.bfloat16, DEV, g)
        k = inputs.randn((1, L, H, d), torch.bfloat16, DEV, g)
        v = inputs.randn((1, L, H, d), torch.bfloat16, DEV, g)
        o_p = ssa.prefill(q, k, v, **PAT)
        npg = -(-L // 128)
        table, n = inputs.page_table_for((L,), 128, seed=L)
        kc = torch.zeros((n, 128, H, d), dtype=torch.bfloat16, device=DEV)
        vc = torch.zeros_like(kc)
        pad = npg * 128 - L
        kp = torch.nn.functional.pad(k[0], (0, 0, 0, 0, 0, pad)).view(npg, 128, H, d)
        vp = torch.nn.functional.pad(v[0], (0, 0, 0, 0, 0, pad)).view(npg, 128, H, d)
        idx = torch.from_numpy(table[0, :npg].astype(np.int64)).to(DEV)
        kc[idx] = kp
        vc[idx] = vp
        o_d = ssa.decode(q[:, L - 1].contiguous(), kc, vc, torch.from_numpy(table).to(DEV),
                         torch.tensor([L], dtype=torch.int32, device=DEV), **PAT)
        diff = (o_d.float() - o_p[:, L - 1].float()).abs().max().item()
        assert diff <= 2e-2, (L, diff)


@pytest.mark.gpu
@pytest.mark.parametrize("latent", [False, True])
def test_context_length_clamped_to_table_row(latent):
    """A context length past the page table's capacity (max_pages x
    page_size) attends as the capacity: bit-identical to the call at exactly
    the capacity, and the other sequence is unaffected. (Were the length not
    clamped, sequence 0 would read sequence 1's table row, still inside the
    table.)"""
    page, max_pages = 16, 8
    cap = page * max_pages
    g = torch.Generator(device=DEV).manual_seed(91)
    if latent:
        Hq, Hkv, dqk, dv = 16, 1, 576, 512
    else:
        Hq, Hkv, dqk, dv = 4, 2, 128, 128
    n_pages = 2 * max_pages
    kc = torch.randn(n_pages, page, Hkv, dqk, device=DEV, generator=g).bfloat16()
    vc = kc if latent else torch.randn(n_pages, page, Hkv, dv, device=DEV, generator=g).bfloat16()
    perm = torch.randperm(n_pages, generator=torch.Generator().manual_seed(92)).to(torch.int32)
    table = perm.view(2, max_pages).to(DEV)
    q = torch.randn(2, Hq, dqk, device=DEV, generator=g).bfloat16()
    say("decode clamp", "latent" if latent else "mha", cap)
    for full in (False, True):
        call = ssa.full_decode if full else ssa.decode
        kw = {} if full else dict(block=16, sink=1, local=3)
        if latent:
            kw["scale"] = 1.0 / math.sqrt(dqk)
            vv = kc[..., :dv]
        else:
            vv = vc
        ref, ref_lse = call(q, kc, vv, table, torch.tensor([cap, 100], dtype=torch.int32, device=DEV),
                            return_lse=True, **kw)
        got, got_lse = call(q, kc, vv, table, torch.tensor([cap + 37, 100], dtype=torch.int32, device=DEV),
                            return_lse=True, **kw)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), ("full" if full else "ssa")
        assert torch.equal(got_lse, ref_lse), ("full" if full else "ssa")
