"""Seeded random sweeps against the oracle: prefill and backward (sequence
lengths, batch, grouped heads, head dims, dtypes, (block, sink, local)) and
decode (MHA / GQA / latent heads, page sizes, context lengths from 0, SSA and
full attention), drawn at random with fixed seeds, so that combinations the
hand-picked cases do not list are also compared element by element."""
import math

import numpy as np
import pytest
import torch

import block_sparse_streaming_amd as ssa
import oracle
from block_sparse_streaming_amd import inputs
from tests.gpu_util import assert_grad_parity, assert_lse, assert_parity, compact_paged, host, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _draw(n_cases: int, seed: int):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n_cases):
        dtype = torch.float32 if rng.random() < 0.25 else torch.bfloat16
        dims = [(64, 64), (128, 128)] + ([(192, 128)] if dtype == torch.bfloat16 else [])
        d_qk, d_v = dims[rng.integers(len(dims))]
        hkv = int(rng.integers(1, 3))
        group = int(rng.choice([1, 2, 4]))
        block = int(rng.choice([8, 16, 32, 48, 64, 96, 128, 130, 200, 256]))
        sink = int(rng.integers(0, 4))
        local = int(rng.integers(1, 10))
        n = int(rng.integers(1, 2600))
        b = int(rng.integers(1, 3))
        cases.append((dtype, b, n, hkv * group, hkv, d_qk, d_v, (block, sink, local), int(rng.integers(1 << 30))))
    return cases


CASES = _draw(16, 20261203)


def _ids(c):
    return (f"{str(c[0])[6:]}-B{c[1]}N{c[2]}H{c[3]}/{c[4]}-d{c[5]}/{c[6]}"
            f"-b{c[7][0]}s{c[7][1]}l{c[7][2]}")


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_prefill_random(case):
    dtype, B, N, Hq, Hkv, dqk, dv, (b, s, l), seed = case
    g = inputs.generator(DEV, seed)
    q = inputs.randn((B, N, Hq, dqk), dtype, DEV, g)
    k = inputs.randn((B, N, Hkv, dqk), dtype, DEV, g)
    v = inputs.randn((B, N, Hkv, dv), dtype, DEV, g)
    pattern = dict(block=b, sink=s, local=l)
    scale = 1.0 / math.sqrt(dqk)
    say("random prefill", _ids(case))
    o, lse = ssa.prefill(q, k, v, **pattern, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    ro, rl, _ = oracle.prefill(host(q), host(k), host(v), **pattern, scale=scale)
    assert_parity(o, ro, dtype, _ids(case))
    assert_lse(lse, rl, dtype, _ids(case))


BWD_CASES = [c for c in CASES if c[0] == torch.bfloat16][:8]


@pytest.mark.parametrize("case", BWD_CASES, ids=_ids)
def test_backward_random(case):
    _, B, N, Hq, Hkv, dqk, dv, (b, s, l), seed = case
    g = inputs.generator(DEV, seed + 1)
    q = inputs.randn((B, N, Hq, dqk), torch.bfloat16, DEV, g)
    k = inputs.randn((B, N, Hkv, dqk), torch.bfloat16, DEV, g)
    v = inputs.randn((B, N, Hkv, dv), torch.bfloat16, DEV, g)
    do = inputs.randn((B, N, Hq, dv), torch.bfloat16, DEV, g)
    pattern = dict(block=b, sink=s, local=l)
    scale = 1.0 / math.sqrt(dqk)
    say("random backward", _ids(case))
    o, lse = ssa.prefill(q, k, v, **pattern, scale=scale, return_lse=True)
    dq, dk, dvv = ssa.prefill_backward(q, k, v, o, lse, do, **pattern, scale=scale)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.backward(host(q), host(k), host(v), host(do), **pattern, scale=scale)
    for got, ref, name in ((dq, rq, "dq"), (dk, rk, "dk"), (dvv, rv, "dv")):
        assert_grad_parity(got, ref, _ids(case) + " " + name)


def _draw_decode(n_cases: int, seed: int):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n_cases):
        latent = rng.random() < 0.3
        if latent:
            dtype, hkv, group, d_qk, d_v = torch.bfloat16, 1, int(rng.choice([16, 32, 64])), 576, 512
        else:
            dtype = torch.float32 if rng.random() < 0.3 else torch.bfloat16
            d = int(rng.choice([64, 128, 256]))
            group = int(rng.choice([g for g in (1, 2, 4, 8) if g * d <= 1024 and not (g == 8 and d == 256)]))
            hkv, d_qk, d_v = int(rng.integers(1, 3)), d, d
        page = int(rng.choice([1, 16, 64, 128, 256]))
        block = int(rng.choice([16, 64, 100, 128]))
        sink = int(rng.integers(0, 3))
        local = int(rng.integers(1, 9))
        nseq = int(rng.integers(1, 5))
        lens = tuple(int(x) for x in rng.integers(0, 6000, size=nseq))
        full = bool(rng.random() < 0.3)
        cases.append((dtype, hkv * group, hkv, d_qk, d_v, latent, page, (block, sink, local), lens, full,
                      int(rng.integers(1 << 30))))
    return cases


DEC_CASES = _draw_decode(14, 20261204)


def _dec_ids(c):
    dtype, hq, hkv, dqk, dv, latent, page, (b, s, l), lens, full, _ = c
    return (f"{str(dtype)[6:]}-H{hq}/{hkv}-d{dqk}/{dv}{'-latent' if latent else ''}-page{page}"
            f"-b{b}s{s}l{l}-{len(lens)}seq{'-full' if full else ''}")


@pytest.mark.parametrize("case", DEC_CASES, ids=_dec_ids)
def test_decode_random(case):
    dtype, hq, hkv, dqk, dv, latent, page, (b, s, l), lens, full, seed = case
    cfg = inputs.DecodeConfig("random", dtype, hq, hkv, dqk, dv, latent, seed)
    inp = inputs.decode_inputs(cfg, DEV, lens=lens, page_size=page, spare_pages=2)
    pattern = dict(block=b, sink=s, local=l)
    say("random decode", _dec_ids(case), lens)
    if full:
        o, lse = ssa.full_decode(inp.q, inp.k_cache, inp.v_cache, inp.page_table, inp.ctx_lens,
                                 scale=cfg.scale, return_lse=True)
    else:
        o, lse = ssa.decode(inp.q, inp.k_cache, inp.v_cache, inp.page_table, inp.ctx_lens, **pattern,
                            scale=cfg.scale, return_lse=True)
    torch.cuda.synchronize()
    kc, vc, table = compact_paged(inp.k_cache, inp.v_cache, inp.table_np, inp.lens, page, b, s, l, full,
                                  latent_dv=dv if latent else None)
    ro, rl = oracle.decode_paged(host(inp.q), kc, vc, table, np.array(inp.lens, np.int32),
                                 **(dict(block=1, sink=0, local=1) if full else pattern),
                                 scale=cfg.scale, full=full)
    assert_parity(o, ro, dtype, _dec_ids(case))
    assert_lse(lse, rl, dtype, _dec_ids(case))
