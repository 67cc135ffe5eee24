"""Seeded random sweeps of the paths whose hand-picked cases go shape family
by shape family: hybrid_decode (latent and MHA / GQA heads, list lengths,
padding, page sizes, windows), ssa_extend (chunks from one row to several
tiles, so both kernels, page sizes, patterns) and the dual forward (lengths,
GQA, head dims, patterns, alpha). Each case is compared with the oracle
element by element through the same checks as the family's own test file."""
import math

import numpy as np
import pytest
import torch

from tests.gpu_util import say
from tests.test_gpu_dual import _problem as dual_problem
from tests.test_gpu_dual import _run as dual_run
from tests.test_gpu_extend import _inp as extend_inp
from tests.test_gpu_extend import _run as extend_run
from tests.test_gpu_hybrid import _case as hybrid_case

pytestmark = pytest.mark.gpu

LAT_DQK, LAT_DV = 576, 512


def _pattern(rng):
    return dict(block=int(rng.choice([16, 64, 100, 128])), sink=int(rng.integers(0, 3)),
                local=int(rng.integers(1, 9)))


def _mha_heads(rng, dims):
    d = int(rng.choice(dims))
    group = int(rng.choice([g for g in (1, 2, 4, 8) if g * d <= 1024 and not (g == 8 and d == 256)]))
    hkv = int(rng.integers(1, 3))
    return d, hkv * group, hkv


def _draw_hybrid(n_cases: int, seed: int):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n_cases):
        latent = bool(rng.random() < 0.5)
        if latent:
            dtype, d, hq, hkv = torch.bfloat16, LAT_DQK, int(rng.choice([16, 32, 64])), 1
        else:
            dtype = torch.float32 if rng.random() < 0.3 else torch.bfloat16
            d, hq, hkv = _mha_heads(rng, [64, 128, 256])
        lens = tuple(int(x) for x in rng.integers(1, 12000, size=int(rng.integers(1, 4))))
        K = int(rng.integers(1, 600))
        pad = int(rng.integers(0, K // 2 + 1))
        page = int(rng.choice([16, 64, 128, 256]))
        if rng.random() < 0.5:
            pattern = dict(block=1, sink=16, local=int(rng.choice([256, 1024])))
        else:
            pattern = _pattern(rng)
        cases.append((latent, dtype, d, hq, hkv, lens, K, pad, page, pattern, int(rng.integers(1 << 30))))
    return cases


def _hybrid_id(c):
    latent, dtype, d, hq, hkv, lens, K, pad, page, p, _ = c
    return (f"{'latent' if latent else str(dtype)[6:]}-H{hq}/{hkv}-d{d}-{len(lens)}seq-K{K}p{pad}-page{page}"
            f"-b{p['block']}s{p['sink']}l{p['local']}")


@pytest.mark.parametrize("case", _draw_hybrid(10, 20261205), ids=_hybrid_id)
def test_hybrid_random(case):
    latent, dtype, d, hq, hkv, lens, K, pad, page, pattern, seed = case
    dv = LAT_DV if latent else d
    hybrid_case(lens, K, hq, pattern, seed % 100000, page_size=page, pad=pad, Hkv=hkv, dqk=d, dv=dv,
                dtype=dtype)


def _draw_extend(n_cases: int, seed: int):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n_cases):
        kind = rng.random()
        if kind < 0.25:
            dtype, dqk, dv, hq, hkv, latent = torch.bfloat16, LAT_DQK, LAT_DV, int(rng.choice([16, 64])), 1, True
        else:
            latent = False
            dtype = torch.float32 if rng.random() < 0.25 else torch.bfloat16
            dims = [64, 128, 256] + ([192] if dtype == torch.bfloat16 else [])
            dqk, hq, hkv = _mha_heads(rng, dims)
            if dqk == 192:
                dv, hq, hkv = 128, hkv, hkv  # the d_qk = 192 kernels take MHA shapes here
            else:
                dv = dqk
        nseq = int(rng.integers(1, 4))
        lens = [int(x) for x in rng.integers(1, 6000, size=nseq)]
        short = bool(rng.random() < 0.4)
        top = 8 if short else 700
        qlens = [int(rng.integers(1, min(L, top) + 1)) for L in lens]
        page = int(rng.choice([1, 16, 64, 128, 256]))
        cases.append((dtype, dqk, dv, hq, hkv, latent, tuple(lens), tuple(qlens), page, _pattern(rng),
                      int(rng.integers(1 << 30))))
    return cases


def _extend_id(c):
    dtype, dqk, dv, hq, hkv, latent, lens, qlens, page, p, _ = c
    return (f"{'latent' if latent else str(dtype)[6:]}-H{hq}/{hkv}-d{dqk}/{dv}-{len(lens)}seq"
            f"-q{max(qlens)}-page{page}-b{p['block']}s{p['sink']}l{p['local']}")


@pytest.mark.parametrize("case", _draw_extend(10, 20261206), ids=_extend_id)
def test_extend_random(case):
    dtype, dqk, dv, hq, hkv, latent, lens, qlens, page, pattern, seed = case
    inp = extend_inp(lens, qlens, hq, hkv, dqk, dv, dtype, seed % 100000, page_size=page, latent=latent,
                     spare_pages=2)
    extend_run(inp, pattern, 1.0 / math.sqrt(dqk), _extend_id(case), latent_dv=dv if latent else None,
               page_size=page)


def _draw_dual(n_cases: int, seed: int):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n_cases):
        dqk, dv = [(64, 64), (128, 128), (192, 128)][int(rng.integers(3))]
        hkv = int(rng.integers(1, 3))
        group = int(rng.choice([1, 2]))
        n = int(rng.integers(1, 2200))
        alpha = float(np.round(rng.random(), 3))
        cases.append((int(rng.integers(1, 3)), n, hkv * group, hkv, dqk, dv, _pattern(rng), alpha,
                      int(rng.integers(1 << 30))))
    return cases


def _dual_id(c):
    B, n, hq, hkv, dqk, dv, p, alpha, _ = c
    return f"B{B}N{n}H{hq}/{hkv}-d{dqk}/{dv}-b{p['block']}s{p['sink']}l{p['local']}-a{alpha}"


@pytest.mark.parametrize("case", _draw_dual(6, 20261207), ids=_dual_id)
def test_dual_random(case):
    B, n, hq, hkv, dqk, dv, pattern, alpha, seed = case
    say("random dual", _dual_id(case))
    q, k, v = dual_problem(B, n, hq, hkv, dqk, dv, seed % 100000)
    dual_run(q, k, v, pattern, 1.0 / math.sqrt(dqk), alpha, what=_dual_id(case))
