"""Seeded random sweep of prefill and backward shapes and patterns against the
oracle: sequence lengths, batch, grouped heads, head dims, dtypes and
(block, sink, local) drawn at random (fixed seed), so that combinations the
hand-picked cases do not list are also compared element by element."""
import math

import numpy as np
import pytest
import torch

import block_sparse_streaming_amd as ssa
import oracle
from block_sparse_streaming_amd import inputs
from tests.gpu_util import assert_grad_parity, assert_lse, assert_parity, host, say

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
