"""GPU parity of ssa_prefill_dual (SSA attention, full causal attention and
their alpha-mix in one pass) against the CPU oracle, through the C ABI.

Small and mid-size cases compare every element of the five outputs. The 32K
workload, in the launch configuration the benchmark times, compares sampled
query tiles (rows are independent), and checks at every row that the mix is
the stated combination of the two halves and that the SSA half is bitwise the
plain forward's output (the dual kernel visits the SSA keys first, with the
same arithmetic).
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_streaming_amd as ssa
import oracle
from block_sparse_streaming_amd import inputs
from tests.gpu_util import as_f64, assert_lse, assert_parity, host, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BF16 = torch.bfloat16


def _gen(shape, seed):
    return inputs.randn(shape, BF16, DEV, inputs.generator(DEV, seed))


def _problem(B, N, Hq, Hkv, dqk, dv, seed):
    return _gen((B, N, Hq, dqk), seed), _gen((B, N, Hkv, dqk), seed + 1), _gen((B, N, Hkv, dv), seed + 2)


def _check(got, ref, rows, what):
    o_ssa, o_full, o_mix, l_ssa, l_full = got
    r_ssa, rl_ssa, r_full, rl_full, r_mix = ref
    if rows is not None:
        idx = torch.as_tensor(rows, device=DEV)
        o_ssa, o_full, o_mix = o_ssa[:, idx], o_full[:, idx], o_mix[:, idx]
        l_ssa, l_full = l_ssa[:, :, idx], l_full[:, :, idx]
    res = [assert_parity(o_ssa, r_ssa, BF16, what + " o_ssa"),
           assert_parity(o_full, r_full, BF16, what + " o_full"),
           assert_parity(o_mix, r_mix, BF16, what + " o_mix")]
    assert_lse(l_ssa, rl_ssa, BF16, what + " lse_ssa")
    assert_lse(l_full, rl_full, BF16, what + " lse_full")
    say("  max|err| / rel Frobenius:", " ".join(f"{a:.2e}/{r:.2e}" for a, r in res))


def _run(q, k, v, pattern, scale, alpha, rows=None, what=""):
    say("dual", what, tuple(q.shape), tuple(k.shape), tuple(v.shape), pattern, "alpha", alpha)
    got = ssa.prefill_dual(q, k, v, **pattern, scale=scale, alpha=alpha, return_lse=True)
    torch.cuda.synchronize()
    ref = oracle.prefill_dual(host(q), host(k), host(v), **pattern, scale=scale, alpha=alpha,
                              rows=rows)
    _check(got, ref, rows, what)
    return got


SMALL = [
    # B, N, Hq, Hkv, d_qk, d_v, (b, s, l), alpha
    (1, 2048, 2, 2, 128, 128, (128, 1, 7), 0.5),
    (2, 1500, 4, 2, 128, 128, (128, 1, 7), 0.25),     # GQA, ragged tail
    (1, 2100, 2, 1, 192, 128, (128, 1, 7), 0.8),      # d_qk = 192
    (1, 3000, 2, 2, 64, 64, (128, 1, 7), 0.1),
    (1, 1, 1, 1, 128, 128, (128, 1, 7), 0.5),         # one token
    (1, 77, 2, 2, 128, 128, (128, 1, 7), 0.5),        # shorter than the window: halves equal
    (1, 1300, 2, 2, 128, 128, (64, 2, 3), 0.0),
    (1, 1300, 2, 2, 128, 128, (16, 1, 4), 1.0),       # blocks smaller than a sub-tile
    (1, 1300, 2, 2, 128, 128, (100, 1, 2), 0.6),      # blocks not aligned to tiles
    (1, 1300, 2, 2, 128, 128, (50, 3, 5), 0.4),       # sink straddles a key tile
    (1, 1300, 2, 2, 128, 128, (128, 0, 1), 0.5),      # no sink, own block only
    (1, 1300, 2, 2, 128, 128, (7, 5, 1), 0.3),
    (1, 1300, 2, 2, 128, 128, (300, 1, 2), 0.7),      # sink spans several key tiles
    (1, 700, 8, 2, 64, 64, (32, 2, 3), 0.5),          # GQA group 4
    (1, 900, 2, 2, 192, 128, (128, 12, 1), 0.5),      # every key is a sink key
    (1, 3000, 2, 2, 128, 128, (64, 1, 16), 0.5),      # waves of one tile take different loop copies
    (1, 3000, 2, 1, 64, 64, (192, 1, 5), 0.5),        # window starts inside a tile
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"B{c[0]}N{c[1]}H{c[2]}/{c[3]}-d{c[4]}/{c[5]}"
                         f"-b{c[6][0]}s{c[6][1]}l{c[6][2]}-a{c[7]}")
def test_small_shapes(case):
    B, N, Hq, Hkv, dqk, dv, (b, s, l), alpha = case
    q, k, v = _problem(B, N, Hq, Hkv, dqk, dv, seed=4000 + N + 7 * b + s + l)
    _run(q, k, v, dict(block=b, sink=s, local=l), 1.0 / math.sqrt(dqk), alpha, what=str(case))


def test_without_mix_and_lse():
    """o_mix and both lse outputs are optional."""
    q, k, v = _problem(1, 1000, 2, 2, 128, 128, seed=4100)
    say("dual without mix")
    o_ssa, o_full = ssa.prefill_dual(q, k, v, block=64, sink=1, local=3)
    torch.cuda.synchronize()
    r_ssa, _, r_full, _, _ = oracle.prefill_dual(host(q), host(k), host(v), block=64, sink=1,
                                                 local=3, scale=128 ** -0.5)
    assert_parity(o_ssa, r_ssa, BF16, "o_ssa")
    assert_parity(o_full, r_full, BF16, "o_full")


def test_strided_inputs_and_outputs():
    """q, k, v views of one packed tensor; the three outputs views of one
    packed output tensor."""
    B, N, H, d = 1, 1100, 2, 128
    qkv = _gen((B, N, 3, H, d), 4200)
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    outs = torch.full((B, N, 3, H, d), float("nan"), dtype=BF16, device=DEV)
    pattern = dict(block=64, sink=1, local=4)
    say("dual strided", tuple(qkv.shape))
    ssa.prefill_dual(q, k, v, **pattern, alpha=0.35, out=(outs[:, :, 0], outs[:, :, 1], outs[:, :, 2]))
    torch.cuda.synchronize()
    r_ssa, _, r_full, _, r_mix = oracle.prefill_dual(host(q), host(k), host(v), **pattern,
                                                     scale=d ** -0.5, alpha=0.35)
    assert_parity(outs[:, :, 0], r_ssa, BF16, "o_ssa")
    assert_parity(outs[:, :, 1], r_full, BF16, "o_full")
    assert_parity(outs[:, :, 2], r_mix, BF16, "o_mix")


def test_full_size_32k_sampled():
    """The 32K, 16-head, d=128 workload: sampled query tiles of two heads
    against the oracle, every row checked for the mix and for the SSA half
    matching the plain forward bit for bit."""
    cfg = inputs.PREFILL_BF16_32K
    q, k, v = inputs.prefill_inputs(cfg, DEV)
    alpha = 0.375
    say("dual full size", cfg.name)
    o_ssa, o_full, o_mix, l_ssa, l_full = ssa.prefill_dual(q, k, v, **inputs.PATTERN, scale=cfg.scale,
                                                           alpha=alpha, return_lse=True)
    o_plain, l_plain = ssa.prefill(q, k, v, **inputs.PATTERN, scale=cfg.scale, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o_ssa.view(torch.int16), o_plain.view(torch.int16)), "SSA half differs"
    assert torch.equal(l_ssa, l_plain)
    # the mix at every row, from the two stored halves (each rounded to bf16)
    for h in range(cfg.Hq):
        want = alpha * o_full[:, :, h].float() + (1 - alpha) * o_ssa[:, :, h].float()
        err = (o_mix[:, :, h].float() - want).abs().max().item()
        assert err <= 2 ** -7 * (1 + want.abs().max().item()), f"head {h}: mix off by {err:.3e}"
    assert torch.isfinite(o_full).all() and torch.isfinite(l_full).all()
    heads = [0, 15]
    tiles = [0, 7, 8, 131, 255]
    rows = np.concatenate([np.arange(t * 128, min(cfg.N, t * 128 + 128)) for t in tiles])
    sl = lambda t: host(t[:, :, heads].contiguous())  # noqa: E731
    ref = oracle.prefill_dual(sl(q), sl(k), sl(v), **inputs.PATTERN, scale=cfg.scale, alpha=alpha,
                              rows=rows)
    idx = torch.as_tensor(rows, device=DEV)
    got = (o_ssa[:, idx][:, :, heads], o_full[:, idx][:, :, heads], o_mix[:, idx][:, :, heads],
           l_ssa[:, heads][:, :, idx], l_full[:, heads][:, :, idx])
    _check(got, ref, None, cfg.name)
