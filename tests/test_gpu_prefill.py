"""GPU parity of ssa_prefill against the CPU oracle (called through the C ABI).

Small cases compare every output element; the full-size workloads compare
whole query tiles sampled across the sequence (rows are independent, so each
sampled row is checked exactly)."""
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


def _gen(shape, dtype, seed):
    g = inputs.generator(DEV, seed)
    return inputs.randn(shape, dtype, DEV, g)


def _run_and_check(q, k, v, pattern, scale, rows=None, what=""):
    dtype = q.dtype
    say("prefill", what, tuple(q.shape), tuple(k.shape), tuple(v.shape), pattern, dtype)
    o, lse = ssa.prefill(q, k, v, **pattern, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    ro, rl, _ = oracle.prefill(host(q), host(k), host(v), **pattern, scale=scale, rows=rows)
    if rows is not None:
        idx = torch.as_tensor(rows, device=o.device)
        o = o[:, idx]
        lse = lse[:, :, idx]
    assert_parity(o, ro, dtype, what)
    assert_lse(lse, rl, dtype, what)
    return o


def test_fp32_2k_full():
    cfg = inputs.PREFILL_FP32_2K
    q, k, v = inputs.prefill_inputs(cfg, DEV)
    _run_and_check(q, k, v, inputs.PATTERN, cfg.scale, what=cfg.name)


SMALL = [
    # dtype, B, N, Hq, Hkv, d_qk, d_v, (b, s, l)
    (torch.bfloat16, 1, 2048, 2, 2, 128, 128, (128, 1, 7)),
    (torch.bfloat16, 2, 1500, 4, 2, 128, 128, (128, 1, 7)),     # GQA, ragged tail
    (torch.bfloat16, 1, 2100, 2, 1, 192, 128, (128, 1, 7)),
    (torch.bfloat16, 1, 1000, 2, 2, 64, 64, (128, 1, 7)),       # shorter than the window
    (torch.bfloat16, 1, 1, 1, 1, 128, 128, (128, 1, 7)),        # one token
    (torch.bfloat16, 1, 77, 2, 2, 128, 128, (128, 1, 7)),
    (torch.bfloat16, 1, 1300, 2, 2, 128, 128, (64, 2, 3)),
    (torch.bfloat16, 1, 1300, 2, 2, 128, 128, (16, 1, 4)),      # blocks smaller than a sub-tile
    (torch.bfloat16, 1, 1300, 2, 2, 128, 128, (100, 1, 2)),     # blocks not aligned to tiles
    (torch.bfloat16, 1, 1300, 2, 2, 128, 128, (50, 3, 5)),
    (torch.bfloat16, 1, 1300, 2, 2, 128, 128, (300, 1, 2)),
    (torch.bfloat16, 1, 1300, 2, 2, 128, 128, (128, 0, 1)),     # no sink, own block only
    (torch.bfloat16, 1, 1300, 2, 2, 128, 128, (7, 5, 1)),
    (torch.bfloat16, 1, 1300, 2, 2, 128, 128, (128, 1, 64)),    # window longer than N
    # 64-key blocks, long window: in every late tile the two waves of the
    # upper rows take the loop copy without masks, the two lower ones the
    # general copy (their window starts one block later)
    (torch.bfloat16, 1, 3000, 2, 2, 128, 128, (64, 1, 16)),
    (torch.bfloat16, 1, 3000, 2, 1, 64, 64, (192, 1, 5)),       # window starts inside a tile
    # d_qk = 192 visits the whole local sub-tile pairs in a rotated order;
    # with blocks that are not 128 the rotation meets the loop copy without
    # masks and the general one in the same tile
    (torch.bfloat16, 1, 1700, 2, 2, 192, 128, (64, 1, 16)),
    (torch.bfloat16, 1, 1900, 2, 2, 192, 128, (100, 2, 5)),
    (torch.float32, 1, 1300, 2, 2, 128, 128, (128, 1, 7)),
    (torch.float32, 2, 700, 4, 2, 64, 64, (32, 2, 3)),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"{str(c[0])[6:]}-B{c[1]}N{c[2]}H{c[3]}/{c[4]}"
                         f"-d{c[5]}/{c[6]}-b{c[7][0]}s{c[7][1]}l{c[7][2]}")
def test_small_shapes(case):
    dtype, B, N, Hq, Hkv, dqk, dv, (b, s, l) = case
    seed = 7 + N + 13 * b + s + l
    q = _gen((B, N, Hq, dqk), dtype, seed)
    k = _gen((B, N, Hkv, dqk), dtype, seed + 1)
    v = _gen((B, N, Hkv, dv), dtype, seed + 2)
    _run_and_check(q, k, v, dict(block=b, sink=s, local=l), 1.0 / math.sqrt(dqk), what=str(case))


def test_strided_layout():
    """Head-major storage (strides other than [B, N, H, d] contiguous) and an
    output written into a strided view."""
    N, H, d = 900, 4, 128
    base = _gen((1, H, N, 3 * d), torch.bfloat16, 99)
    q = base[..., :d].transpose(1, 2)
    k = base[..., d:2 * d].transpose(1, 2)
    v = base[..., 2 * d:].transpose(1, 2)
    out_store = torch.zeros((1, H, N, d), dtype=torch.bfloat16, device=DEV)
    out = out_store.transpose(1, 2)
    pattern = dict(block=128, sink=1, local=7)
    ssa.prefill(q, k, v, **pattern, out=out)
    ro, _, _ = oracle.prefill(host(q).copy(), host(k).copy(), host(v).copy(), **pattern,
                              scale=d ** -0.5)
    assert_parity(out, ro, torch.bfloat16, "strided")


def _sample_tiles(num_tiles, fixed, n_random, seed):
    rng = np.random.default_rng(seed)
    fixed = [t for t in fixed if t < num_tiles]
    rest = sorted(set(range(num_tiles)) - set(fixed))
    extra = rng.choice(rest, size=min(n_random, len(rest)), replace=False) if rest else []
    return sorted(set(fixed) | set(int(x) for x in extra))


def test_bf16_32k_sampled_tiles():
    cfg = inputs.PREFILL_BF16_32K
    q, k, v = inputs.prefill_inputs(cfg, DEV)
    tiles = _sample_tiles(cfg.N // 128, [0, 1, 6, 7, 8, 9, 128, 255], 6, 2)
    rows = np.concatenate([np.arange(t * 128, (t + 1) * 128) for t in tiles])
    _run_and_check(q, k, v, inputs.PATTERN, cfg.scale, rows=rows, what=cfg.name)


def test_bf16_256k_stratified_sample():
    """Every head; query blocks 0..8, 1023, 1024, 2047 and 32 seeded random blocks."""
    cfg = inputs.PREFILL_BF16_256K
    q, k, v = inputs.prefill_inputs(cfg, DEV)
    tiles = _sample_tiles(cfg.N // 128, list(range(9)) + [1023, 1024, 2047], 32, 4)
    rows = np.concatenate([np.arange(t * 128, (t + 1) * 128) for t in tiles])
    _run_and_check(q, k, v, inputs.PATTERN, cfg.scale, rows=rows, what=cfg.name)


def _attended_union(rows, N, b, s, l):
    j = np.arange(N)
    used = np.zeros(N, dtype=bool)
    for i in rows:
        used |= (j <= i) & ((j // b < s) | (j // b > i // b - l))
    return used


def test_out_of_window_keys_have_no_effect():
    """Keys outside a 128-row query block's attended set, perturbed by +-1e4,
    leave that block's output bit-identical (masked probabilities are exactly
    zero)."""
    N, H, d, tile = 3000, 2, 128, 17
    pattern = dict(block=128, sink=1, local=7)
    q = _gen((1, N, H, d), torch.bfloat16, 5)
    k = _gen((1, N, H, d), torch.bfloat16, 6)
    v = _gen((1, N, H, d), torch.bfloat16, 7)
    ref = ssa.prefill(q, k, v, **pattern)
    rows = np.arange(tile * 128, min((tile + 1) * 128, N))
    bad = torch.from_numpy(~_attended_union(rows, N, 128, 1, 7)).to(DEV)
    k2, v2 = k.clone(), v.clone()
    k2[:, bad] += 1e4
    v2[:, bad] -= 1e4
    got = ssa.prefill(q, k2, v2, **pattern)
    sl = slice(int(rows[0]), int(rows[-1]) + 1)
    assert torch.equal(got[:, sl], ref[:, sl])


def test_keys_outside_every_window_are_never_read():
    """NaN in every key/value outside the attended sets of a 256-row span of
    queries leaves those rows finite and bit-identical: such keys are never
    loaded."""
    N, H, d = 3000, 2, 128
    pattern = dict(block=128, sink=1, local=7)
    q = _gen((1, N, H, d), torch.bfloat16, 8)
    k = _gen((1, N, H, d), torch.bfloat16, 9)
    v = _gen((1, N, H, d), torch.bfloat16, 10)
    ref = ssa.prefill(q, k, v, **pattern)
    rows = np.arange(2048, 2304)
    bad = torch.from_numpy(~_attended_union(rows, N, 128, 1, 7)).to(DEV)
    k2, v2 = k.clone(), v.clone()
    k2[:, bad] = float("nan")
    v2[:, bad] = float("nan")
    got = ssa.prefill(q, k2, v2, **pattern)
    sl = slice(int(rows[0]), int(rows[-1]) + 1)
    assert torch.isfinite(got[:, sl].float()).all()
    assert torch.equal(got[:, sl], ref[:, sl])


def test_short_sequence_matches_library_causal_attention():
    """N <= (s+l)*b: SSA is causal attention; compare with torch SDPA in float64 on the CPU."""
    N, H, d = 1024, 4, 128
    q = _gen((1, N, H, d), torch.bfloat16, 11)
    k = _gen((1, N, H, d), torch.bfloat16, 12)
    v = _gen((1, N, H, d), torch.bfloat16, 13)
    out = ssa.prefill(q, k, v, block=128, sink=1, local=7)
    qc, kc, vc = (t.cpu().double().transpose(1, 2).contiguous() for t in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(qc, kc, vc, is_causal=True)
    assert_parity(out, ref.transpose(1, 2).numpy(), torch.bfloat16, "sdpa")
