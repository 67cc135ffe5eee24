"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: a
hand-enumerated literal, the pages' window size, a brute-force masked softmax
built from the block sets, a library routine in a special case the method
reduces to, a closed form, or an invariant. A plausible slip anywhere in the
oracle (an off-by-one in the local window, sink measured in tokens, a dropped
causal mask, a missing scale, a wrong GQA head mapping, L instead of L - 1 in
decode, a wrong page lookup) fails at least one of them.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from tests.bruteforce import (bf16_bits_to_f32, block_set_mask, f32_to_bf16_bits,
                              masked_attention)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "masks.txt")


def _rand(rng, *shape):
    return rng.standard_normal(shape).astype(np.float32)


def _read_golden():
    cases, cur = [], None
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("case"):
                _, b, s, l, n = line.split()
                cur = dict(b=int(b), s=int(s), l=int(l), N=int(n), rows={})
                cases.append(cur)
            else:
                i, keys = line.split(":")
                cur["rows"][int(i)] = [int(x) for x in keys.split()]
    return cases


@pytest.mark.parametrize("case", _read_golden(), ids=lambda c: f"b{c['b']}s{c['s']}l{c['l']}")
def test_mask_literal(case):
    """Hand-enumerated A(i) (tests/golden/masks.txt) equals the oracle's support."""
    b, s, l, N = case["b"], case["s"], case["l"], case["N"]
    rng = np.random.default_rng(1)
    q, k, v = (0.1 * _rand(rng, 1, N, 1, 4) for _ in range(3))
    _, _, w = oracle.prefill(q, k, v, block=b, sink=s, local=l, scale=0.5, weights=True)
    assert len(case["rows"]) == N
    for i, keys in case["rows"].items():
        assert list(np.nonzero(w[0, 0, i])[0]) == keys, f"row {i}"


def test_deployed_window_is_1024_tokens():
    """b=128, s=1, l=7 gives a 1,024-token window (163.com digest, section 01 part (2))."""
    N = 2048
    rng = np.random.default_rng(2)
    q, k, v = (0.05 * _rand(rng, 1, N, 1, 2) for _ in range(3))
    _, _, w = oracle.prefill(q, k, v, block=128, sink=1, local=7, scale=1.0, weights=True)
    counts = (w[0, 0] > 0).sum(axis=1)
    assert counts.max() == 1024
    # rows past the first 8 blocks: sink block + 6 full local blocks + own block prefix
    i = np.arange(1024, N)
    assert np.array_equal(counts[1024:], 128 + 6 * 128 + (i % 128) + 1)
    # per steady-state query block: 7 full tiles plus the causal triangle
    assert counts[1024:1152].sum() == 7 * 128 * 128 + 128 * 129 // 2 == 122944


@pytest.mark.parametrize("seed", range(40))
def test_bruteforce_tiny(seed):
    """Oracle == dense masked softmax over the block-set mask, random tiny shapes."""
    rng = np.random.default_rng(100 + seed)
    b = int(rng.integers(1, 10))
    s = int(rng.integers(0, 4))
    l = int(rng.integers(1, 6))
    N = int(rng.integers(1, 65))
    Hkv = int(rng.choice([1, 2]))
    Hq = Hkv * int(rng.choice([1, 2, 3]))
    d_qk = int(rng.integers(1, 9))
    d_v = int(rng.integers(1, 9))
    B = int(rng.integers(1, 3))
    scale = float(rng.uniform(0.2, 1.5))
    q = _rand(rng, B, N, Hq, d_qk)
    k = _rand(rng, B, N, Hkv, d_qk)
    v = _rand(rng, B, N, Hkv, d_v)
    o, lse, w = oracle.prefill(q, k, v, block=b, sink=s, local=l, scale=scale, weights=True)
    M = block_set_mask(N, b, s, l)
    for bb in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            ro, rw, rl = masked_attention(q[bb, :, h], k[bb, :, g], v[bb, :, g], M, scale)
            np.testing.assert_allclose(o[bb, :, h], ro, rtol=0, atol=1e-12)
            np.testing.assert_allclose(w[bb, h], rw, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[bb, h], rl, rtol=0, atol=1e-12)


def test_strided_inputs_and_bf16_bits():
    """Non-contiguous inputs and bf16 bit patterns give the same result as float32 copies."""
    rng = np.random.default_rng(3)
    B, N, H, d = 2, 40, 2, 8
    full = _rand(rng, B, H, N, 3 * d)           # head-major storage, q|k|v packed per row
    q = full[..., :d].transpose(0, 2, 1, 3)      # [B, N, H, d] views with odd strides
    k = full[..., d:2 * d].transpose(0, 2, 1, 3)
    v = full[..., 2 * d:].transpose(0, 2, 1, 3)
    o1, l1, _ = oracle.prefill(q, k, v, block=4, sink=1, local=2, scale=0.3)
    o2, l2, _ = oracle.prefill(np.ascontiguousarray(q), np.ascontiguousarray(k),
                               np.ascontiguousarray(v), block=4, sink=1, local=2, scale=0.3)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    qb, kb, vb = (f32_to_bf16_bits(np.ascontiguousarray(x)) for x in (q, k, v))
    o3, l3, _ = oracle.prefill(qb, kb, vb, block=4, sink=1, local=2, scale=0.3)
    o4, l4, _ = oracle.prefill(bf16_bits_to_f32(qb), bf16_bits_to_f32(kb), bf16_bits_to_f32(vb),
                               block=4, sink=1, local=2, scale=0.3)
    assert np.array_equal(o3, o4) and np.array_equal(l3, l4)
    M = block_set_mask(N, 4, 1, 2)
    ro, _, _ = masked_attention(bf16_bits_to_f32(qb)[0, :, 1], bf16_bits_to_f32(kb)[0, :, 1],
                                bf16_bits_to_f32(vb)[0, :, 1], M, 0.3)
    np.testing.assert_allclose(o3[0, :, 1], ro, rtol=0, atol=1e-12)


def test_bf16_rounding_helper():
    """The test-side bf16 rounding agrees with torch's round-to-nearest-even."""
    x = np.random.default_rng(4).standard_normal(10000).astype(np.float32) * 100
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), ref)


def _sdpa(q, k, v, scale, causal=True):
    """torch scaled_dot_product_attention in float64; [N, H, d] numpy in and out."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).transpose(0, 1)
                  for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq[None], tk[None], tv[None], is_causal=causal, scale=scale)
    return out[0].transpose(0, 1).numpy()


@pytest.mark.parametrize("b,s,l,N", [(16, 1, 3, 64), (16, 1, 3, 50), (128, 1, 7, 1024),
                                     (8, 2, 2, 32), (5, 0, 4, 20)])
def test_short_sequence_is_full_causal(b, s, l, N):
    """N <= (s+l)*b: SSA reduces to full causal attention (library SDPA, float64)."""
    assert N <= (s + l) * b
    rng = np.random.default_rng(5)
    H, d = 2, 16
    q, k, v = (_rand(rng, 1, N, H, d) for _ in range(3))
    scale = d ** -0.5
    o, _, _ = oracle.prefill(q, k, v, block=b, sink=s, local=l, scale=scale)
    ref = _sdpa(q[0], k[0], v[0], scale)
    np.testing.assert_allclose(o[0], ref, rtol=0, atol=1e-12)


def test_full_mode_is_causal_sdpa():
    rng = np.random.default_rng(6)
    N, H, d = 300, 2, 8
    q, k, v = (_rand(rng, 1, N, H, d) for _ in range(3))
    o, _, _ = oracle.prefill(q, k, v, scale=0.25, full=True)
    np.testing.assert_allclose(o[0], _sdpa(q[0], k[0], v[0], 0.25), rtol=0, atol=1e-12)


@pytest.mark.parametrize("N", [64, 70])
def test_no_sink_one_local_is_blockwise_causal(N):
    """s=0, l=1: each block attends causally within itself only (SDPA per chunk)."""
    b = 16
    rng = np.random.default_rng(7)
    H, d = 2, 8
    q, k, v = (_rand(rng, 1, N, H, d) for _ in range(3))
    o, _, _ = oracle.prefill(q, k, v, block=b, sink=0, local=1, scale=0.4)
    for c0 in range(0, N, b):
        c1 = min(c0 + b, N)
        ref = _sdpa(q[0, c0:c1], k[0, c0:c1], v[0, c0:c1], 0.4)
        np.testing.assert_allclose(o[0, c0:c1], ref, rtol=0, atol=1e-12)


def test_weights_sum_to_one_and_lse():
    rng = np.random.default_rng(8)
    N = 700
    q, k, v = (_rand(rng, 1, N, 1, 8) for _ in range(3))
    _, lse, w = oracle.prefill(q, k, v, block=32, sink=1, local=3, scale=0.35, weights=True)
    np.testing.assert_allclose(w[0, 0].sum(axis=1), 1.0, rtol=0, atol=1e-12)
    # LSE: weights are exp(score - lse)
    scores = 0.35 * (q[0, :, 0].astype(np.float64) @ k[0, :, 0].astype(np.float64).T)
    nz = w[0, 0] > 0
    np.testing.assert_allclose(w[0, 0][nz], np.exp(scores - lse[0, 0][:, None])[nz],
                               rtol=1e-12, atol=0)


def test_out_of_window_keys_have_no_effect():
    """Perturbing K/V outside A(i) by +-1e4 leaves row i bit-identical."""
    b, s, l, N = 32, 1, 3, 600
    rng = np.random.default_rng(9)
    q, k, v = (_rand(rng, 1, N, 2, 8) for _ in range(3))
    M = block_set_mask(N, b, s, l)
    for i in [0, 31, 32, 95, 96, 127, 128, 200, 450, 599]:
        k2, v2 = k.copy(), v.copy()
        outside = ~M[i]
        k2[0, outside] += 1e4 * np.sign(rng.standard_normal(k2[0, outside].shape)).astype(np.float32)
        v2[0, outside] -= 1e4
        o1, l1, _ = oracle.prefill(q, k, v, block=b, sink=s, local=l, scale=0.3, rows=[i])
        o2, l2, _ = oracle.prefill(q, k2, v2, block=b, sink=s, local=l, scale=0.3, rows=[i])
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("b,s,l", [(128, 1, 7), (16, 2, 3), (10, 0, 2), (7, 3, 1)])
def test_zero_keys_give_mean_of_window(b, s, l):
    """K = 0 makes every weight equal, so with V[j] = j the output is the mean
    attended position. The closed form uses the range description
    A(i) = [0, min(sb, i+1)) U [max(sb, (i//b - l + 1) b), i+1)."""
    N = 2100
    q = np.ones((1, N, 1, 4), np.float32)
    k = np.zeros((1, N, 1, 4), np.float32)
    v = np.broadcast_to(np.arange(N, dtype=np.float32)[None, :, None, None], (1, N, 1, 2)).copy()
    o, lse, _ = oracle.prefill(q, k, v, block=b, sink=s, local=l, scale=1.0)
    i = np.arange(N)
    sb = s * b
    a1 = np.minimum(sb, i + 1)                                  # [0, a1)
    lo = np.maximum(sb, (i // b - l + 1) * b)                   # [lo, i+1)
    n2 = np.maximum(0, i + 1 - lo)
    count = a1 + n2
    total = a1 * (a1 - 1) / 2 + n2 * (lo + i) / 2
    np.testing.assert_allclose(o[0, :, 0, 0], total / count, rtol=1e-13, atol=0)
    np.testing.assert_allclose(lse[0, 0], np.log(count), rtol=0, atol=1e-12)


def _page(k_full, v_full, lens, page_size, rng, spare=0):
    """Scatter per-sequence [L, H, d] rows into a shuffled paged cache."""
    B = len(lens)
    pages_per = [-(-L // page_size) for L in lens]
    total = sum(pages_per) + spare
    perm = rng.permutation(total).astype(np.int32)
    max_pages = max(pages_per + [1])
    table = np.zeros((B, max_pages), np.int32)
    H, dk = k_full[0].shape[1:]
    dv = v_full[0].shape[2]
    kc = np.full((total, page_size, H, dk), np.nan, np.float32)
    vc = np.full((total, page_size, H, dv), np.nan, np.float32)
    nxt = 0
    for bb, L in enumerate(lens):
        for p in range(pages_per[bb]):
            phys = perm[nxt]
            nxt += 1
            table[bb, p] = phys
            t0, t1 = p * page_size, min((p + 1) * page_size, L)
            kc[phys, :t1 - t0] = k_full[bb][t0:t1]
            vc[phys, :t1 - t0] = v_full[bb][t0:t1]
    return kc, vc, table


@pytest.mark.parametrize("L", [1, 127, 128, 129, 1023, 1024, 1025, 1300])
def test_decode_equals_last_prefill_row(L):
    """Decode at context L (query at position L-1, paged and shuffled) equals prefill row L-1."""
    rng = np.random.default_rng(10 + L)
    H, d = 2, 8
    q, k, v = (_rand(rng, 1, L, H, d) for _ in range(3))
    o_p, lse_p, _ = oracle.prefill(q, k, v, block=128, sink=1, local=7, scale=0.3, rows=[L - 1])
    kc, vc, table = _page([k[0]], [v[0]], [L], 128, rng, spare=3)
    o_d, lse_d = oracle.decode_paged(q[:, L - 1], kc, vc, table, np.array([L], np.int32),
                                     block=128, sink=1, local=7, scale=0.3)
    np.testing.assert_allclose(o_d, o_p[:, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_d, lse_p[:, :, 0], rtol=0, atol=1e-12)
    o_f, _ = oracle.decode_paged(q[:, L - 1], kc, vc, table, np.array([L], np.int32),
                                 scale=0.3, full=True)
    ref = _sdpa(q[0, L - 1:L], k[0], v[0], 0.3, causal=False)
    np.testing.assert_allclose(o_f[0], ref[0], rtol=0, atol=1e-12)


def test_decode_page_permutation_and_ragged_batch():
    """Different physical page orders give bit-identical decode output; ragged
    batch rows match brute force; L = 0 gives zeros and lse = -inf."""
    rng = np.random.default_rng(11)
    lens = [300, 0, 37, 128, 1000]
    Hq, Hkv, dk, dv, ps = 4, 2, 8, 6, 16
    ks = [_rand(rng, max(L, 1), Hkv, dk) for L in lens]
    vs = [_rand(rng, max(L, 1), Hkv, dv) for L in lens]
    q = _rand(rng, len(lens), Hq, dk)
    kc1, vc1, t1 = _page(ks, vs, lens, ps, np.random.default_rng(1))
    kc2, vc2, t2 = _page(ks, vs, lens, ps, np.random.default_rng(2), spare=5)
    cl = np.array(lens, np.int32)
    o1, l1 = oracle.decode_paged(q, kc1, vc1, t1, cl, block=32, sink=2, local=3, scale=0.4)
    o2, l2 = oracle.decode_paged(q, kc2, vc2, t2, cl, block=32, sink=2, local=3, scale=0.4)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    for bb, L in enumerate(lens):
        if L == 0:
            assert np.all(o1[bb] == 0) and np.all(np.isneginf(l1[bb]))
            continue
        M = block_set_mask(L, 32, 2, 3)[L - 1:L]
        for h in range(Hq):
            g = h // (Hq // Hkv)
            ro, _, rl = masked_attention(q[bb, h][None], ks[bb][:, g], vs[bb][:, g], M, 0.4)
            np.testing.assert_allclose(o1[bb, h], ro[0], rtol=0, atol=1e-12)
            np.testing.assert_allclose(l1[bb, h], rl[0], rtol=0, atol=1e-12)


def test_decode_latent_alias():
    """A latent cache row whose first d_v entries serve as the value (an
    absorbed MLA layout) matches brute force with V = K[:, :d_v]."""
    rng = np.random.default_rng(12)
    L, Hq, dk, dv, ps = 700, 8, 24, 16, 64
    lat = _rand(rng, L, 1, dk)
    kc, _, table = _page([lat], [lat], [L], ps, rng, spare=2)
    vc = kc[..., :dv]                     # a view: same rows, first d_v entries
    q = _rand(rng, 1, Hq, dk)
    o, lse = oracle.decode_paged(q, kc, vc, table, np.array([L], np.int32),
                                 block=64, sink=1, local=7, scale=dk ** -0.5)
    M = block_set_mask(L, 64, 1, 7)[L - 1:L]
    for h in range(Hq):
        ro, _, rl = masked_attention(q[0, h][None], lat[:, 0], lat[:, 0, :dv], M, dk ** -0.5)
        np.testing.assert_allclose(o[0, h], ro[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, h], rl[0], rtol=0, atol=1e-12)


def test_oracle_rejects_bad_arguments():
    x = np.zeros((1, 4, 1, 2), np.float32)
    with pytest.raises(ValueError):
        oracle.prefill(x, x, x, block=2, sink=1, local=0, scale=1.0)
    with pytest.raises(ValueError):
        oracle.prefill(x, x, x, block=0, sink=1, local=1, scale=1.0)
    with pytest.raises(ValueError):
        oracle.prefill(x, x, x, block=2, sink=1, local=1, scale=1.0, rows=[4])
    kc = np.zeros((2, 4, 1, 2), np.float32)
    table = np.array([[0, 5]], np.int32)             # page 5 does not exist
    with pytest.raises(ValueError):
        oracle.decode_paged(np.zeros((1, 1, 2), np.float32), kc, kc, table,
                            np.array([8], np.int32), scale=1.0, block=2)
