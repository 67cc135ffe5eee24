"""Pins of the oracle's ``extend`` (new tokens of each sequence against a
paged cache) against routes that do not go through it.

* a chunk that is the whole sequence equals the oracle's prefill over the
  contiguous K/V (itself pinned) and the brute-force masked softmax;
* a ragged batch (chunks of 0, 1, 3, 40 rows and whole sequences, shuffled
  pages) matches brute force row by row, each row at its own position;
* one-row chunks equal ``decode_paged``;
* the page order does not matter;
* malformed prefix sums and chunks longer than their context are rejected.
"""
import numpy as np
import pytest

import oracle
from tests.bruteforce import block_set_mask, masked_attention
from tests.test_oracle import _page


def _rand(rng, *shape):
    return rng.standard_normal(shape).astype(np.float32)


def test_whole_sequence_chunk_is_prefill():
    rng = np.random.default_rng(600)
    L, Hq, Hkv, d = 300, 4, 2, 8
    q, k, v = _rand(rng, 1, L, Hq, d), _rand(rng, 1, L, Hkv, d), _rand(rng, 1, L, Hkv, d)
    kc, vc, table = _page([k[0]], [v[0]], [L], 16, rng, spare=3)
    kw = dict(block=16, sink=1, local=3, scale=0.35)
    o, lse = oracle.extend(q[0], kc, vc, table, np.array([L], np.int32), np.array([0, L]), **kw)
    po, pl, _ = oracle.prefill(q, k, v, **kw)
    np.testing.assert_allclose(o, po[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, pl[0].T, rtol=0, atol=1e-12)
    M = block_set_mask(L, 16, 1, 3)
    for h in range(Hq):
        bo, _, bl = masked_attention(q[0, :, h], k[0, :, h // 2], v[0, :, h // 2], M, 0.35)
        np.testing.assert_allclose(o[:, h], bo, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[:, h], bl, rtol=0, atol=1e-12)


@pytest.mark.parametrize("b,s,l,ps", [(8, 1, 3, 16), (5, 2, 2, 7), (16, 0, 2, 1)])
def test_ragged_chunks_match_bruteforce(b, s, l, ps):
    rng = np.random.default_rng(610 + b)
    lens = [90, 41, 5, 200, 64, 3]
    qlens = [3, 40, 5, 1, 0, 3]          # a whole sequence, an empty chunk, one-row chunks
    Hq, Hkv, dk, dv = 4, 2, 8, 6
    ks = [_rand(rng, L, Hkv, dk) for L in lens]
    vs = [_rand(rng, L, Hkv, dv) for L in lens]
    kc, vc, table = _page(ks, vs, lens, ps, rng, spare=4)
    cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    q = _rand(rng, int(cu[-1]), Hq, dk)
    o, lse = oracle.extend(q, kc, vc, table, np.array(lens, np.int32), cu, block=b, sink=s,
                           local=l, scale=0.4)
    for bb, (L, n) in enumerate(zip(lens, qlens)):
        M = block_set_mask(L, b, s, l)
        for r in range(n):
            p, row = L - n + r, cu[bb] + r
            for h in range(Hq):
                g = h // (Hq // Hkv)
                bo, _, bl = masked_attention(q[row, h][None], ks[bb][:, g], vs[bb][:, g], M[p:p + 1], 0.4)
                np.testing.assert_allclose(o[row, h], bo[0], rtol=0, atol=1e-12)
                np.testing.assert_allclose(lse[row, h], bl[0], rtol=0, atol=1e-12)


def test_one_row_chunks_are_decode_and_page_order_is_irrelevant():
    rng = np.random.default_rng(620)
    lens = [130, 1, 1025]
    Hq, Hkv, d = 2, 1, 8
    ks = [_rand(rng, L, Hkv, d) for L in lens]
    vs = [_rand(rng, L, Hkv, d) for L in lens]
    q = _rand(rng, len(lens), Hq, d)
    cl = np.array(lens, np.int32)
    cu = np.arange(len(lens) + 1, dtype=np.int32)
    kc1, vc1, t1 = _page(ks, vs, lens, 128, np.random.default_rng(1))
    kc2, vc2, t2 = _page(ks, vs, lens, 128, np.random.default_rng(2), spare=6)
    o1, l1 = oracle.extend(q, kc1, vc1, t1, cl, cu, scale=0.3)
    o2, l2 = oracle.extend(q, kc2, vc2, t2, cl, cu, scale=0.3)
    od, ld = oracle.decode_paged(q, kc1, vc1, t1, cl, scale=0.3)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.array_equal(o1, od) and np.array_equal(l1, ld)


def test_extend_rejects_bad_prefix_sums():
    rng = np.random.default_rng(630)
    ks, vs = [_rand(rng, 10, 1, 8)], [_rand(rng, 10, 1, 8)]
    kc, vc, table = _page(ks, vs, [10], 4, rng)
    q = _rand(rng, 4, 1, 8)
    cl = np.array([10], np.int32)
    for cu in ([1, 4], [0, 3], [0, 5]):
        with pytest.raises(ValueError):
            oracle.extend(q, kc, vc, table, cl, np.array(cu), block=4, scale=0.5)
    with pytest.raises(ValueError):   # a chunk longer than its context
        oracle.extend(_rand(rng, 11, 1, 8), kc, vc, table, cl, np.array([0, 11]), block=4, scale=0.5)
