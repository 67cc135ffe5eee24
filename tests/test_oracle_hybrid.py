"""Pins of the oracle's hybrid decode (SSA window plus listed tokens) against
routes that do not go through it.

* an empty list (padding only) is the oracle's paged decode;
* a list of every token outside the window is full-attention decode;
* the HFA construction: the window's decode and a brute-force softmax over
  the listed tokens alone, merged by their log-sum-exp, give the result;
* with block 1, sink 16, local 1024 the window is 16 sink tokens plus the
  last 1,024 tokens, checked by brute force on token sets;
* list order, page order and entries inside the window, past the context or
  negative do not change the result.
"""
import numpy as np
import pytest

import oracle
from tests.bruteforce import masked_attention
from tests.test_oracle import _page


def _rand(rng, *shape):
    return rng.standard_normal(shape).astype(np.float32)


def _setup(rng, lens, Hq, Hkv, dk, dv, ps, spare=3):
    ks = [_rand(rng, L, Hkv, dk) for L in lens]
    vs = [_rand(rng, L, Hkv, dv) for L in lens]
    kc, vc, table = _page(ks, vs, lens, ps, rng, spare=spare)
    q = _rand(rng, len(lens), Hq, dk)
    return q, ks, vs, kc, vc, table


def _window(L, b, s, l):
    j = np.arange(L)
    return (j // b < s) | (j // b > (L - 1) // b - l)


@pytest.mark.parametrize("b,s,l", [(8, 1, 3), (1, 16, 64), (16, 0, 2)])
def test_padding_only_list_is_decode(b, s, l):
    rng = np.random.default_rng(800)
    lens = [300, 1, 57, 999]
    q, ks, vs, kc, vc, table = _setup(rng, lens, 4, 2, 8, 6, 16)
    cl = np.array(lens, np.int32)
    topk = np.full((len(lens), 5), -1, np.int32)
    o, lse = oracle.hybrid_decode(q, kc, vc, table, cl, topk, block=b, sink=s, local=l, scale=0.4)
    od, ld = oracle.decode_paged(q, kc, vc, table, cl, block=b, sink=s, local=l, scale=0.4)
    np.testing.assert_allclose(o, od, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ld, rtol=0, atol=1e-12)


def test_list_of_everything_outside_window_is_full_decode():
    rng = np.random.default_rng(801)
    lens = [400, 130, 33]
    q, ks, vs, kc, vc, table = _setup(rng, lens, 2, 1, 8, 8, 32)
    b, s, l = 16, 1, 2
    K = max(lens)
    topk = np.full((len(lens), K), -1, np.int32)
    for i, L in enumerate(lens):
        out = np.flatnonzero(~_window(L, b, s, l))
        topk[i, :out.size] = rng.permutation(out)
    cl = np.array(lens, np.int32)
    o, lse = oracle.hybrid_decode(q, kc, vc, table, cl, topk, block=b, sink=s, local=l, scale=0.3)
    of, lf = oracle.decode_paged(q, kc, vc, table, cl, scale=0.3, full=True)
    np.testing.assert_allclose(o, of, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lf, rtol=0, atol=1e-12)


def test_merge_of_window_and_list_branches():
    """The two branches computed apart (window: paged decode; list: a dense
    masked softmax over the listed keys) and merged by lse."""
    rng = np.random.default_rng(802)
    lens = [2000, 1500]
    Hq, Hkv = 4, 1
    q, ks, vs, kc, vc, table = _setup(rng, lens, Hq, Hkv, 12, 10, 64)
    b, s, l = 1, 16, 256
    K = 100
    topk = np.zeros((2, K), np.int32)
    for i, L in enumerate(lens):
        topk[i] = rng.choice(np.flatnonzero(~_window(L, b, s, l)), K, replace=False)
    cl = np.array(lens, np.int32)
    o, lse = oracle.hybrid_decode(q, kc, vc, table, cl, topk, block=b, sink=s, local=l, scale=0.25)
    ow, lw = oracle.decode_paged(q, kc, vc, table, cl, block=b, sink=s, local=l, scale=0.25)
    for i, L in enumerate(lens):
        mask = np.zeros((1, L), bool)
        mask[0, topk[i]] = True
        for h in range(Hq):
            ol, _, ll = masked_attention(q[i, h][None], ks[i][:, 0], vs[i][:, 0], mask, 0.25)
            m = max(lw[i, h], ll[0])
            wa, wb = np.exp(lw[i, h] - m), np.exp(ll[0] - m)
            np.testing.assert_allclose(o[i, h], (wa * ow[i, h] + wb * ol[0]) / (wa + wb), rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[i, h], m + np.log(wa + wb), rtol=0, atol=1e-12)


def test_sink16_window1024_is_the_fixed_token_sets():
    """Block 1, sink 16, local 1024: the first 16 and the last 1,024 tokens."""
    rng = np.random.default_rng(803)
    L = 3000
    q, ks, vs, kc, vc, table = _setup(rng, [L], 2, 1, 8, 8, 128)
    listed = rng.choice(np.arange(16, L - 1024), 40, replace=False).astype(np.int32)
    o, lse = oracle.hybrid_decode(q, kc, vc, table, np.array([L], np.int32), listed[None], scale=0.35)
    mask = np.zeros((1, L), bool)
    mask[0, :16] = True
    mask[0, L - 1024:] = True
    mask[0, listed] = True
    for h in range(2):
        ro, _, rl = masked_attention(q[0, h][None], ks[0][:, 0], vs[0][:, 0], mask, 0.35)
        np.testing.assert_allclose(o[0, h], ro[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, h], rl[0], rtol=0, atol=1e-12)


def test_order_pages_and_skipped_entries_do_not_matter():
    rng = np.random.default_rng(804)
    lens = [900, 700]
    Hq, Hkv = 2, 2
    ks = [_rand(rng, L, Hkv, 8) for L in lens]
    vs = [_rand(rng, L, Hkv, 8) for L in lens]
    q = _rand(rng, 2, Hq, 8)
    kc1, vc1, t1 = _page(ks, vs, lens, 16, np.random.default_rng(1))
    kc2, vc2, t2 = _page(ks, vs, lens, 16, np.random.default_rng(2), spare=7)
    kw = dict(block=1, sink=16, local=100, scale=0.3)
    cl = np.array(lens, np.int32)
    base = np.stack([rng.choice(np.arange(16, L - 100), 30, replace=False) for L in lens]).astype(np.int32)
    o1, l1 = oracle.hybrid_decode(q, kc1, vc1, t1, cl, base, **kw)
    o2, l2 = oracle.hybrid_decode(q, kc2, vc2, t2, cl, base[:, ::-1].copy(), **kw)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)
    # entries inside the window, past the context, and padding
    extra = np.array([[3, 899, 5000, -1, -7], [0, 650, 700, -1, 12]], np.int32)
    o3, l3 = oracle.hybrid_decode(q, kc1, vc1, t1, cl, np.concatenate([base, extra], axis=1), **kw)
    np.testing.assert_allclose(o3, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l3, l1, rtol=0, atol=1e-13)
