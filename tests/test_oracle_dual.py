"""Pins of the oracle's calibration forward (SSA, full causal attention and
their alpha-mix) against routes that do not go through the oracle.

* the SSA half equals the brute-force masked softmax built from the block sets;
* the full half equals torch's scaled_dot_product_attention (causal, float64);
* the two halves are consistent with the keys SSA leaves out: merging the SSA
  softmax with a brute-force softmax over the complement keys (causal and not
  selected) by their lse gives the full result, lse included;
* alpha = 0 and alpha = 1 return the two halves exactly, and a middle alpha
  equals the mix of the two independent routes;
* a sequence no longer than the (s + l) * b window has SSA = full attention.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.bruteforce import block_set_mask, masked_attention


def _rand(rng, *shape):
    return rng.standard_normal(shape).astype(np.float32)


def _sdpa(q, k, v, scale):
    """Causal SDPA in float64; [N, H, d] numpy in, [N, H, d_v] out."""
    tq, tk, tv = (torch.tensor(np.asarray(x, np.float64)).transpose(0, 1)[None] for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
    return o[0].transpose(0, 1).numpy()


CASES = [  # seed, N, b, s, l, Hq, Hkv
    (0, 53, 4, 1, 2, 2, 1),
    (1, 97, 8, 2, 3, 4, 2),
    (2, 40, 5, 0, 2, 1, 1),
    (3, 150, 16, 1, 7, 2, 2),
    (4, 61, 3, 3, 1, 3, 3),
]


@pytest.mark.parametrize("seed,N,b,s,l,Hq,Hkv", CASES)
def test_dual_halves_match_independent_routes(seed, N, b, s, l, Hq, Hkv):
    rng = np.random.default_rng(500 + seed)
    d_qk, d_v, scale = 10, 6, 0.41
    q, k, v = _rand(rng, 1, N, Hq, d_qk), _rand(rng, 1, N, Hkv, d_qk), _rand(rng, 1, N, Hkv, d_v)
    o_ssa, lse_ssa, o_full, lse_full, o_mix = oracle.prefill_dual(
        q, k, v, block=b, sink=s, local=l, scale=scale, alpha=0.3)
    M = block_set_mask(N, b, s, l)
    causal = np.tril(np.ones((N, N), dtype=bool))
    comp = causal & ~M
    group = Hq // Hkv
    for h in range(Hq):
        g = h // group
        bo, _, bl = masked_attention(q[0, :, h], k[0, :, g], v[0, :, g], M, scale)
        np.testing.assert_allclose(o_ssa[0, :, h], bo, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse_ssa[0, h], bl, rtol=0, atol=1e-12)
        fo = _sdpa(q[0, :, h:h + 1], k[0, :, g:g + 1], v[0, :, g:g + 1], scale)[:, 0]
        np.testing.assert_allclose(o_full[0, :, h], fo, rtol=0, atol=1e-12)
        # merge of the SSA softmax and the complement softmax by lse
        has_c = comp.any(axis=1)
        co, _, cl = masked_attention(q[0, has_c, h], k[0, :, g], v[0, :, g], comp[has_c], scale)
        want_o, want_l = bo.copy(), bl.copy()
        m = np.maximum(bl[has_c], cl)
        ws, wc = np.exp(bl[has_c] - m), np.exp(cl - m)
        want_o[has_c] = (ws[:, None] * bo[has_c] + wc[:, None] * co) / (ws + wc)[:, None]
        want_l[has_c] = m + np.log(ws + wc)
        np.testing.assert_allclose(o_full[0, :, h], want_o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse_full[0, h], want_l, rtol=0, atol=1e-12)
        np.testing.assert_allclose(o_mix[0, :, h], 0.3 * fo + 0.7 * bo, rtol=0, atol=1e-12)


def test_alpha_ends_return_each_half():
    rng = np.random.default_rng(510)
    q, k, v = (_rand(rng, 2, 70, 2, 8) for _ in range(3))
    kw = dict(block=8, sink=1, local=2, scale=0.5)
    o_ssa, _, o_full, _, m0 = oracle.prefill_dual(q, k, v, alpha=0.0, **kw)
    _, _, _, _, m1 = oracle.prefill_dual(q, k, v, alpha=1.0, **kw)
    assert np.array_equal(m0, o_ssa) and np.array_equal(m1, o_full)
    assert oracle.prefill_dual(q, k, v, **kw)[4] is None
    for bad in (-0.1, 1.5):
        with pytest.raises(ValueError):
            oracle.prefill_dual(q, k, v, alpha=bad, **kw)


@pytest.mark.parametrize("b,s,l,N", [(4, 1, 2, 12), (16, 1, 7, 128), (8, 0, 3, 20)])
def test_short_sequence_ssa_equals_full(b, s, l, N):
    """Every causal key lies in the window: both halves coincide."""
    rng = np.random.default_rng(520)
    q, k, v = (_rand(rng, 1, N, 2, 8) for _ in range(3))
    o_ssa, lse_ssa, o_full, lse_full, _ = oracle.prefill_dual(q, k, v, block=b, sink=s, local=l,
                                                              scale=0.3)
    np.testing.assert_allclose(o_ssa, o_full, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse_ssa, lse_full, rtol=0, atol=1e-13)
