"""Pins of the oracle's backward (gradients of q, k, v) against what the
mathematics fixes, independent of the oracle's own chain rule.

* float64 autograd of a dense masked softmax whose mask is built from the
  block sets (the brute-force route), with GQA, ragged lengths and bf16 bits;
* central finite differences of the oracle's FORWARD (itself pinned), so the
  gradient is checked against the function it differentiates;
* full causal attention through torch's scaled_dot_product_attention backward
  (float64), and the short-sequence case that reduces to it;
* closed forms: the softmax is unchanged when every key of a row moves by the
  same vector, so sum_j dk_j = 0 per kv head; the weights of a row sum to one,
  so sum_j dv_j equals the sum of the group's upstream gradients; equal key
  rows give dq = 0;
* selection: a row's terms reach only the keys it attends.

A dropped term, a wrong sign, a transposed operand, a missing scale or a wrong
GQA group fails at least one of these.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.bruteforce import bf16_bits_to_f32, block_set_mask, f32_to_bf16_bits


def _rand(rng, *shape):
    return rng.standard_normal(shape).astype(np.float32)


def _autograd_reference(q, k, v, dout, mask, scale):
    """dq, dk, dv of sum(dout * o) with o a dense masked softmax attention,
    differentiated by torch autograd in float64. q [N, Hq, d], k/v [N, Hkv, d]."""
    Hq, Hkv = q.shape[1], k.shape[1]
    group = Hq // Hkv
    tq, tk, tv = (torch.tensor(np.asarray(x, np.float64), requires_grad=True) for x in (q, k, v))
    td = torch.tensor(np.asarray(dout, np.float64))
    tm = torch.tensor(mask)
    loss = 0.0
    for h in range(Hq):
        g = h // group
        s = scale * (tq[:, h] @ tk[:, g].T)
        s = s.masked_fill(~tm, float("-inf"))
        o = torch.softmax(s, dim=1) @ tv[:, g]
        loss = loss + (o * td[:, h]).sum()
    loss.backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("seed,b,s,l,N,Hq,Hkv", [
    (0, 4, 1, 2, 37, 2, 1),
    (1, 8, 2, 3, 61, 4, 2),
    (2, 5, 0, 2, 23, 3, 3),
    (3, 16, 1, 7, 150, 2, 2),
    (4, 3, 3, 1, 29, 4, 1),
])
def test_backward_matches_autograd_of_bruteforce(seed, b, s, l, N, Hq, Hkv):
    rng = np.random.default_rng(100 + seed)
    d_qk, d_v = 12, 8
    q, k = _rand(rng, 1, N, Hq, d_qk), _rand(rng, 1, N, Hkv, d_qk)
    v, do = _rand(rng, 1, N, Hkv, d_v), _rand(rng, 1, N, Hq, d_v)
    scale = 0.37
    dq, dk, dv = oracle.backward(q, k, v, do, block=b, sink=s, local=l, scale=scale)
    rq, rk, rv = _autograd_reference(q[0], k[0], v[0], do[0], block_set_mask(N, b, s, l), scale)
    np.testing.assert_allclose(dq[0], rq, rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk[0], rk, rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv[0], rv, rtol=0, atol=1e-11)


def test_backward_bf16_bits_and_strides():
    """bf16 bit patterns and strided views give the gradient of the rounded
    values, the same as float32 copies of them."""
    rng = np.random.default_rng(7)
    N, H, d = 45, 2, 8
    qkv = f32_to_bf16_bits(_rand(rng, 1, N, 3, H, d))
    do = f32_to_bf16_bits(_rand(rng, 1, N, H, d))
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]      # strided views
    got = oracle.backward(q, k, v, do, block=4, sink=1, local=3, scale=0.5)
    ref = oracle.backward(*(np.ascontiguousarray(bf16_bits_to_f32(x)) for x in (q, k, v, do)),
                          block=4, sink=1, local=3, scale=0.5)
    for a, r in zip(got, ref):
        assert np.array_equal(a, r)


def _loss(q, k, v, do, **kw):
    o, _, _ = oracle.prefill(q, k, v, **kw)
    return float((o * do.astype(np.float64)).sum())


def test_backward_matches_finite_differences_of_forward():
    rng = np.random.default_rng(11)
    b, s, l, N, Hq, Hkv, d = 4, 1, 2, 30, 2, 1, 6
    kw = dict(block=b, sink=s, local=l, scale=0.45)
    q, k, v = _rand(rng, 1, N, Hq, d), _rand(rng, 1, N, Hkv, d), _rand(rng, 1, N, Hkv, d)
    do = _rand(rng, 1, N, Hq, d)
    grads = oracle.backward(q, k, v, do, **kw)
    eps = np.float32(2.0 ** -9)
    for which, (x, gx) in enumerate(zip((q, k, v), grads)):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            step = float(xp[idx]) - float(xm[idx])          # exact fp32 difference
            args = [q, k, v]
            args[which] = xp
            lp = _loss(*args, do, **kw)
            args[which] = xm
            lm = _loss(*args, do, **kw)
            fd = (lp - lm) / step
            assert abs(fd - gx[idx]) <= 2e-5 * max(1.0, abs(gx[idx])), (which, idx, fd, gx[idx])


def _sdpa_grads(q, k, v, do, scale):
    """torch SDPA (causal, float64) backward; [N, H, d] numpy in and out."""
    tq, tk, tv = (torch.tensor(np.asarray(x, np.float64)).transpose(0, 1)[None].requires_grad_()
                  for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
    out.backward(torch.tensor(np.asarray(do, np.float64)).transpose(0, 1)[None])
    return tuple(t.grad[0].transpose(0, 1).numpy() for t in (tq, tk, tv))


def test_full_mode_backward_is_sdpa_backward():
    rng = np.random.default_rng(12)
    N, H, d = 200, 2, 8
    q, k, v, do = (_rand(rng, 1, N, H, d) for _ in range(4))
    got = oracle.backward(q, k, v, do, scale=0.3, full=True)
    for a, r in zip(got, _sdpa_grads(q[0], k[0], v[0], do[0], 0.3)):
        np.testing.assert_allclose(a[0], r, rtol=0, atol=1e-11)


@pytest.mark.parametrize("b,s,l,N", [(4, 1, 2, 12), (8, 0, 3, 24), (16, 1, 7, 128)])
def test_short_sequence_backward_is_full_causal(b, s, l, N):
    """N <= (s+l)*b: SSA is full causal attention, and so are its gradients."""
    rng = np.random.default_rng(13)
    q, k, v, do = (_rand(rng, 1, N, 2, 8) for _ in range(4))
    got = oracle.backward(q, k, v, do, block=b, sink=s, local=l, scale=0.35)
    for a, r in zip(got, _sdpa_grads(q[0], k[0], v[0], do[0], 0.35)):
        np.testing.assert_allclose(a[0], r, rtol=0, atol=1e-11)


@pytest.mark.parametrize("b,s,l,Hq,Hkv", [(8, 1, 3, 4, 2), (5, 2, 2, 3, 1), (16, 0, 4, 2, 2)])
def test_backward_closed_form_sums(b, s, l, Hq, Hkv):
    """Shift invariance of each row's softmax gives sum_j dk_j = 0 for every kv
    head; weights summing to one give sum_j dv_j = sum over the group's query
    heads and rows of dout."""
    rng = np.random.default_rng(14)
    N, d = 90, 8
    q, k = _rand(rng, 2, N, Hq, d), _rand(rng, 2, N, Hkv, d)
    v, do = _rand(rng, 2, N, Hkv, d), _rand(rng, 2, N, Hq, d)
    _, dk, dv = oracle.backward(q, k, v, do, block=b, sink=s, local=l, scale=0.5)
    group = Hq // Hkv
    for bb in range(2):
        for g in range(Hkv):
            np.testing.assert_allclose(dk[bb, :, g].sum(axis=0), 0.0, rtol=0, atol=1e-10)
            want = do[bb, :, g * group:(g + 1) * group].astype(np.float64).sum(axis=(0, 1))
            np.testing.assert_allclose(dv[bb, :, g].sum(axis=0), want, rtol=0, atol=1e-10)


def test_equal_keys_give_zero_dq():
    """Every key row equal: each row's scores are constant, so no change of q
    moves the output and dq = 0 exactly up to rounding."""
    rng = np.random.default_rng(15)
    N, d = 70, 8
    q, v, do = _rand(rng, 1, N, 2, d), _rand(rng, 1, N, 1, d), _rand(rng, 1, N, 2, d)
    k = np.broadcast_to(_rand(rng, 1, 1, 1, d), (1, N, 1, d)).copy()
    dq, _, _ = oracle.backward(q, k, v, do, block=8, sink=1, local=2, scale=0.6)
    np.testing.assert_allclose(dq, 0.0, rtol=0, atol=1e-12)


def test_row_terms_reach_only_attended_keys():
    """With one row evaluated, dk and dv vanish outside that row's window, and
    the window's share matches autograd of that row alone."""
    b, s, l, N = 8, 1, 3, 96
    rng = np.random.default_rng(16)
    q, k, v, do = (_rand(rng, 1, N, 1, 8) for _ in range(4))
    M = block_set_mask(N, b, s, l)
    for i in [0, 7, 8, 23, 24, 50, 95]:
        dq, dk, dv = oracle.backward(q, k, v, do, block=b, sink=s, local=l, scale=0.4, rows=[i])
        out = ~M[i]
        assert not dk[0, out].any() and not dv[0, out].any()
        row_mask = np.zeros_like(M)
        row_mask[i] = M[i]
        row_mask[np.arange(N) != i, 0] = True     # other rows: any valid mask, zero upstream
        do_i = np.zeros_like(do[0])
        do_i[i] = do[0, i]
        rq, rk, rv = _autograd_reference(q[0], k[0], v[0], do_i, row_mask, 0.4)
        np.testing.assert_allclose(dq[0, 0], rq[i], rtol=0, atol=1e-12)
        np.testing.assert_allclose(dk[0], rk, rtol=0, atol=1e-12)
        np.testing.assert_allclose(dv[0], rv, rtol=0, atol=1e-12)


def test_backward_rejects_bad_arguments():
    x = np.zeros((1, 4, 1, 2), np.float32)
    with pytest.raises(ValueError):
        oracle.backward(x, x, x, x, block=2, sink=1, local=0, scale=1.0)
    with pytest.raises(ValueError):
        oracle.backward(x, x, x, x, block=2, sink=1, local=1, scale=1.0, rows=[-1])
    with pytest.raises(ValueError):
        oracle.backward(x, x, x, np.zeros((1, 4, 1, 3), np.float32), block=2, scale=1.0)


@pytest.mark.parametrize("seed,b,s,l,N,Hq,Hkv,keys", [
    (0, 4, 1, 2, 37, 2, 1, [0, 1, 2, 3]),                 # the sink block
    (1, 8, 2, 3, 61, 4, 2, [0, 9, 15, 16, 30, 60]),       # sink, local and last keys
    (2, 5, 0, 2, 23, 3, 3, [4, 5, 22]),                   # no sink
    (3, 16, 1, 7, 150, 2, 2, list(range(16))),
])
def test_backward_keys_matches_autograd_of_bruteforce(seed, b, s, l, N, Hq, Hkv, keys):
    """The key-side gradient (dk, dv of chosen keys from all their rows,
    through the forward's lse and output) against float64 autograd of the
    dense block-set mask, and against the full backward's dk / dv."""
    rng = np.random.default_rng(300 + seed)
    d_qk, d_v = 12, 8
    q, k = _rand(rng, 1, N, Hq, d_qk), _rand(rng, 1, N, Hkv, d_qk)
    v, do = _rand(rng, 1, N, Hkv, d_v), _rand(rng, 1, N, Hq, d_v)
    scale = 0.41
    dk, dv = oracle.backward_keys(q, k, v, do, keys, block=b, sink=s, local=l, scale=scale)
    _, rk, rv = _autograd_reference(q[0], k[0], v[0], do[0], block_set_mask(N, b, s, l), scale)
    np.testing.assert_allclose(dk[0], rk[keys], rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv[0], rv[keys], rtol=0, atol=1e-11)
    _, ok, ov = oracle.backward(q, k, v, do, block=b, sink=s, local=l, scale=scale)
    np.testing.assert_allclose(dk[0], ok[0, keys], rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv[0], ov[0, keys], rtol=0, atol=1e-11)


def test_backward_keys_bf16_bits():
    rng = np.random.default_rng(310)
    N, Hq, Hkv, d_qk, d_v = 300, 2, 1, 16, 8
    q, k = f32_to_bf16_bits(_rand(rng, 1, N, Hq, d_qk)), f32_to_bf16_bits(_rand(rng, 1, N, Hkv, d_qk))
    v, do = f32_to_bf16_bits(_rand(rng, 1, N, Hkv, d_v)), f32_to_bf16_bits(_rand(rng, 1, N, Hq, d_v))
    keys = list(range(0, 32)) + [200, 299]
    dk, dv = oracle.backward_keys(q, k, v, do, keys, block=32, sink=1, local=3, scale=0.25)
    _, ok, ov = oracle.backward(q, k, v, do, block=32, sink=1, local=3, scale=0.25)
    np.testing.assert_allclose(dk[0], ok[0, keys], rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv[0], ov[0, keys], rtol=0, atol=1e-11)
