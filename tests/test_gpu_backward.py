"""GPU parity of ssa_prefill_backward against the CPU oracle (through the C ABI).

The forward runs on the GPU first (its o and lse feed the backward, as in
training); the oracle recomputes everything from q, k, v and dout in double.
Small and mid-size cases compare every element of dq, dk and dv. The full-size
workloads compare sampled query tiles (dq rows are independent) and sampled
key tiles past the sink (their dk/dv rows take terms only from the rows
[k0, (k1-1)//b*b + l*b), which the oracle evaluates), and check the sums that
hold at any size: sum_j dk_j = 0 and sum_j dv_j = sum_i dout_i per kv head.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_streaming_amd as ssa
import oracle
from block_sparse_streaming_amd import inputs
from tests.gpu_util import assert_grad_parity, host, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _gen(shape, dtype, seed):
    g = inputs.generator(DEV, seed)
    return inputs.randn(shape, dtype, DEV, g)


def _problem(B, N, Hq, Hkv, dqk, dv, seed, dtype=torch.bfloat16):
    q = _gen((B, N, Hq, dqk), dtype, seed)
    k = _gen((B, N, Hkv, dqk), dtype, seed + 1)
    v = _gen((B, N, Hkv, dv), dtype, seed + 2)
    do = _gen((B, N, Hq, dv), dtype, seed + 3)
    return q, k, v, do


def _gpu_backward(q, k, v, do, pattern, scale, **kw):
    o, lse = ssa.prefill(q, k, v, **pattern, scale=scale, return_lse=True)
    return ssa.prefill_backward(q, k, v, o, lse, do, **pattern, scale=scale, **kw)


def _check_all(q, k, v, do, pattern, scale, what):
    say("backward", what, tuple(q.shape), tuple(k.shape), tuple(v.shape), pattern)
    dq, dk, dv = _gpu_backward(q, k, v, do, pattern, scale)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.backward(host(q), host(k), host(v), host(do), **pattern, scale=scale)
    res = [assert_grad_parity(x, r, what + " " + n) for x, r, n in ((dq, rq, "dq"), (dk, rk, "dk"),
                                                                  (dv, rv, "dv"))]
    say("  max|err| / rel Frobenius:", " ".join(f"{a:.2e}/{r:.2e}" for a, r in res))
    return dq, dk, dv


SMALL = [
    # B, N, Hq, Hkv, d_qk, d_v, (b, s, l)
    (1, 2048, 2, 2, 128, 128, (128, 1, 7)),
    (2, 1500, 4, 2, 128, 128, (128, 1, 7)),      # GQA, ragged tail
    (1, 2100, 2, 1, 192, 128, (128, 1, 7)),      # GQA group 2, d_qk = 192
    (1, 1000, 2, 2, 64, 64, (128, 1, 7)),        # shorter than the window
    (1, 1, 1, 1, 128, 128, (128, 1, 7)),         # one token
    (1, 77, 2, 2, 128, 128, (128, 1, 7)),        # less than a sub-tile
    (1, 1300, 2, 2, 128, 128, (64, 2, 3)),
    (1, 1300, 2, 2, 128, 128, (16, 1, 4)),       # blocks smaller than a sub-tile; 3 sink chunks
    (1, 1300, 2, 2, 128, 128, (100, 1, 2)),      # blocks not aligned to tiles
    (1, 1300, 2, 2, 128, 128, (50, 3, 5)),       # sink straddles a key tile
    (1, 1300, 2, 2, 128, 128, (300, 1, 2)),      # sink spans three key tiles
    (1, 1300, 2, 2, 128, 128, (128, 0, 1)),      # no sink, own block only
    (1, 1300, 2, 2, 128, 128, (7, 5, 1)),
    (1, 1300, 2, 2, 128, 128, (128, 1, 64)),     # window longer than N
    (1, 700, 8, 2, 64, 64, (32, 2, 3)),          # GQA group 4
    (1, 900, 2, 2, 192, 128, (128, 12, 1)),      # every key is a sink key
    (1, 1700, 2, 2, 192, 128, (64, 1, 16)),      # d_qk = 192, long window of small blocks
    (1, 1900, 2, 2, 192, 128, (100, 2, 5)),      # d_qk = 192, blocks not aligned to tiles
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"B{c[0]}N{c[1]}H{c[2]}/{c[3]}-d{c[4]}/{c[5]}"
                         f"-b{c[6][0]}s{c[6][1]}l{c[6][2]}")
def test_small_shapes(case):
    B, N, Hq, Hkv, dqk, dv, (b, s, l) = case
    q, k, v, do = _problem(B, N, Hq, Hkv, dqk, dv, seed=3000 + N + 7 * b + s + l)
    _check_all(q, k, v, do, dict(block=b, sink=s, local=l), 1.0 / math.sqrt(dqk), str(case))


@pytest.mark.parametrize("dqk,dv", [(128, 128), (192, 128)])
def test_several_sink_chunks_deployed_pattern(dqk, dv):
    """b=128, s=1, l=7 over 8192 tokens: three sink chunks plus key tiles
    whose rows run into the ragged end."""
    q, k, v, do = _problem(1, 8000, 2, 2, dqk, dv, seed=3100 + dqk)
    _check_all(q, k, v, do, inputs.PATTERN, 1.0 / math.sqrt(dqk), f"N8000 d{dqk}")


def test_strided_inputs_and_outputs():
    """q, k, v views of one packed tensor; gradients written into the views of
    a packed gradient tensor."""
    B, N, H, d = 1, 1100, 2, 128
    qkv = _gen((B, N, 3, H, d), torch.bfloat16, 3200)
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    do = _gen((B, N, H, d), torch.bfloat16, 3201)
    grads = torch.full((B, N, 3, H, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    pattern = dict(block=64, sink=1, local=4)
    say("backward strided", tuple(qkv.shape))
    _gpu_backward(q, k, v, do, pattern, d ** -0.5, dq=grads[:, :, 0], dk=grads[:, :, 1],
                  dv=grads[:, :, 2])
    torch.cuda.synchronize()
    rq, rk, rv = oracle.backward(host(q), host(k), host(v), host(do), **pattern, scale=d ** -0.5)
    assert_grad_parity(grads[:, :, 0], rq, "dq")
    assert_grad_parity(grads[:, :, 1], rk, "dk")
    assert_grad_parity(grads[:, :, 2], rv, "dv")


def test_deterministic_and_workspace_reuse():
    """No atomics: two calls give identical bits, also with a reused,
    dirty workspace."""
    q, k, v, do = _problem(1, 3000, 2, 2, 128, 128, seed=3300)
    pattern = dict(block=32, sink=2, local=3)
    o, lse = ssa.prefill(q, k, v, **pattern, return_lse=True)
    need = ssa.backward_workspace_size(q.dtype, 1, 3000, 2, 2, 128, 128, **pattern)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    say("backward determinism")
    a = ssa.prefill_backward(q, k, v, o, lse, do, **pattern, workspace=ws)
    b = ssa.prefill_backward(q, k, v, o, lse, do, **pattern, workspace=ws)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_rejects_small_workspace():
    q, k, v, do = _problem(1, 600, 2, 2, 128, 128, seed=3400)
    o, lse = ssa.prefill(q, k, v, return_lse=True)
    need = ssa.backward_workspace_size(q.dtype, 1, 600, 2, 2, 128, 128)
    ws = torch.empty(need - 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(ssa.SSAError) as e:
        ssa.prefill_backward(q, k, v, o, lse, do, workspace=ws)
    assert e.value.status == 3


def _head_slice(t, heads):
    return host(t[:, :, heads].contiguous())


def _sampled_full_size(cfg, q_tiles, k_tiles, heads, sink_head=None):
    """Backward at a full workload's shape, checked on sampled tiles of the
    given heads (GQA-free shapes: query head h reads kv head h). With
    sink_head, the first key tile (the sink keys, attended by every row) of
    that head is checked element by element against the oracle over all rows:
    that tile's dk / dv are the chunked partial sums of the finalize launch."""
    pattern = inputs.PATTERN
    b, l = pattern["block"], pattern["local"]
    N = cfg.N
    q, k, v = inputs.prefill_inputs(cfg, DEV)
    do = inputs.prefill_grad(cfg, DEV)
    say("backward full size", cfg.name, "heads", heads)
    dq, dk, dv = _gpu_backward(q, k, v, do, pattern, cfg.scale)
    torch.cuda.synchronize()
    qh, kh, vh, dh = (_head_slice(t, heads) for t in (q, k, v, do))
    # dq on whole query tiles.
    rows = np.concatenate([np.arange(t * 128, min(N, t * 128 + 128)) for t in q_tiles])
    rq, _, _ = oracle.backward(qh, kh, vh, dh, **pattern, scale=cfg.scale, rows=rows)
    idx = torch.as_tensor(rows, device=DEV)
    assert_grad_parity(dq[:, idx][:, :, heads], rq, cfg.name + " dq rows")
    # dk / dv of key tiles past the sink: the rows that attend them.
    for t in k_tiles:
        k0, k1 = t * 128, min(N, t * 128 + 128)
        r1 = min(N, ((k1 - 1) // b + l) * b)
        _, rk, rv = oracle.backward(qh, kh, vh, dh, **pattern, scale=cfg.scale,
                                    rows=np.arange(k0, r1))
        assert_grad_parity(dk[:, k0:k1][:, :, heads], rk[:, k0:k1], f"{cfg.name} dk tile {t}")
        assert_grad_parity(dv[:, k0:k1][:, :, heads], rv[:, k0:k1], f"{cfg.name} dv tile {t}")
    if sink_head is not None:
        hs = [sink_head]
        qs_, ks_, vs_, ds_ = (_head_slice(t, hs) for t in (q, k, v, do))
        k1 = min(N, 128)
        rk, rv = oracle.backward_keys(qs_, ks_, vs_, ds_, np.arange(k1), **pattern, scale=cfg.scale)
        assert_grad_parity(dk[:, :k1][:, :, hs], rk, f"{cfg.name} dk sink tile, head {sink_head}")
        assert_grad_parity(dv[:, :k1][:, :, hs], rv, f"{cfg.name} dv sink tile, head {sink_head}")
        del rk, rv
    # Sums that hold at any size (the sink rows included), per kv head, in
    # double on the device, one head at a time.
    for h in range(cfg.Hkv):
        dkh, dvh = dk[:, :, h].double(), dv[:, :, h].double()
        sum_dk = dkh.sum(dim=1)
        assert (sum_dk.abs() <= 1e-3 * dkh.abs().sum(dim=1).amax()).all(), f"head {h}: sum of dk"
        want = do[:, :, h].double().sum(dim=1)          # GQA-free: one query head per kv head
        err = (dvh.sum(dim=1) - want).abs().max().item()
        assert err <= 1e-3 * want.abs().max().item(), f"head {h}: sum of dv off by {err:.3e}"
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()


def test_full_size_32k_sampled():
    """The 32K, 16-head, d=128 workload in the launch configuration the
    benchmark times."""
    _sampled_full_size(inputs.PREFILL_BF16_32K, q_tiles=[0, 1, 7, 8, 131, 255],
                       k_tiles=[1, 2, 100, 250, 255], heads=[0, 15])


def test_full_size_256k_sampled():
    """The 256K, 64-head, d_qk=192 / d_v=128 workload."""
    _sampled_full_size(inputs.PREFILL_BF16_256K, q_tiles=[0, 8, 1024, 2047],
                       k_tiles=[1, 1023, 2047], heads=[0, 63], sink_head=0)
