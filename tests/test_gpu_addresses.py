"""Prefill and backward on tensors placed at device addresses whose low 32-bit
word has bit 31 set, or whose rows cross that bit inside a tile.

The forward and backward kernels issue their K / V (and Q / dO) transfers
from a wave-uniform 64-bit base kept in two 32-bit scalar halves; a low
half widened with sign extension would corrupt the high one exactly at such
addresses. The results must equal, bit for bit, those of the same inputs at
the allocator's own addresses (which the parity tests compare with the
oracle)."""
import math

import pytest
import torch

import block_sparse_streaming_amd as ssa
from block_sparse_streaming_amd import inputs
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BIT31 = 0x80000000


class Placer:
    """Views of one 4 GiB + 64 MiB device buffer whose data pointers have a
    chosen low 32-bit word (16-byte aligned, non-overlapping for the targets
    used below)."""

    def __init__(self):
        self.buf = torch.empty((1 << 32) + (64 << 20), dtype=torch.uint8, device=DEV)
        self.base = self.buf.data_ptr()

    def place(self, t: torch.Tensor, low: int) -> torch.Tensor:
        nbytes = t.numel() * t.element_size()
        off = (low - self.base) % (1 << 32)
        assert off % 16 == 0 and off + nbytes <= self.buf.numel()
        view = self.buf[off:off + nbytes].view(t.dtype).view(t.shape)
        view.copy_(t)
        assert (view.data_ptr() & 0xFFFFFFFF) == low % (1 << 32)
        return view


@pytest.fixture(scope="module")
def placer():
    p = Placer()
    yield p
    del p.buf
    torch.cuda.empty_cache()


def _gen(shape, seed):
    g = inputs.generator(DEV, seed)
    return inputs.randn(shape, torch.bfloat16, DEV, g)


# (N, H, d): d = 128 and d = 64 take the scalar-base transfers.
CASES = [(2348, 2, 128), (1900, 3, 64)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"N{c[0]}H{c[1]}d{c[2]}")
def test_prefill_and_backward_at_high_addresses(placer, case):
    N, H, d = case
    pattern = dict(block=128, sink=1, local=7)
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = (_gen((1, N, H, d), 300 + n + d) for n in range(4))
    o_ref, lse_ref = ssa.prefill(q, k, v, **pattern, scale=scale, return_lse=True)
    dq_ref, dk_ref, dv_ref = ssa.prefill_backward(q, k, v, o_ref, lse_ref, do, **pattern, scale=scale)
    torch.cuda.synchronize()

    half = (k.numel() * k.element_size() // 2) & ~255
    # k crosses bit 31 of the low word half way; the other tensors sit above it.
    k2 = placer.place(k, BIT31 - half)
    q2 = placer.place(q, BIT31 + (64 << 20))
    v2 = placer.place(v, BIT31 + (128 << 20))
    do2 = placer.place(do, BIT31 + (192 << 20))
    o2 = placer.place(torch.zeros_like(o_ref), 0xC0000000)
    dq2 = placer.place(torch.zeros_like(q), BIT31 + (256 << 20))
    dk2 = placer.place(torch.zeros_like(k), 0xD0000000)
    dv2 = placer.place(torch.zeros_like(v), 0xE0000000)
    say("addresses", case, hex(k2.data_ptr()), hex(q2.data_ptr()), hex(o2.data_ptr()))

    _, lse2 = ssa.prefill(q2, k2, v2, **pattern, scale=scale, out=o2, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o2, o_ref), "prefill output differs at high addresses"
    assert torch.equal(lse2, lse_ref)
    ssa.prefill_backward(q2, k2, v2, o2, lse2, do2, **pattern, scale=scale, dq=dq2, dk=dk2, dv=dv2)
    torch.cuda.synchronize()
    assert torch.equal(dq2, dq_ref), "dq differs at high addresses"
    assert torch.equal(dk2, dk_ref), "dk differs at high addresses"
    assert torch.equal(dv2, dv_ref), "dv differs at high addresses"
