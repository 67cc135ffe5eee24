"""ssa_decode_noalloc (the decode entry point for callers that cannot
allocate: it runs in the library's fixed per-GPU scratch) against ssa_decode
with a caller workspace, through the C ABI: the same kernels and split plan,
so the outputs and lse must be bit-identical. Two calls in a row, the second
with a smaller input, since the scratch keeps the last call's contents."""
import numpy as np
import pytest
import torch

import block_sparse_streaming_amd as ssa
from block_sparse_streaming_amd import inputs
from tests.gpu_util import say

DEV = "cuda:0"


def _pair(cfg, lens, what):
    inp = inputs.decode_inputs(cfg, DEV, lens=lens)
    say("noalloc", what, cfg.Hq, cfg.Hkv, cfg.d_qk, cfg.d_v, "lens", lens)
    o_ref, l_ref = ssa.decode(inp.q, inp.k_cache, inp.v_cache, inp.page_table, inp.ctx_lens,
                              **inputs.PATTERN, scale=cfg.scale, return_lse=True)
    o, l = ssa.decode_noalloc(inp.q, inp.k_cache, inp.v_cache, inp.page_table, inp.ctx_lens,
                              **inputs.PATTERN, scale=cfg.scale, return_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    assert torch.equal(o, o_ref), what
    assert torch.equal(l, l_ref), what


@pytest.mark.gpu
@pytest.mark.parametrize("latent", [True, False])
def test_noalloc_matches_workspace_call(latent):
    if latent:
        cfg = inputs.DecodeConfig("noalloc", torch.bfloat16, 64, 1, 576, 512, True, 5151)
        first, second = (131072,) * 8 + (5000, 777), (3000, 130, 1)
    else:
        cfg = inputs.DecodeConfig("noalloc", torch.bfloat16, 16, 16, 128, 128, False, 5152)
        first, second = (40000, 9000, 1025, 1024, 300), (2000, 129)
    _pair(cfg, first, "first call")
    _pair(cfg, second, "second call, smaller")


@pytest.mark.gpu
def test_noalloc_rejects_calls_beyond_the_scratch():
    """A call whose workspace would exceed the 32 MiB scratch returns
    SSA_ERR_WORKSPACE and launches nothing (200 sequences x 64 heads at
    d = 128: 8 splits of fp32 partial outputs, 52 MB)."""
    B, H, d = 200, 64, 128
    assert ssa.decode_workspace_size(torch.bfloat16, B, H, H, d, d, 128, 8) > 32 << 20
    q = torch.zeros((B, H, d), dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros((4, 128, H, d), dtype=torch.bfloat16, device=DEV)
    table = torch.zeros((B, 8), dtype=torch.int32, device=DEV)
    lens = torch.ones((B,), dtype=torch.int32, device=DEV)
    out = torch.full((B, H, d), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ssa.SSAError) as e:
        ssa.decode_noalloc(q, kc, kc, table, lens, out=out)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
