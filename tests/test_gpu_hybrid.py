"""GPU parity of hybrid_decode (SSA window plus listed tokens, merged by
log-sum-exp) against the CPU oracle, through the C ABI, on the latent decode
shape (MFMA split kernel) and on MHA / GQA shapes in bf16 and fp32 (VALU split
kernel). The oracle reads only the pages of the window and of the listed
tokens; every other page is NaN, so a wrong page read would show. Lists are
distinct positions drawn from the whole context: entries that fall inside the
window are skipped by the kernel and absorbed by the oracle's union; padding
(-1) and positions past the context are skipped by both.
"""
import numpy as np
import pytest
import torch

import block_sparse_streaming_amd as ssa
import oracle
from block_sparse_streaming_amd import inputs
from tests.gpu_util import assert_lse, assert_parity, compact_pages, host, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
LAT_DQK, LAT_DV = 576, 512


def _needed_pages(L, lst, P, b, s, l):
    if L <= 0:
        return np.zeros(0, np.int64)
    j = np.arange(L)
    keep = (j // b < s) | (j // b > (L - 1) // b - l)
    keep[lst[(lst >= 0) & (lst < L)]] = True
    return np.unique(j[keep] // P)


def _case(lens, K, Hq, pattern, seed, *, page_size=inputs.PAGE_SIZE, pad=0, extra=None, rows=None,
          Hkv=1, dqk=LAT_DQK, dv=LAT_DV, dtype=torch.bfloat16):
    latent = dqk == LAT_DQK
    inp = inputs.extend_inputs(lens, (1,) * len(lens), Hq, Hkv, dqk, dv, dtype, DEV, seed,
                               page_size=page_size, latent=latent, spare_pages=2)
    lst = inputs.token_lists(lens, K, seed + 1, pad_per_row=pad)
    if extra is not None:
        lst = np.concatenate([lst, extra], axis=1)
    topk = torch.from_numpy(lst).to(DEV)
    scale = dqk ** -0.5
    say("hybrid", "lens", lens[:6], len(lens), "K", lst.shape[1], "Hq", Hq, "Hkv", Hkv, "d", dqk, dv, dtype,
        pattern, "page", page_size)
    o, lse = ssa.hybrid_decode(inp.q, inp.k_cache, inp.v_cache, inp.page_table, inp.ctx_lens, topk,
                               **pattern, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    rows = np.arange(len(lens)) if rows is None else np.asarray(rows)
    need = [_needed_pages(lens[b], lst[b], page_size, pattern["block"], pattern["sink"], pattern["local"])
            if b in set(rows.tolist()) else np.zeros(0, np.int64) for b in range(len(lens))]
    kc, vc, table = compact_pages(inp.k_cache, inp.v_cache, inp.table_np, need,
                                  latent_dv=LAT_DV if latent else None)
    ro, rl = oracle.hybrid_decode(host(inp.q)[rows], kc, vc, table[rows], np.array(lens)[rows],
                                  lst[rows], **pattern, scale=scale)
    idx = torch.as_tensor(rows, device=DEV)
    assert_parity(o[idx], ro, dtype, "hybrid")
    assert_lse(lse[idx], rl, dtype, "hybrid lse")
    return o, lse


def test_lsa_configuration_context_edges():
    """16 sink tokens, a 1,024-token window, 1,024 listed tokens; contexts
    from one token to past the fixed budget."""
    lens = (1, 16, 17, 1040, 1041, 2064, 5000, 40000)
    _case(lens, 1024, 64, inputs.HYBRID_PATTERN, seed=900)


@pytest.mark.parametrize("K", [1, 37, 128, 300])
def test_list_lengths(K):
    """Lists shorter than a split, ragged in the last split, exactly one
    split, several splits."""
    _case((3000, 9000, 129), K, 64, inputs.HYBRID_PATTERN, seed=910 + K)


def test_padding_and_skipped_entries():
    """Half of each list is padding; extra entries inside the window, at and
    past the context length and negative are skipped."""
    lens = (4000, 2500, 1100)
    extra = np.array([[3, 3999, 4000, 10 ** 6, -5], [0, 2400, 2500, -1, 15],
                      [1099, 16, 1100, -1, -1]], np.int32)
    _case(lens, 200, 64, inputs.HYBRID_PATTERN, seed=920, pad=100, extra=extra)


@pytest.mark.parametrize("Hq", [16, 128])
def test_head_counts(Hq):
    _case((6000, 1500), 256, Hq, inputs.HYBRID_PATTERN, seed=930 + Hq)


@pytest.mark.parametrize("pattern", [dict(block=128, sink=1, local=7), dict(block=64, sink=2, local=3)],
                         ids=lambda p: f"b{p['block']}s{p['sink']}l{p['local']}")
def test_ssa_window_with_list(pattern):
    _case((7000, 300, 20000), 512, 64, pattern, seed=940 + pattern["block"])


@pytest.mark.parametrize("page_size", [16, 64])
def test_page_sizes(page_size):
    _case((5000, 1200), 400, 64, inputs.HYBRID_PATTERN, seed=950 + page_size, page_size=page_size)


def test_empty_list_equals_ssa_decode_bitwise():
    """A list of padding only adds splits with no attended key: the merge
    gives them weight zero, and the result is ssa_decode's, bit for bit."""
    lens = (3000, 70000, 1)
    inp = inputs.extend_inputs(lens, (1,) * 3, 64, 1, LAT_DQK, LAT_DV, torch.bfloat16, DEV, 960,
                               latent=True)
    topk = torch.full((3, 256), -1, dtype=torch.int32, device=DEV)
    say("hybrid empty list")
    o, lse = ssa.hybrid_decode(inp.q, inp.k_cache, inp.v_cache, inp.page_table, inp.ctx_lens, topk,
                               **inputs.HYBRID_PATTERN, return_lse=True)
    od, ld = ssa.decode(inp.q, inp.k_cache, inp.v_cache, inp.page_table, inp.ctx_lens,
                        **inputs.HYBRID_PATTERN, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), od.view(torch.int16))
    assert torch.equal(lse, ld)


def test_full_size_workload_sampled():
    """The benchmark's workload: 32 sequences at 128K tokens, 64 heads, the
    LSA budget; four sampled sequences against the oracle."""
    lens = (inputs.EXTEND_MTP_LEN,) * 32
    _case(lens, inputs.HYBRID_K, 64, inputs.HYBRID_PATTERN, seed=inputs.HYBRID_SEED, rows=[0, 7, 19, 31])


def test_widest_list_splits():
    """128 sequences: the planner widens the splits to 1,024 tokens, the most
    the latent kernel's LDS table of listed rows holds; 1,000 listed tokens
    per row leave a padded tail in that table. Eight sampled rows against the
    oracle (the short contexts among them too)."""
    rng = np.random.default_rng(971)
    lens = tuple(int(x) for x in rng.integers(1500, 9000, size=128))
    lens = lens[:5] + (1, 17, 1040) + lens[8:]
    assert ssa.hybrid_decode_workspace_size(torch.bfloat16, 128, 64, 1, LAT_DQK, LAT_DV, inputs.PAGE_SIZE,
                                            max(-(-L // inputs.PAGE_SIZE) for L in lens), 1000) > 0
    _case(lens, 1000, 64, inputs.HYBRID_PATTERN, seed=972, rows=[0, 5, 6, 7, 63, 64, 100, 127])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("Hq,Hkv,d", [(4, 4, 128), (8, 2, 64), (8, 2, 256), (16, 2, 128)])
def test_mha_gqa_shapes(dtype, Hq, Hkv, d):
    """The VALU split kernel with a list: GQA groups 1, 4 and 8, head dims 64,
    128 and 256, bf16 and fp32, contexts around and beyond the window, a
    half-padded list with skipped entries."""
    if Hq // Hkv == 8 and d == 256:
        pytest.skip("no compiled variant (group * d_v > 1024)")
    lens = (1, 1040, 1041, 3000, 20000)
    extra = np.array([[0, 1, 5, -1], [3, 1039, 1040, -1], [1040, 2000, 17, -9], [2999, 3000, 16, 15],
                      [19999, 5, 10 ** 6, -1]], np.int32)
    _case(lens, 300, Hq, inputs.HYBRID_PATTERN, seed=970 + Hq + d, pad=50, extra=extra, Hkv=Hkv, dqk=d, dv=d,
          dtype=dtype)


def test_mha_ssa_window_with_list():
    _case((7000, 300, 20000), 512, 4, dict(block=128, sink=1, local=7), seed=980, Hkv=4, dqk=128, dv=128)
