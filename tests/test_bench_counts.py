"""Host-side counts of bench.py: the algorithmic work every reported rate is
divided by, and the benchmark's own guards. CPU only.

Each count is checked against the block-set mask of tests/bruteforce.py (the
sink and local block sets as the LongCat ZigZag Attention digest, section 01
part (1), defines them) or against a closed form worked out by hand here.
"""
import json
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

import bench
from tests.bruteforce import block_set_mask

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PATTERNS = [(16, 1, 2), (16, 2, 3), (32, 1, 1), (7, 3, 2), (64, 0, 2), (50, 2, 4), (128, 1, 7)]


@pytest.mark.parametrize("N", [1, 37, 300, 611])
@pytest.mark.parametrize("pattern", PATTERNS)
def test_attended_pairs_is_the_mask_count(N, pattern):
    b, s, l = pattern
    assert bench.attended_pairs(N, b, s, l) == int(block_set_mask(N, b, s, l).sum())


def test_headline_pair_count_closed_form():
    """N = 32768, b = 128, s = 1, l = 7, one head. Block 0 (rows 0..127)
    attends only its causal prefix: 1 + 2 + ... + 128 = 8256 pairs. Blocks
    1..6 attend every earlier key, i + 1 per row: 128 * 128 qb + 8256 per
    block. Blocks 7..255 attend the sink block, the six full blocks before
    their own and their own causal prefix: 7 * 128 + (i % 128) + 1 per row,
    128 * 896 + 8256 = 122944 per block."""
    per_head = 8256 + sum(128 * 128 * qb + 8256 for qb in range(1, 7)) + 249 * 122944
    assert per_head == 31_014_912
    assert bench.attended_pairs(32768, 128, 1, 7) * 16 == per_head * 16 == 496_238_592
    # 2 (d_qk + d_v) flops per pair at d = 128: the headline's 254.07 GFLOP
    assert per_head * 16 * 2 * (128 + 128) == 254_074_159_104


@pytest.mark.parametrize("pattern", PATTERNS)
def test_decode_selection_is_the_last_row_of_the_mask(pattern):
    b, s, l = pattern
    for L in [1, 2, b - 1 if b > 1 else 1, b, b + 1, 5 * b + 3, 400]:
        M = block_set_mask(L, b, s, l)
        assert bench.decode_selected_tokens(L, b, s, l) == int(M[L - 1].sum()), L
    assert bench.decode_selected_tokens(0, 16, 1, 2) == 0


@pytest.mark.parametrize("pattern", PATTERNS)
def test_extend_counts_are_the_mask_rows(pattern):
    b, s, l = pattern
    lens, qlens = [300, 77, 512], [40, 77, 1]
    got = bench.extend_row_counts(lens, qlens, b, s, l)
    want = np.concatenate([block_set_mask(L, b, s, l)[L - n:].sum(axis=1) for L, n in zip(lens, qlens)])
    assert np.array_equal(got, want)
    for L, n in zip(lens, qlens):
        union = int(block_set_mask(L, b, s, l)[L - n:].any(axis=0).sum())
        assert bench.extend_union_tokens(L, n, b, s, l) == union, (L, n)


def test_hybrid_bytes_hand_count():
    """L = 300, b = 16, s = 1, l = 2, pages of 16 tokens. The window is block
    0 (tokens 0..15) and blocks 17, 18 (272..299): 44 rows on pages 0, 17, 18.
    Of the list [0, 5, 100, 299, -1, 350] only 100 lies outside the window
    (-1 is padding, 350 is past the context): one more row and one more page
    id. Bytes: 45 rows x 1152 + q and o (64 heads x (576 + 512) x 2) + 4 page
    ids x 4 + 6 list entries x 4 + one length x 4."""
    lst = np.array([0, 5, 100, 299, -1, 350])
    want = 45 * 1152 + 64 * 1088 * 2 + 4 * 4 + 6 * 4 + 4
    assert want == 191_148
    assert bench.hybrid_bytes([300], [lst], 16, 1, 2, page_size=16, Hq=64) == want


def test_backward_flops_per_pair():
    class Cfg:
        N, B, Hq, d_qk, d_v = 32768, 1, 16, 128, 128
    assert bench.backward_flops(Cfg) == 496_238_592 * 2 * (3 * 128 + 2 * 128)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_record_needs_unchanged_sources(tmp_path, monkeypatch):
    """A traffic record counts only while the kernel sources hash to the value
    stored beside it; an unknown kernel or a changed source gives None."""
    csrc = tmp_path / "block_sparse_streaming_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text("kernel source\n")
    import hashlib
    digest = hashlib.sha256(b"kernel source\n").hexdigest()
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic.json").write_text(json.dumps({
        "k grid=64": {"bytes_per_launch": 1000.0, "sources": ["k.hip"], "source_sha256": digest},
        "m tag": {"bytes_per_launch": 24.0, "sources": ["k.hip"], "source_sha256": digest}}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_traffic(["k grid=64"]) == 1000.0
    assert bench.recorded_traffic(["k grid=64", "m tag"]) == 1024.0
    assert bench.recorded_traffic(["k grid=64", "missing"]) is None
    (csrc / "k.hip").write_text("kernel source, edited\n")
    assert bench.recorded_traffic(["k grid=64"]) is None
    shutil.rmtree(prof)
    assert bench.recorded_traffic(["k grid=64"]) is None
