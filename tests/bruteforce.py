"""Brute-force streaming sparse attention on tiny inputs (numpy, float64).

An independent second route to what the oracle computes, used only to pin the
oracle. The mask is built from the two block SETS themselves, as the LongCat
ZigZag Attention digest (163.com, section 01 part (1), SSA paragraph) describes
them: the sink blocks are the first s blocks, the local blocks of query i are
the l blocks ending at i's own block; a key is attended when its block is in
the union and it is causal. The attention is a dense masked softmax.
"""
import numpy as np


def block_set_mask(N: int, b: int, s: int, l: int) -> np.ndarray:
    """M[i, j] = True iff key j is attended by query i."""
    pos = np.arange(N)
    block_of = pos // b
    M = np.zeros((N, N), dtype=bool)
    for i in range(N):
        qb = i // b
        sink_blocks = set(range(0, s))
        local_blocks = set(range(qb - l + 1, qb + 1))
        chosen = sorted((sink_blocks | local_blocks) & set(range(0, qb + 1)))
        M[i] = np.isin(block_of, chosen) & (pos <= i)
    return M


def masked_attention(q, k, v, mask, scale):
    """q [R, d_qk], k [N, d_qk], v [N, d_v], mask [R, N] -> (o, w, lse)."""
    scores = scale * (q.astype(np.float64) @ k.astype(np.float64).T)
    scores = np.where(mask, scores, -np.inf)
    m = scores.max(axis=1, keepdims=True)
    e = np.where(mask, np.exp(scores - m), 0.0)
    denom = e.sum(axis=1, keepdims=True)
    w = e / denom
    lse = (m + np.log(denom))[:, 0]
    return w @ v.astype(np.float64), w, lse


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even) and return the bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)
