"""Helpers for the GPU parity tests: host copies for the oracle and the
tolerances the parity bar fixes (fp32: max |err| <= 1e-5; bf16: max |err| <=
2e-2 and relative Frobenius error <= 5e-3, against the oracle run on the same
bf16-rounded inputs)."""
import sys

import numpy as np
import torch

F32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_REL_FRO = 5e-3
# Log-sum-exp: GPU lse within these of the oracle's means sum_j exp(s_j - lse)
# is 1 to about the same relative error.
LSE_ATOL = {torch.float32: 2e-6, torch.bfloat16: 1e-4}


def say(*args):
    """Name the case before a GPU step, flushed, so a failing run shows it."""
    print("[case]", *args, flush=True)
    sys.stdout.flush()


def host(t: torch.Tensor) -> np.ndarray:
    """Exact host copy for the oracle: float32, or bf16 bit patterns as uint16."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(t.dtype)


def as_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_parity(out: torch.Tensor, ref: np.ndarray, dtype: torch.dtype, what: str = ""):
    got = as_f64(out)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    max_abs = float(err.max()) if err.size else 0.0
    if dtype == torch.float32:
        assert max_abs <= F32_MAX_ABS, f"{what}: max |err| {max_abs:.3e} > {F32_MAX_ABS}"
        return max_abs, None
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    assert max_abs <= BF16_MAX_ABS, f"{what}: max |err| {max_abs:.3e} > {BF16_MAX_ABS}"
    assert rel <= BF16_REL_FRO, f"{what}: rel Frobenius {rel:.3e} > {BF16_REL_FRO}"
    return max_abs, rel


def assert_lse(lse: torch.Tensor, ref: np.ndarray, dtype: torch.dtype, what: str = ""):
    got = lse.detach().cpu().numpy().astype(np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    # empty contexts: both sides report -inf
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"{what}: -inf pattern differs"
    fin = np.isfinite(ref)
    assert np.isfinite(got[fin]).all(), f"{what}: non-finite lse"
    err = float(np.abs(got[fin] - ref[fin]).max()) if fin.any() else 0.0
    assert err <= LSE_ATOL[dtype], f"{what}: lse max |err| {err:.3e}"


def attended_logical_pages(L: int, page_size: int, block: int, sink: int, local: int,
                           full: bool = False) -> np.ndarray:
    """Logical pages holding a key of the last query's window (block-set rule)."""
    if L <= 0:
        return np.zeros(0, dtype=np.int64)
    j = np.arange(L)
    if full:
        keep = np.ones(L, dtype=bool)
    else:
        c, qb = j // block, (L - 1) // block
        keep = (c < sink) | (c > qb - local)
    return np.unique(j[keep] // page_size)


def compact_paged(k_cache, v_cache, table_np, lens, page_size, block, sink, local, full=False,
                  latent_dv=None):
    """Copy to the host only the pages the oracle will read; every other logical
    page points to a NaN page, so a wrong read by the oracle would show."""
    need = [attended_logical_pages(L, page_size, block, sink, local, full) for L in lens]
    return compact_pages(k_cache, v_cache, table_np, need, latent_dv)


def rows_logical_pages(L: int, positions, page_size: int, block: int, sink: int, local: int):
    """Logical pages holding a key that some query at one of `positions`
    (all < L) attends: the sink blocks and [lo(min position), max position]."""
    if len(positions) == 0:
        return np.zeros(0, dtype=np.int64)
    pmin, pmax = int(min(positions)), int(max(positions))
    j = np.arange(pmax + 1)
    lo = max(0, (pmin // block - local + 1) * block)
    keep = (j // block < sink) | (j >= lo)
    return np.unique(j[keep] // page_size)


def compact_pages(k_cache, v_cache, table_np, need, latent_dv=None):
    """Host copy of the logical pages need[b] of each sequence b, renumbered;
    every other page of the table points to a NaN page."""
    B = len(need)
    phys = np.concatenate([table_np[b, need[b]] for b in range(B)] + [np.zeros(0, np.int64)])
    phys_t = torch.from_numpy(phys.astype(np.int64)).to(k_cache.device)
    kh = host(k_cache[phys_t]) if phys.size else None
    dummy = phys.size
    new_table = np.full(table_np.shape, dummy, dtype=np.int32)
    off = 0
    for b in range(B):
        new_table[b, need[b]] = np.arange(off, off + need[b].size, dtype=np.int32)
        off += need[b].size
    shape = (phys.size + 1,) + tuple(k_cache.shape[1:])
    nan_bits = np.uint16(0x7FC0) if kh is None or kh.dtype == np.uint16 else np.float32(np.nan)
    dtype = np.uint16 if k_cache.dtype == torch.bfloat16 else np.float32
    kc = np.full(shape, nan_bits if dtype == np.uint16 else np.nan, dtype=dtype)
    if phys.size:
        kc[:phys.size] = kh
    if latent_dv is not None:
        vc = kc[..., :latent_dv]
    else:
        vh = host(v_cache[phys_t]) if phys.size else None
        vshape = (phys.size + 1,) + tuple(v_cache.shape[1:])
        vc = np.full(vshape, nan_bits if dtype == np.uint16 else np.nan, dtype=dtype)
        if phys.size:
            vc[:phys.size] = vh
    return kc, vc, new_table


def assert_grad_parity(out: torch.Tensor, ref: np.ndarray, what: str = ""):
    """bf16 gradient parity. The relative Frobenius bar is the forward's
    (5e-3). The absolute bar is the forward's 2e-2 scaled by the tensor's
    magnitude when that exceeds 1: a gradient entry is a sum over many rows
    (a sink key's dv collects P_ij dout_i from every later row, with the early
    rows weighted near 1, and reaches a few units), and bf16 rounding of the
    P / dS operands and of the output errs in proportion to that sum."""
    got = as_f64(out)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    if not ref.size:
        return 0.0, 0.0
    err = np.abs(got - ref)
    max_abs = float(err.max())
    scale = max(1.0, float(np.abs(ref).max()))
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    where = np.unravel_index(int(err.argmax()), err.shape)
    msg = (f"{what}: max |err| {max_abs:.3e} at {where} (ref {ref[where]:.4g}), "
           f"bound {BF16_MAX_ABS * scale:.3e}; rel Frobenius {rel:.3e}")
    assert max_abs <= BF16_MAX_ABS * scale, msg
    assert rel <= BF16_REL_FRO, msg
    return max_abs, rel
