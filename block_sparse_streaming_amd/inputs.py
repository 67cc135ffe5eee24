"""Seeded synthetic inputs for the SSA workloads (no attention arithmetic here).

Shared by the tests and the benchmark: both sides of every parity check get
their bytes from these generators. Values are N(0, 1) drawn in fp32 from a
seeded torch generator and rounded once to the compute dtype (bf16 by
round-to-nearest-even). Paged caches deal out a seeded random permutation of
the physical pages to the sequences in logical order.

Workloads (the pages run the method at b=128, s=1, l=7 over 32K-256K contexts
and compare decode kernels at 128K; these shapes stand in for their models):
  1  prefill fp32 : B=1, N=2048,   H=4,  d=64
  2  prefill bf16 : B=1, N=32768,  H=16, d=128
  3  decode  bf16 : B=32, 64 query heads on one 576-dim latent KV head (value =
                    first 512 dims), L=131072 per sequence, 128-token pages
  4  prefill bf16 : B=1, N=262144, H=64, d_qk=192, d_v=128
  5  decode  bf16 : 64 sequences, L log-uniform in [4096, 1048576], plus one
                    sequence with L in [1, 1023]; 16 heads, d=128, 128-token pages
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

PAGE_SIZE = 128
PATTERN = dict(block=128, sink=1, local=7)


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    dtype: torch.dtype
    B: int
    N: int
    Hq: int
    Hkv: int
    d_qk: int
    d_v: int
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d_qk)


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    dtype: torch.dtype
    Hq: int
    Hkv: int
    d_qk: int
    d_v: int
    latent: bool                 # value = first d_v entries of the key row
    seed: int
    lens: tuple = field(default=())

    @property
    def B(self) -> int:
        return len(self.lens)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d_qk)


def ragged_lens(seed: int = 1005) -> tuple:
    """64 context lengths floor(exp(U(ln 4096, ln 1048576))) plus one in [1, 1023]."""
    rng = np.random.default_rng(seed)
    u = rng.uniform(math.log(4096), math.log(1048576), size=64)
    lens = [int(math.floor(math.exp(x))) for x in u]
    lens.append(int(rng.integers(1, 1024)))
    return tuple(lens)


# The workloads, each named by its shape.
PREFILL_FP32_2K = PrefillConfig("prefill_fp32_b1_n2048_h4_d64", torch.float32, 1, 2048, 4, 4, 64, 64, 1001)
PREFILL_BF16_32K = PrefillConfig("prefill_bf16_b1_n32768_h16_d128", torch.bfloat16, 1, 32768, 16, 16, 128,
                                 128, 1002)
DECODE_LATENT_128K = DecodeConfig("decode_bf16_latent_b32_h64_d576_L131072", torch.bfloat16, 64, 1, 576, 512,
                                  True, 1003, lens=(131072,) * 32)
PREFILL_BF16_256K = PrefillConfig("prefill_bf16_b1_n262144_h64_dqk192_dv128", torch.bfloat16, 1, 262144, 64,
                                  64, 192, 128, 1004)
DECODE_RAGGED = DecodeConfig("decode_bf16_ragged_65seq_h16_d128", torch.bfloat16, 16, 16, 128, 128, False,
                             1005, lens=ragged_lens())
WORKLOADS = {c.name: c for c in (PREFILL_FP32_2K, PREFILL_BF16_32K, DECODE_LATENT_128K, PREFILL_BF16_256K,
                                 DECODE_RAGGED)}


def randn(shape, dtype: torch.dtype, device, gen: torch.Generator, chunk_elems: int = 1 << 28):
    """N(0,1) drawn in fp32 and rounded once to ``dtype``; filled in chunks so a
    huge bf16 tensor never needs an fp32 copy of itself."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    for s in range(0, flat.numel(), chunk_elems):
        n = min(chunk_elems, flat.numel() - s)
        flat[s:s + n] = torch.randn(n, generator=gen, device=device, dtype=torch.float32).to(dtype)
    return out


def generator(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def prefill_inputs(cfg: PrefillConfig, device, seed: int | None = None):
    """q [B, N, Hq, d_qk], k [B, N, Hkv, d_qk], v [B, N, Hkv, d_v]."""
    gen = generator(device, cfg.seed if seed is None else seed)
    q = randn((cfg.B, cfg.N, cfg.Hq, cfg.d_qk), cfg.dtype, device, gen)
    k = randn((cfg.B, cfg.N, cfg.Hkv, cfg.d_qk), cfg.dtype, device, gen)
    v = randn((cfg.B, cfg.N, cfg.Hkv, cfg.d_v), cfg.dtype, device, gen)
    return q, k, v


def page_table_for(lens, page_size: int, seed: int, spare_pages: int = 0):
    """Deal a seeded permutation of all physical pages to the sequences.

    Returns (page_table [B, max_pages] int32 numpy, num_pages). Entries past a
    sequence's last page are 0 (never read)."""
    pages_per = [max(1, -(-int(L) // page_size)) for L in lens]
    total = sum(pages_per) + spare_pages
    perm = np.random.default_rng(seed).permutation(total).astype(np.int32)
    table = np.zeros((len(lens), max(pages_per)), dtype=np.int32)
    nxt = 0
    for b, n in enumerate(pages_per):
        table[b, :n] = perm[nxt:nxt + n]
        nxt += n
    return table, total


@dataclass
class DecodeInputs:
    q: torch.Tensor            # [B, Hq, d_qk]
    k_cache: torch.Tensor      # [pages, page_size, Hkv, d_qk]
    v_cache: torch.Tensor      # [pages, page_size, Hkv, d_v] (a view of k_cache when latent)
    page_table: torch.Tensor   # [B, max_pages] int32
    ctx_lens: torch.Tensor     # [B] int32
    table_np: np.ndarray
    lens: tuple


def decode_inputs(cfg: DecodeConfig, device, *, lens=None, seed: int | None = None,
                  spare_pages: int = 0, page_size: int = PAGE_SIZE) -> DecodeInputs:
    lens = tuple(cfg.lens if lens is None else lens)
    seed = cfg.seed if seed is None else seed
    table, num_pages = page_table_for(lens, page_size, seed, spare_pages)
    gen = generator(device, seed)
    q = randn((len(lens), cfg.Hq, cfg.d_qk), cfg.dtype, device, gen)
    k_cache = randn((num_pages, page_size, cfg.Hkv, cfg.d_qk), cfg.dtype, device, gen)
    if cfg.latent:
        v_cache = k_cache[..., :cfg.d_v]
    else:
        v_cache = randn((num_pages, page_size, cfg.Hkv, cfg.d_v), cfg.dtype, device, gen)
    return DecodeInputs(q, k_cache, v_cache, torch.from_numpy(table).to(device),
                        torch.tensor(lens, dtype=torch.int32, device=device), table, lens)


# Chunked prefill workload: four sequences with 32K-128K tokens of context,
# each appending an 8,192-token chunk (16 heads, d = 128, 128-token pages).
EXTEND_CHUNK_LENS = (32768, 65536, 98304, 131072)
EXTEND_CHUNK_QLENS = (8192, 8192, 8192, 8192)
EXTEND_SEED = 1006
# Multi-token decode workload: the latent decode shape (32 sequences at 128K
# tokens, 64 query heads on one 576-wide latent head) with four new tokens
# per sequence (the current token and three draft tokens).
EXTEND_MTP_LEN = 131072
EXTEND_MTP_Q = 4
EXTEND_MTP_SEED = 1007


@dataclass
class ExtendInputs:
    q: torch.Tensor            # [total_q, Hq, d_qk] packed rows of the new tokens
    k_cache: torch.Tensor      # [pages, page_size, Hkv, d_qk]
    v_cache: torch.Tensor      # [pages, page_size, Hkv, d_v] (a view of k_cache when latent)
    page_table: torch.Tensor   # [B, max_pages] int32
    ctx_lens: torch.Tensor     # [B] int32, new tokens included
    cu_q: torch.Tensor         # [B + 1] int32 prefix sums of the chunk lengths
    table_np: np.ndarray
    lens: tuple
    qlens: tuple


def extend_inputs(lens, qlens, Hq: int, Hkv: int, d_qk: int, d_v: int, dtype: torch.dtype, device,
                  seed: int, *, page_size: int = PAGE_SIZE, latent: bool = False,
                  spare_pages: int = 0) -> ExtendInputs:
    """A shuffled paged cache holding each sequence's lens[b] tokens and the
    queries of its last qlens[b] tokens, packed by sequence."""
    lens, qlens = tuple(int(x) for x in lens), tuple(int(x) for x in qlens)
    table, num_pages = page_table_for(lens, page_size, seed, spare_pages)
    gen = generator(device, seed)
    cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    q = randn((int(cu[-1]), Hq, d_qk), dtype, device, gen)
    k_cache = randn((num_pages, page_size, Hkv, d_qk), dtype, device, gen)
    v_cache = k_cache[..., :d_v] if latent else randn((num_pages, page_size, Hkv, d_v), dtype, device, gen)
    return ExtendInputs(q, k_cache, v_cache, torch.from_numpy(table).to(device),
                        torch.tensor(lens, dtype=torch.int32, device=device),
                        torch.from_numpy(cu).to(device), table, lens, qlens)


def token_lists(lens, K: int, seed: int, *, pad_per_row: int = 0) -> np.ndarray:
    """[B, K] int32 lists of distinct token positions drawn uniformly from
    [0, L) of each sequence (an indexer's choice stands in for nothing more
    than that), the last pad_per_row entries of a row and any entry beyond
    L set to -1 (padding)."""
    rng = np.random.default_rng(seed)
    out = np.full((len(lens), K), -1, dtype=np.int32)
    for b, L in enumerate(lens):
        n = max(0, min(K - pad_per_row, int(L)))
        if n:
            out[b, :n] = rng.choice(int(L), n, replace=False)
    return out


# Hybrid decode workload: the latent decode shape (32 sequences at 128K, 64
# query heads on one 576-wide latent head) with 16 sink tokens, a 1,024-token
# window and 1,024 listed tokens per sequence.
HYBRID_PATTERN = dict(block=1, sink=16, local=1024)
HYBRID_K = 1024
HYBRID_SEED = 1008


def prefill_grad(cfg: PrefillConfig, device, seed: int | None = None):
    """Upstream gradient dout [B, N, Hq, d_v] for the backward of a prefill workload."""
    gen = generator(device, cfg.seed + 50 if seed is None else seed)
    return randn((cfg.B, cfg.N, cfg.Hq, cfg.d_v), cfg.dtype, device, gen)
