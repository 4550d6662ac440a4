"""Seeded synthetic KV inputs for the tests and the benchmark.

This module only draws random tensors; it holds none of the quantization
arithmetic. Each generator is deterministic for a given (seed, device): the
same call on the same device type gives the same fp16 tensor. CPU and GPU
generators produce different streams, so a parity test draws once on one
device and copies to the other.

Recipes (value distributions from the workload descriptions of the pages'
configurations):
  * sym_layer: N(0,1) K/V rows [tokens][heads][D]; per head, ceil(1% * D)
    channels scaled x10; optionally a fraction of token positions drawn from
    Laplace(0,1) instead of N(0,1) ("Laplace tails").
  * kivi_kv: keys N(0,1) with `hot` channels per head at sigma 8, values
    N(0, sigma=0.5); layout [B][H][S][D].
  * student_t: Student-t(nu) samples, [BH][S][D].
"""
from __future__ import annotations

import math

import torch


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(int(seed))
    return g


def outlier_channels(n_groups: int, D: int, count: int, seed: int) -> torch.Tensor:
    """[n_groups][count] distinct channel indices per group (CPU, int64)."""
    g = _gen(seed, "cpu")
    return torch.stack([torch.randperm(D, generator=g)[:count] for _ in range(n_groups)]) \
        if count > 0 else torch.zeros((n_groups, 0), dtype=torch.int64)


def sym_layer(n_tokens: int, H: int, D: int, *, seed: int, device="cpu",
              outlier_frac: float = 0.01, outlier_scale: float = 10.0,
              laplace_token_frac: float = 0.0, channel_seed: int | None = None) -> torch.Tensor:
    """fp16 [n_tokens][H][D] for one layer of K or V."""
    g = _gen(seed, device)
    x = torch.randn((n_tokens, H, D), generator=g, device=device, dtype=torch.float32)
    if laplace_token_frac > 0:
        pick = torch.rand((n_tokens,), generator=g, device=device) < laplace_token_frac
        u = torch.rand((n_tokens, H, D), generator=g, device=device) - 0.5
        u = u.clamp(-0.5 + 1e-7, 0.5 - 1e-7)
        lap = -torch.sign(u) * torch.log1p(-2.0 * u.abs())
        x = torch.where(pick[:, None, None], lap, x)
    count = int(math.ceil(outlier_frac * D)) if outlier_frac > 0 else 0
    if count:
        ch = outlier_channels(H, D, count, seed + 1000 if channel_seed is None else channel_seed)
        mult = torch.ones((H, D), dtype=torch.float32)
        mult.scatter_(1, ch, outlier_scale)
        x = x * mult.to(device)[None]
    return x.to(torch.float16)


def kivi_kv(B: int, H: int, S: int, D: int, *, seed: int, device="cpu", hot: int = 4,
            hot_sigma: float = 8.0, v_sigma: float = 0.5):
    """(keys, values) fp16 [B][H][S][D]."""
    g = _gen(seed, device)
    k = torch.randn((B, H, S, D), generator=g, device=device, dtype=torch.float32)
    ch = outlier_channels(H, D, hot, seed + 1000)
    mult = torch.ones((H, D), dtype=torch.float32)
    if hot:
        mult.scatter_(1, ch, hot_sigma)
    k = k * mult.to(device)[None, :, None, :]
    v = torch.randn((B, H, S, D), generator=g, device=device, dtype=torch.float32) * v_sigma
    return k.to(torch.float16), v.to(torch.float16)


def student_t(shape, nu: int = 4, *, seed: int, device="cpu") -> torch.Tensor:
    """fp16 Student-t(nu) samples: Z / sqrt(chi2_nu / nu), chi2 as a sum of nu squared normals."""
    g = _gen(seed, device)
    z = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    chi = torch.zeros(tuple(shape), device=device, dtype=torch.float32)
    for _ in range(nu):
        chi += torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32) ** 2
    return (z / torch.sqrt(chi / nu)).to(torch.float16)


def paged_block_table(n_seqs: int, tokens_per_seq: int, page_size: int, *, seed: int,
                      extra_pages: int = 0):
    """Random page assignment: (block_table int32 [n_seqs][max_blocks] CPU, num_pages).

    Pages of all sequences are a seeded permutation of the pool, so a
    sequence's pages are scattered through it as after fragmentation.
    """
    blocks = (tokens_per_seq + page_size - 1) // page_size
    num_pages = n_seqs * blocks + extra_pages
    g = _gen(seed, "cpu")
    perm = torch.randperm(num_pages, generator=g)[: n_seqs * blocks]
    return perm.view(n_seqs, blocks).to(torch.int32).contiguous(), num_pages


def slot_mapping_for(block_table: torch.Tensor, page_size: int, start: int, count: int) -> torch.Tensor:
    """int32 [n_seqs * count]: slots of positions [start, start+count) of every sequence,
    sequence-major (the token order of a batched prefill/decode input)."""
    pos = torch.arange(start, start + count, dtype=torch.int64)
    pages = block_table.to(torch.int64)[:, pos // page_size]
    return (pages * page_size + (pos % page_size)[None, :]).reshape(-1).to(torch.int32)
