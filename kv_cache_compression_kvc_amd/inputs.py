"""Seeded synthetic inputs: KV tensors, paged pools, block tables.

This module draws random numbers and nothing else: no step of the encode or
decode lives here, so the HIP path and the CPU oracle can both take their
inputs from it.

Recipe (one torch generator per (preset, layer, K/V) chunk, so any slice of
a large workload can be regenerated on its own):

  * values ~ N(0, sigma^2) in float32 (sigma = k_sigma for K, v_sigma for V);
  * K only: ``k_outlier_channels`` head_dim channels per layer, drawn
    without replacement, are multiplied by ``outlier_scale`` for every
    token and head of that layer;
  * K and V: with probability ``spike_prob`` an element is multiplied by
    ``spike_scale``;
  * the result is rounded to bf16 / fp16 (round to nearest even).

Paged presets: lengths ~ U{len_min..len_max} per request, a pool of
sum(ceil(len / block_size)) blocks plus ``spare_blocks`` unused ones, and a
block table that assigns the blocks of a seeded random permutation to the
requests' logical blocks in order (unused table entries are -1).
"""

import hashlib
import math

import numpy as np
import torch

from .presets import Preset

TORCH_DTYPE = {"bf16": torch.bfloat16, "fp16": torch.float16}


def _seed(*parts) -> int:
    h = hashlib.blake2b("/".join(str(p) for p in parts).encode(), digest_size=8)
    return int.from_bytes(h.digest(), "little") & ((1 << 63) - 1)


def outlier_channels(p: Preset, layer: int) -> torch.Tensor:
    g = torch.Generator(device="cpu").manual_seed(_seed(p.name, "outliers", layer))
    return torch.randperm(p.head_dim, generator=g)[: p.k_outlier_channels]


def kv_chunk(p: Preset, layer: int, kv: int, lead_shape, device="cpu") -> torch.Tensor:
    """One (layer, K/V) chunk of shape lead_shape + (H, D) in the preset dtype."""
    g = torch.Generator(device=device).manual_seed(_seed(p.name, layer, kv))
    shape = tuple(lead_shape) + (p.kv_heads, p.head_dim)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    x *= p.k_sigma if kv == 0 else p.v_sigma
    if kv == 0 and p.k_outlier_channels:
        ch = outlier_channels(p, layer).to(device)
        x[..., ch] *= p.outlier_scale
    if p.spike_prob > 0:
        u = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
        x = torch.where(u < p.spike_prob, x * p.spike_scale, x)
    return x.to(TORCH_DTYPE[p.dtype])


def make_kv(p: Preset, device="cpu", layers=None, tokens=None) -> torch.Tensor:
    """Contiguous [L, 2, T, H, D] KV tensor (optionally fewer layers / tokens)."""
    L = p.layers if layers is None else layers
    T = p.tokens if tokens is None else tokens
    out = torch.empty((L, 2, T, p.kv_heads, p.head_dim), dtype=TORCH_DTYPE[p.dtype], device=device)
    for l in range(L):
        for kv in range(2):
            out[l, kv] = kv_chunk(p, l, kv, (T,), device)
    return out


def request_lengths(p: Preset, num_requests=None, len_min=None, len_max=None) -> np.ndarray:
    R = p.num_requests if num_requests is None else num_requests
    lo = p.len_min if len_min is None else len_min
    hi = p.len_max if len_max is None else len_max
    rng = np.random.Generator(np.random.PCG64(_seed(p.name, "lengths")))
    return rng.integers(lo, hi + 1, size=R).astype(np.int32)


def block_table(p: Preset, seq_lens, max_blocks=None):
    """(table int32 [R, max_blocks] with -1 padding, num_blocks of the pool)."""
    bs = p.block_size
    need = [int(math.ceil(int(n) / bs)) for n in seq_lens]
    used = sum(need)
    num_blocks = used + int(math.ceil(used * p.spare_blocks))
    mb = max(need + [1]) if max_blocks is None else max_blocks
    rng = np.random.Generator(np.random.PCG64(_seed(p.name, "blocks")))
    perm = rng.permutation(num_blocks).astype(np.int32)
    table = np.full((len(seq_lens), mb), -1, dtype=np.int32)
    pos = 0
    for r, k in enumerate(need):
        table[r, :k] = perm[pos:pos + k]
        pos += k
    return table, num_blocks


def make_pool(p: Preset, num_blocks: int, device="cpu", layers=None) -> torch.Tensor:
    """Paged pool [L, 2, num_blocks, block_size, H, D] filled per (layer, K/V)."""
    L = p.layers if layers is None else layers
    out = torch.empty((L, 2, num_blocks, p.block_size, p.kv_heads, p.head_dim),
                      dtype=TORCH_DTYPE[p.dtype], device=device)
    for l in range(L):
        for kv in range(2):
            out[l, kv] = kv_chunk(p, l, kv, (num_blocks, p.block_size), device)
    return out


def as_u16(t: torch.Tensor) -> np.ndarray:
    """Host uint16 storage of a bf16 / fp16 tensor (exact bit copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
