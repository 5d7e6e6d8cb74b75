"""Seeded +/-1 sign vector for the randomized Hadamard transform.

The episode notes of *FastKVComp: checking whether high-throughput KV
compression pays off* (radioguide.fm) call the first stage a randomized
Hadamard transform but do not say how the random signs are drawn.  Reading
taken here: one sign per head_dim index j, shared by every layer, K/V slab,
token and head of a call, drawn from SplitMix64 -- the counter-based
generator of Steele, Lea and Flood ("Fast splittable pseudorandom number
generators", OOPSLA 2014) in the public-domain form that Vigna publishes as
``splitmix64.c``:

    state_{j+1} = state_j + 0x9E3779B97F4A7C15          (mod 2**64)
    z = state_{j+1}
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9             (mod 2**64)
    z = (z ^ (z >> 27)) * 0x94D049BB133111EB             (mod 2**64)
    out_j = z ^ (z >> 31)

with state_0 = seed.  s_j = -1 when bit 63 of out_j is set, else +1.  The
generator is counter based, so s_j for j < 64 is the same whatever head_dim
is.  Python integers keep the arithmetic exact.
"""

import numpy as np

_MASK64 = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15
_MIX1 = 0xBF58476D1CE4E5B9
_MIX2 = 0x94D049BB133111EB


def splitmix64_outputs(seed: int, count: int) -> list:
    """First ``count`` outputs of a SplitMix64 stream seeded with ``seed``."""
    if not 0 <= seed <= _MASK64:
        raise ValueError("seed must fit in 64 unsigned bits")
    out = []
    state = seed
    for _ in range(count):
        state = (state + _GAMMA) & _MASK64
        z = state
        z = ((z ^ (z >> 30)) * _MIX1) & _MASK64
        z = ((z ^ (z >> 27)) * _MIX2) & _MASK64
        out.append(z ^ (z >> 31))
    return out


def sign_vector(seed: int, head_dim: int) -> np.ndarray:
    """s in {-1,+1}^head_dim as float64 (s_j = -1 iff bit 63 of out_j)."""
    outs = splitmix64_outputs(seed, head_dim)
    return np.array([-1.0 if (z >> 63) & 1 else 1.0 for z in outs], dtype=np.float64)


def sign_bits_mask(seed: int, head_dim: int) -> int:
    """The same signs as an integer whose bit j is set iff s_j = -1."""
    mask = 0
    for j, z in enumerate(splitmix64_outputs(seed, head_dim)):
        if (z >> 63) & 1:
            mask |= 1 << j
    return mask
