"""Randomized Hadamard transform along head_dim, as an explicit matrix product.

The episode notes of *FastKVComp: checking whether high-throughput KV
compression pays off* (radioguide.fm) name a randomized Hadamard transform
as the distribution transformation that precedes quantization; the abstract
of *Beyond Compression Ratio: High-Throughput KV Compression for
Disaggregated LLM Serving* calls it the "distribution transformation" stage.

Readings taken where the pages are silent:
  * the matrix is the Sylvester Hadamard matrix in natural order,
    H[i][j] = (-1)**popcount(i & j) (so H_{2n} = [[H_n, H_n], [H_n, -H_n]]);
  * the transform is orthonormal: y = H (s * x) / sqrt(D), sign flip first;
  * the inverse is x = s * (H y) / sqrt(D) (H is symmetric and H H = D I).

Everything is float64 and uses a library matrix multiply as the only
primitive; no fast transform, blocking or reordering.
"""

import numpy as np


def _popcount(a: np.ndarray) -> np.ndarray:
    a = a.astype(np.int64)
    c = np.zeros_like(a)
    while np.any(a):
        c += a & 1
        a = a >> 1
    return c


def hadamard(D: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order D (a power of two), float64."""
    if D < 1 or D & (D - 1):
        raise ValueError("D must be a power of two")
    i = np.arange(D)
    return np.where(_popcount(i[:, None] & i[None, :]) % 2 == 0, 1.0, -1.0)


def rotate_raw(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """Rows of x (..., D) -> u = H (s * x), the transform before the 1/sqrt(D)."""
    x = np.asarray(x, dtype=np.float64)
    return (x * signs) @ hadamard(x.shape[-1])


def rotate(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """Rows of x (..., D) -> y = H (s * x) / sqrt(D), float64."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    H = hadamard(D)
    return ((x * signs) @ H) / np.sqrt(D)


def unrotate(y: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """Inverse of :func:`rotate`: x = s * (H y) / sqrt(D), float64."""
    y = np.asarray(y, dtype=np.float64)
    D = y.shape[-1]
    H = hadamard(D)
    return signs * ((y @ H) / np.sqrt(D))
