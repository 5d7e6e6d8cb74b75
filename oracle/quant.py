"""Per-group asymmetric min/max low-bit quantization and sub-byte packing.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The episode notes of *FastKVComp: checking whether high-throughput KV
compression pays off* (radioguide.fm) name "low-bit quantization" as the
second stage and say it is the only step that loses information; they give
no formula.  The reading implemented here, on the rotated values y of one
head_dim vector (the orthonormal transform's output, float64):

  * a group is G consecutive rotated coordinates of one head_dim vector
    (G divides D; groups never span tokens, heads or K/V);
  * per group, with mn = min y and mx = max y over the group:
        zero  = RD16(mn)                        fp16, rounded toward -inf
        scale = RU16((mx - zero) / (2**b - 1))  fp16, rounded toward +inf
    so that every t = (y - zero) / scale lies in [0, 2**b - 1] and
    |y - yhat| <= scale / 2 holds against the stored scale;
  * codes: q = the code k in [0, 2**b - 1] whose level zero + k * scale is
    nearest to y, ties to the even k -- that is, round-half-even of
    t = (y - zero) / scale, clipped to the code range;
  * a constant group (mx == zero) has scale 0: every code is 0 and the
    group decodes to zero exactly;
  * packing: code j of a row sits at bits [b*j, b*j + b) of the row's
    D*b/8 bytes, least significant bits first;
  * dequantization: yhat = zero + q * scale (exact in float64: the operands
    carry 11 + 8 significant bits).

Arithmetic: the definition above, evaluated in float64 step by step -- one
subtraction and one division for the scale, one subtraction and one division
for t, no reciprocal, no fused multiply-add, no folding of constants.  The
float64 result equals the exact one except where an exact intermediate lies
within a few float64 ulps (about 1e-16 relative) of an fp16 grid point or of
a code boundary k + 1/2; the brute-force twin in ``oracle/scalar.py``
decides every such comparison exactly and is checked against this module.

A rotated value outside the fp16 range has no representable meta; the
oracle raises instead of producing infinities.
"""

import numpy as np

from .rounding import rd16, ru16


def _check(bits: int, D: int, G: int):
    if bits not in (2, 4, 8):
        raise ValueError("bits must be 2, 4 or 8")
    if G <= 0 or D % G:
        raise ValueError("group must divide head_dim")


def _groups(a: np.ndarray, G: int) -> np.ndarray:
    D = a.shape[-1]
    return a.reshape(a.shape[:-1] + (D // G, G))


def group_meta(y: np.ndarray, G: int, bits: int):
    """(scale, zero) as float16 arrays of shape (..., D // G).

    y: rotated values, float64 (..., D).
    """
    y = np.asarray(y, dtype=np.float64)
    _check(bits, y.shape[-1], G)
    if y.size and not np.abs(y).max() <= 65504.0:
        raise OverflowError("rotated values exceed the fp16 range of the meta")
    yg = _groups(y, G)
    mn = yg.min(axis=-1) + 0.0       # an exact zero minimum is stored as +0
    mx = yg.max(axis=-1)
    zero = rd16(mn)
    scale = ru16((mx - zero.astype(np.float64)) / float(2 ** bits - 1))
    if not (np.all(np.isfinite(zero)) and np.all(np.isfinite(scale))):
        raise OverflowError("rotated values exceed the fp16 range of the meta")
    return scale, zero


def code_values(y: np.ndarray, scale: np.ndarray, zero: np.ndarray, G: int) -> np.ndarray:
    """Pre-rounding code values t = (y - zero) / scale, float64 (..., D).

    Elements of a group with scale 0 get t = 0.
    """
    y = np.asarray(y, dtype=np.float64)
    s = np.asarray(scale).astype(np.float64)[..., None]
    z = np.asarray(zero).astype(np.float64)[..., None]
    t = np.where(s > 0, (_groups(y, G) - z) / np.where(s > 0, s, 1.0), 0.0)
    return t.reshape(y.shape)


def nearest_codes(t: np.ndarray, bits: int) -> np.ndarray:
    """The code nearest to t among 0 .. 2**b - 1, ties to even (uint8)."""
    return np.clip(np.rint(t), 0.0, float(2 ** bits - 1)).astype(np.uint8)


def quantize(y: np.ndarray, scale: np.ndarray, zero: np.ndarray, G: int, bits: int):
    """Codes q (uint8, same shape as y) and the pre-rounding values t (float64)."""
    y = np.asarray(y, dtype=np.float64)
    _check(bits, y.shape[-1], G)
    t = code_values(y, scale, zero, G)
    return nearest_codes(t, bits), t


def pack_codes(q: np.ndarray, bits: int) -> np.ndarray:
    """(..., D) codes -> (..., D * bits // 8) bytes, LSB-first within each byte."""
    q = np.asarray(q, dtype=np.uint8)
    D = q.shape[-1]
    per_byte = 8 // bits
    if D % per_byte:
        raise ValueError("row does not fill whole bytes")
    if np.any(q >> bits):
        raise ValueError("code wider than bits")
    qb = q.reshape(q.shape[:-1] + (D // per_byte, per_byte)).astype(np.uint16)
    out = np.zeros(qb.shape[:-1], dtype=np.uint16)
    for k in range(per_byte):
        out |= qb[..., k] << (bits * k)
    return out.astype(np.uint8)


def unpack_codes(packed: np.ndarray, bits: int, D: int) -> np.ndarray:
    """Inverse of :func:`pack_codes`."""
    p = np.asarray(packed, dtype=np.uint8)
    per_byte = 8 // bits
    if p.shape[-1] * per_byte != D:
        raise ValueError("packed row size does not match head_dim")
    mask = (1 << bits) - 1
    parts = [(p >> (bits * k)) & mask for k in range(per_byte)]
    return np.stack(parts, axis=-1).reshape(p.shape[:-1] + (D,)).astype(np.uint8)


def dequantize(q: np.ndarray, scale: np.ndarray, zero: np.ndarray, G: int) -> np.ndarray:
    """yhat = zero + q * scale per group, float64 (normalized domain)."""
    q = np.asarray(q)
    qg = _groups(q, G).astype(np.float64)
    yhat = np.asarray(zero).astype(np.float64)[..., None] + qg * np.asarray(scale).astype(np.float64)[..., None]
    return yhat.reshape(q.shape)
