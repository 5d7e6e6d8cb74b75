"""Per-group asymmetric min/max low-bit quantization and sub-byte packing.

The episode notes of *FastKVComp: checking whether high-throughput KV
compression pays off* (radioguide.fm) name "low-bit quantization" as the
second stage and say it is the only lossy step; they give no formula.  The
reading implemented here:

  * a group is G consecutive rotated coordinates of one head_dim vector
    (G divides D; groups never span tokens, heads or K/V);
  * per group: mn = min y, mx = max y;
        zero  = RD16(mn)                          (fp16, toward -inf)
        scale = RU16((mx - zero) / (2**b - 1))    (fp16, toward +inf)
    so every t = (y - zero) / scale lies in [0, 2**b - 1] with no clamp and
    |y - yhat| <= scale / 2 holds against the stored scale;
  * a constant group (mx == zero) has scale 0: every code is 0 and the
    group decodes to zero exactly;
  * codes: q = round-half-even(t);
  * packing: code j of a row sits at bits [b*j, b*j + b) of the row's
    D*b/8 bytes, least significant bits first;
  * dequantization: yhat = zero + q * scale (exact in float64: the operands
    carry 11 + 8 significant bits).

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


def group_meta(y: np.ndarray, G: int, bits: int):
    """(scale, zero) as float16 arrays of shape (..., D // G)."""
    y = np.asarray(y, dtype=np.float64)
    D = y.shape[-1]
    _check(bits, D, G)
    yg = y.reshape(y.shape[:-1] + (D // G, G))
    mn = yg.min(axis=-1)
    mx = yg.max(axis=-1)
    zero = rd16(mn)
    scale = ru16((mx - zero.astype(np.float64)) / float(2 ** bits - 1))
    if not (np.all(np.isfinite(zero)) and np.all(np.isfinite(scale))):
        raise OverflowError("rotated values exceed the fp16 range of the meta")
    return scale, zero


def quantize(y: np.ndarray, scale: np.ndarray, zero: np.ndarray, G: int, bits: int):
    """Codes q (uint8, same shape as y) and the pre-rounding values t (float64).

    t is 0 where the group's scale is 0.
    """
    y = np.asarray(y, dtype=np.float64)
    D = y.shape[-1]
    _check(bits, D, G)
    yg = y.reshape(y.shape[:-1] + (D // G, G))
    s = scale.astype(np.float64)[..., None]
    z = zero.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(s > 0, (yg - z) / np.where(s > 0, s, 1.0), 0.0)
    q = np.rint(t)
    qmax = 2 ** bits - 1
    if np.any(q < 0) or np.any(q > qmax):
        raise AssertionError("code outside [0, 2**b - 1]: meta rounding broken")
    return q.astype(np.uint8).reshape(y.shape), t.reshape(y.shape)


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
    """yhat = zero + q * scale per group, float64."""
    q = np.asarray(q)
    D = q.shape[-1]
    qg = q.reshape(q.shape[:-1] + (D // G, G)).astype(np.float64)
    yhat = zero.astype(np.float64)[..., None] + qg * scale.astype(np.float64)[..., None]
    return yhat.reshape(q.shape)
