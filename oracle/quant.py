"""Per-group asymmetric min/max low-bit quantization and sub-byte packing.

The episode notes of *FastKVComp: checking whether high-throughput KV
compression pays off* (radioguide.fm) name "low-bit quantization" as the
second stage and say it is the only lossy step; they give no formula.  The
reading implemented here:

  * a group is G consecutive rotated coordinates of one head_dim vector
    (G divides D; groups never span tokens, heads or K/V);
  * per group, from the unnormalized rotated values u = H (s * x) (so that
    the rotated value is y = u / sqrt(D)):
        zero  = RD16(mn)   with mn = min y     (fp16, rounded toward -inf)
        scale = RU16((mx - zero) / (2**b - 1)), mx = max y  (toward +inf)
    so every t = (y - zero) / scale lies in [0, 2**b - 1] up to the rounding
    of the decision arithmetic below, and |y - yhat| <= scale / 2 holds
    against the stored scale;
  * a constant group (mx == zero) has scale 0: every code is 0 and the
    group decodes to zero exactly;
  * codes: q = round-half-even(t);
  * packing: code j of a row sits at bits [b*j, b*j + b) of the row's
    D*b/8 bytes, least significant bits first;
  * dequantization: yhat = zero + q * scale (exact in float64: the operands
    carry 11 + 8 significant bits).

Decision precision.  The meta and the codes are discrete results decided by
floating-point arithmetic; this oracle takes those decisions in IEEE
binary32, in the same arithmetic the kernel performs (fl() = round to
nearest binary32, rs = fl(1 / sqrt(D))):

    mn, mx = fl(min u), fl(max u)
    zero   = RD16(fl(mn * rs))
    scale  = RU16(fl(fl(fl(mx * rs) - zero) / (2**b - 1)))
    inv    = fl(1 / scale)          (0 when scale == 0)
    a      = fl(inv * rs),  c = fl(-zero * inv)
    t      = fl(fl(u) * a + c)      (fused multiply-add: one rounding)
    q      = round-half-even(min(max(t, 0), 2**b - 1))

The clamp never acts on ordinary data (t stays within a few 1e-6 of
[0, 2**b - 1]); it bounds the code of a degenerate group -- a huge offset
with a tiny range, where the binary32 rounding of u alone moves t by more
than one half -- so that a code never spills into its neighbour's bits.

Every binary32 operation is evaluated exactly in float64 (products of two
binary32 values are exact there) and rounded once; the two divisions are
rounded correctly by comparing the exact residuals of the three nearest
binary32 candidates.  The transform itself stays float64.

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


def fl(x) -> np.ndarray:
    """Round float64 values to the nearest binary32 value (returned as float64)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def div_f32(num, den) -> np.ndarray:
    """Correctly rounded binary32 quotient of binary32 operands (den != 0).

    The float64 quotient rounded to binary32 gives a candidate; it and its two
    binary32 neighbours are compared by the exact residual |num - c * den|
    (exact in float64: c * den carries at most 48 significant bits), ties to
    the candidate with an even significand.
    """
    num = np.asarray(num, dtype=np.float64)
    den = np.asarray(den, dtype=np.float64)
    c0 = (num / den).astype(np.float32)
    cands = np.stack([np.nextafter(c0, np.float32(-np.inf)), c0, np.nextafter(c0, np.float32(np.inf))])
    res = np.abs(num - cands.astype(np.float64) * den)
    best = np.argmin(res, axis=0)
    # an exact tie between two candidates goes to the even significand
    r_sorted = np.sort(res, axis=0)
    tie = r_sorted[0] == r_sorted[1]
    if np.any(tie):
        odd = (cands.view(np.uint32) & 1).astype(np.float64)
        even_pick = np.argmin(np.where(res == r_sorted[0], odd, 2.0), axis=0)
        best = np.where(tie, even_pick, best)
    return np.take_along_axis(cands, best[None], axis=0)[0].astype(np.float64)


def _rs(D: int) -> float:
    return float(fl(1.0 / np.sqrt(D)))


def group_meta(u: np.ndarray, G: int, bits: int):
    """(scale, zero) as float16 arrays of shape (..., D // G).

    u: unnormalized rotated values H (s * x), float64 (..., D).
    """
    u = np.asarray(u, dtype=np.float64)
    D = u.shape[-1]
    _check(bits, D, G)
    rs = _rs(D)
    ug = u.reshape(u.shape[:-1] + (D // G, G))
    mn = fl(ug.min(axis=-1))
    mx = fl(ug.max(axis=-1))
    zero = rd16(fl(mn * rs))
    zf = zero.astype(np.float64)
    scale = ru16(div_f32(fl(fl(mx * rs) - zf), float(2 ** bits - 1)))
    if not (np.all(np.isfinite(zero)) and np.all(np.isfinite(scale))):
        raise OverflowError("rotated values exceed the fp16 range of the meta")
    return scale, zero


def code_values(u: np.ndarray, scale: np.ndarray, zero: np.ndarray, G: int) -> np.ndarray:
    """Pre-rounding code values t (binary32 decision arithmetic), float64 (..., D)."""
    u = np.asarray(u, dtype=np.float64)
    D = u.shape[-1]
    rs = _rs(D)
    ug = u.reshape(u.shape[:-1] + (D // G, G))
    s = scale.astype(np.float64)
    z = zero.astype(np.float64)
    inv = np.where(s > 0, div_f32(np.ones_like(s), np.where(s > 0, s, 1.0)), 0.0)
    a = fl(inv * rs)
    c = fl(-z * inv)
    t = fl(fl(ug) * a[..., None] + c[..., None])
    return t.reshape(u.shape)


def quantize(u: np.ndarray, scale: np.ndarray, zero: np.ndarray, G: int, bits: int):
    """Codes q (uint8, same shape as u) and the pre-rounding values t (float64)."""
    u = np.asarray(u, dtype=np.float64)
    _check(bits, u.shape[-1], G)
    t = code_values(u, scale, zero, G)
    qmax = 2 ** bits - 1
    q = np.rint(np.clip(t, 0.0, float(qmax)))
    return q.astype(np.uint8), t


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
    D = q.shape[-1]
    qg = q.reshape(q.shape[:-1] + (D // G, G)).astype(np.float64)
    yhat = zero.astype(np.float64)[..., None] + qg * scale.astype(np.float64)[..., None]
    return yhat.reshape(q.shape)
