"""Pure-Python brute-force twin of the numpy oracle, in exact arithmetic.

TEST INFRASTRUCTURE ONLY (see the package docstring).  For tiny shapes.

Every step is computed a second way, from definitions rather than formulas,
and every decision is taken exactly -- with no floating-point rounding at
all -- so this twin pins the float64 oracle in ``oracle/quant.py`` and
``oracle/rht.py``:

  * the transform u = H (s * x) by explicit integer sums over the popcount
    definition of H (storage values are dyadic rationals, so scaling a row
    by a power of two makes every term an integer); the rotated value is
    y = u / sqrt(D), kept as the pair (u, D): y is irrational for odd
    log2(D), and every comparison of y with a rational r is decided by
    the sign of u - r * sqrt(D), from u**2 and r**2 * D when both sides
    carry the same sign;
  * fp16 directed rounding by binary search over the sorted list of every
    finite binary16 value: zero = the largest fp16 value <= min y, scale =
    the smallest fp16 value s >= 0 with zero + (2**b - 1) * s >= max y;
  * codes as the argmin over all 2**b codes k of |y - (zero + k * scale)|,
    ties to the even code, by exact pairwise comparisons of distances;
  * packing and unpacking bit by bit;
  * decode yhat = zero + q * scale and x = s * (H yhat) / sqrt(D) in exact
    rationals, then the nearest bf16 / fp16 value by binary search over the
    format's finite values, ties to the even bit pattern.

Same readings of the pages as the numpy oracle (see ``oracle/quant.py``,
``oracle/rht.py`` and ``oracle/signs.py``): seeded sign flip then
orthonormal Sylvester transform, per-group fp16 zero rounded down and scale
rounded up, nearest code with ties to even, LSB-first packing.  An exact
zero meta value is stored as +0; an exact zero output is +0 times its sign
s_i.
"""

import math
import struct
from fractions import Fraction

from .signs import sign_vector


def _finite_values(fmt):
    """Sorted distinct finite values of fmt as (Fraction, bit pattern); 0 is +0."""
    seen = {}
    for bits in range(65536):
        if fmt == "fp16":
            v = struct.unpack("<e", struct.pack("<H", bits))[0]
        else:
            v = struct.unpack("<f", struct.pack("<I", bits << 16))[0]
        if math.isfinite(v):
            key = Fraction(v)
            if key == 0:
                bits = 0
            seen.setdefault(key, bits)
    vals = sorted(seen)
    return vals, [seen[v] for v in vals]


_GRID = {}


def _grid(fmt):
    if fmt not in _GRID:
        _GRID[fmt] = _finite_values(fmt)
    return _GRID[fmt]


def fp16_bits_of(v) -> int:
    return struct.unpack("<H", struct.pack("<e", float(v)))[0]


def fp16_from_bits(b: int) -> Fraction:
    return Fraction(struct.unpack("<e", struct.pack("<H", b))[0])


def _sign(v) -> int:
    return (v > 0) - (v < 0)


def cmp_root(u: Fraction, D: int, r: Fraction) -> int:
    """sign(u / sqrt(D) - r), exactly (u, r rational, D >= 1)."""
    root = math.isqrt(D)
    if root * root == D:
        return _sign(u - r * root)
    su, sr = _sign(u), _sign(r)
    if su == 0:
        return -sr
    if su != sr:
        return su
    d = _sign(u * u - r * r * D)
    return d if su > 0 else -d


def _last_at_or_below(u, D, vals):
    """Index of the largest vals[i] <= u / sqrt(D), or -1."""
    lo, hi = 0, len(vals)            # invariant: answer in [lo - 1, hi - 1]
    while lo < hi:
        mid = (lo + hi) // 2
        if cmp_root(u, D, vals[mid]) >= 0:
            lo = mid + 1
        else:
            hi = mid
    return lo - 1


def rd16_exact(u: Fraction, D: int) -> Fraction:
    """The largest finite binary16 value <= u / sqrt(D)."""
    vals, _ = _grid("fp16")
    i = _last_at_or_below(u, D, vals)
    if i < 0:
        raise OverflowError("below the fp16 range")
    return vals[i]


def rd16_search(x: float) -> float:
    """Largest finite binary16 value <= x, by search over every finite value."""
    if x == 0.0:
        return x
    return float(rd16_exact(Fraction(x), 1))


def ru16_search(x: float) -> float:
    """Smallest finite binary16 value >= x, by search over every finite value."""
    if x == 0.0:
        return x
    return -float(rd16_exact(-Fraction(x), 1))


def ru16_scale(u_max: Fraction, D: int, zero: Fraction, qmax: int) -> Fraction:
    """The smallest finite binary16 s >= 0 with zero + qmax * s >= u_max / sqrt(D)."""
    vals, _ = _grid("fp16")
    lo, hi = vals.index(Fraction(0)), len(vals)   # first index whose value satisfies it
    while lo < hi:
        mid = (lo + hi) // 2
        if cmp_root(u_max, D, zero + qmax * vals[mid]) <= 0:
            hi = mid
        else:
            lo = mid + 1
    if lo == len(vals):
        raise OverflowError("scale above the fp16 range")
    return vals[lo]


def closer(u, D, a: Fraction, b: Fraction) -> int:
    """-1 if y = u / sqrt(D) is nearer to a than to b, 1 if nearer to b, 0 on a tie."""
    if a == b:
        return 0
    d = cmp_root(u, D, (a + b) / 2)
    return d if a < b else -d


def nearest_code(u: Fraction, D: int, zero: Fraction, scale: Fraction, qmax: int) -> int:
    """argmin over k in [0, qmax] of |y - (zero + k * scale)|, ties to the even k."""
    if scale == 0:
        return 0
    best = 0
    for k in range(1, qmax + 1):
        c = closer(u, D, zero + k * scale, zero + best * scale)
        if c < 0 or (c == 0 and k % 2 == 0):
            best = k
    return best


def nearest_even_pattern(v: Fraction, D: int, fmt: str, zero_sign: int = 1) -> int:
    """Bit pattern of the fmt value nearest to v / sqrt(D), ties to the even
    pattern; an exact zero takes the sign zero_sign."""
    vals, pats = _grid(fmt)
    if v == 0:
        return 0x8000 if zero_sign < 0 else 0
    i = _last_at_or_below(v, D, vals)
    cands = [j for j in (i, i + 1) if 0 <= j < len(vals)]
    best = cands[0]
    for j in cands[1:]:
        c = closer(v, D, vals[j], vals[best])
        if c < 0 or (c == 0 and pats[j] % 2 == 0):
            best = j
    pat = pats[best]
    if vals[best] == 0:                 # a nonzero value rounded to zero keeps its sign
        pat = 0x8000 if v < 0 else 0
    return pat


def hadamard_entry(i: int, j: int) -> int:
    return -1 if bin(i & j).count("1") % 2 else 1


def rotate_rows_raw(x_rows, seed, D):
    """u = H (s * x) per row, exact: lists of Fractions."""
    s = sign_vector(seed, D)
    out = []
    for row in x_rows:
        fr = [Fraction(v) for v in row]
        den = max(f.denominator for f in fr)          # a power of two
        ints = [int(f * den) * int(s[j]) for j, f in enumerate(fr)]
        out.append([Fraction(sum(hadamard_entry(i, j) * ints[j] for j in range(D)), den) for i in range(D)])
    return out


def rotated_values(x_rows, seed, D):
    """y = u / sqrt(D) per row as floats (for display and coarse checks only)."""
    return [[float(v) / math.sqrt(D) for v in u] for u in rotate_rows_raw(x_rows, seed, D)]


def encode_rows(x_rows, D, G, bits, seed):
    """Returns (packed rows as lists of bytes, meta [(scale_bits, zero_bits)], codes)."""
    us = rotate_rows_raw(x_rows, seed, D)
    qmax = 2 ** bits - 1
    packed_rows, metas, codes_rows = [], [], []
    for u in us:
        codes = []
        row_meta = []
        for g in range(D // G):
            part = u[g * G:(g + 1) * G]
            z = rd16_exact(min(part), D)
            s = ru16_scale(max(part), D, z, qmax)
            row_meta.append((fp16_bits_of(s), fp16_bits_of(z)))
            codes.extend(nearest_code(v, D, z, s, qmax) for v in part)
        nbytes = D * bits // 8
        packed = [0] * nbytes
        for j, c in enumerate(codes):
            for i in range(bits):
                pos = bits * j + i
                packed[pos // 8] |= ((c >> i) & 1) << (pos % 8)
        packed_rows.append(packed)
        metas.append(row_meta)
        codes_rows.append(codes)
    return packed_rows, metas, codes_rows


def decode_rows(packed_rows, metas, D, G, bits, seed, out_fmt):
    """Returns (output bit patterns per row, exact decoded values per row as floats)."""
    s = sign_vector(seed, D)
    out_bits, out_vals = [], []
    for packed, row_meta in zip(packed_rows, metas):
        codes = []
        for j in range(D):
            c = 0
            for i in range(bits):
                pos = bits * j + i
                c |= ((packed[pos // 8] >> (pos % 8)) & 1) << i
            codes.append(c)
        yhat = []
        for j in range(D):
            sb, zb = row_meta[j // G]
            yhat.append(fp16_from_bits(zb) + codes[j] * fp16_from_bits(sb))
        v = [int(s[i]) * sum(hadamard_entry(i, j) * yhat[j] for j in range(D)) for i in range(D)]
        out_vals.append([float(vi) / math.sqrt(D) for vi in v])
        # the sign flip multiplies the transformed value: an exact zero is +0
        # times s_i, so -0 where s_i = -1
        out_bits.append([nearest_even_pattern(vi, D, out_fmt, int(s[i])) for i, vi in enumerate(v)])
    return out_bits, out_vals
