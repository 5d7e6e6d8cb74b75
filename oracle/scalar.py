"""Pure-Python brute-force twin of the numpy oracle, for tiny shapes only.

Every step is computed a second way, from definitions rather than formulas:

  * Hadamard entries from (-1)**popcount(i & j), transform by explicit sums;
  * fp16 directed rounding by searching the sorted list of every finite
    binary16 value (largest value <= x, smallest value >= x);
  * every binary32 step of the decision arithmetic (see ``oracle/quant.py``)
    evaluated exactly in rational arithmetic (``fractions.Fraction``) and
    rounded to the nearest binary32 value by an exact integer rounding;
  * codes as the integer nearest to t, ties to even, in rational arithmetic;
  * packing bit by bit;
  * output rounding to bf16 / fp16 by nearest-value search over the format's
    finite values, ties to the even bit pattern.

Same readings of the pages as the numpy oracle (see ``oracle/quant.py`` and
``oracle/rht.py``): seeded sign flip then orthonormal Sylvester transform,
per-group fp16 zero rounded down and scale rounded up, LSB-first packing.
"""

import bisect
import math
import struct
from fractions import Fraction

from .signs import sign_vector


def _all_finite(fmt):
    vals = set()
    for bits in range(65536):
        if fmt == "fp16":
            v = struct.unpack("<e", struct.pack("<H", bits))[0]
        else:
            v = struct.unpack("<f", struct.pack("<I", bits << 16))[0]
        if math.isfinite(v):
            vals.add((v, bits))
    return vals


_GRID = {}


def _grid(fmt):
    if fmt not in _GRID:
        pairs = sorted(_all_finite(fmt))
        # collapse +0/-0 to +0 for searching; zeros are handled separately
        values = []
        patterns = []
        for v, b in pairs:
            if v == 0.0 and values and values[-1] == 0.0:
                continue
            values.append(v)
            patterns.append(b if v != 0.0 else 0)
        _GRID[fmt] = (values, patterns)
    return _GRID[fmt]


def fp16_bits_of(v: float) -> int:
    return struct.unpack("<H", struct.pack("<e", v))[0]


def fp16_from_bits(b: int) -> float:
    return struct.unpack("<e", struct.pack("<H", b))[0]


def rd16_search(x: float) -> float:
    """Largest finite binary16 value <= x (x = 0 keeps its sign)."""
    if x == 0.0:
        return x
    values, _ = _grid("fp16")
    i = bisect.bisect_right(values, x) - 1
    if i < 0:
        return -math.inf
    return values[i]


def ru16_search(x: float) -> float:
    """Smallest finite binary16 value >= x (x = 0 keeps its sign)."""
    if x == 0.0:
        return x
    values, _ = _grid("fp16")
    i = bisect.bisect_left(values, x)
    if i >= len(values):
        return math.inf
    return values[i]


def nearest_even_search(x: float, fmt: str) -> int:
    """Bit pattern of the value of ``fmt`` nearest to x, ties to even pattern."""
    values, patterns = _grid(fmt)
    if x == 0.0:
        return 0x8000 if math.copysign(1.0, x) < 0 else 0
    i = bisect.bisect_left(values, x)
    cands = [j for j in (i - 1, i) if 0 <= j < len(values)]
    best = min(cands, key=lambda j: (abs(values[j] - x), patterns[j] & 1))
    pat = patterns[best]
    if values[best] == 0.0:
        pat = 0x8000 if x < 0 else 0
    return pat


def f32_round(v) -> float:
    """Nearest binary32 value to the rational v, ties to even (exact)."""
    v = Fraction(v)
    if v == 0:
        return 0.0
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 23)
    m = a / quantum
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * float(n * quantum)


def nearest_int_even(v) -> int:
    v = Fraction(v)
    n = math.floor(v)
    rem = v - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def rotate_rows_raw(x_rows, seed, D):
    """u = H (s * x) by exact rational sums."""
    s = sign_vector(seed, D)
    out = []
    for row in x_rows:
        u = []
        for i in range(D):
            acc = Fraction(0)
            for j in range(D):
                h = -1 if bin(i & j).count("1") % 2 else 1
                acc += h * int(s[j]) * Fraction(row[j])
            u.append(acc)
        out.append(u)
    return out


def rotate_rows(x_rows, seed, D):
    s = sign_vector(seed, D)
    inv = math.sqrt(D)
    out = []
    for row in x_rows:
        y = []
        for i in range(D):
            acc = 0.0
            for j in range(D):
                h = -1.0 if bin(i & j).count("1") % 2 else 1.0
                acc += h * s[j] * row[j]
            y.append(acc / inv)
        out.append(y)
    return out


def encode_rows(x_rows, D, G, bits, seed):
    """Returns (packed rows as lists of bytes, meta [(scale_bits, zero_bits)], codes)."""
    us = rotate_rows_raw(x_rows, seed, D)
    qmax = 2 ** bits - 1
    rs = Fraction(f32_round(Fraction(1.0 / math.sqrt(D))))
    packed_rows, metas, codes_rows = [], [], []
    for u in us:
        codes = []
        row_meta = []
        for g in range(D // G):
            part = u[g * G:(g + 1) * G]
            mn = Fraction(f32_round(min(part)))
            mx = Fraction(f32_round(max(part)))
            z = rd16_search(f32_round(mn * rs))
            zq = Fraction(z)
            d = Fraction(f32_round(Fraction(f32_round(mx * rs)) - zq))
            s = ru16_search(f32_round(d / qmax))
            sq = Fraction(s)
            row_meta.append((fp16_bits_of(s), fp16_bits_of(z)))
            if s == 0.0:
                codes.extend([0] * G)
                continue
            inv = Fraction(f32_round(1 / sq))
            a = Fraction(f32_round(inv * rs))
            c = Fraction(f32_round(-zq * inv))
            for v in part:
                t = Fraction(f32_round(Fraction(f32_round(v)) * a + c))
                t = min(max(t, Fraction(0)), Fraction(qmax))
                codes.append(nearest_int_even(t))
        nbytes = D * bits // 8
        packed = [0] * nbytes
        for j, c in enumerate(codes):
            for i in range(bits):
                bit = (c >> i) & 1
                pos = bits * j + i
                packed[pos // 8] |= bit << (pos % 8)
        packed_rows.append(packed)
        metas.append(row_meta)
        codes_rows.append(codes)
    return packed_rows, metas, codes_rows


def decode_rows(packed_rows, metas, D, G, bits, seed, out_fmt):
    """Returns (output bit patterns per row, float64 values per row)."""
    s = sign_vector(seed, D)
    root = math.sqrt(D)
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
        vals = []
        for i in range(D):
            acc = 0.0
            for j in range(D):
                h = -1.0 if bin(i & j).count("1") % 2 else 1.0
                acc += h * yhat[j]
            vals.append(s[i] * (acc / root))
        out_vals.append(vals)
        out_bits.append([nearest_even_search(v, out_fmt) for v in vals])
    return out_bits, out_vals
