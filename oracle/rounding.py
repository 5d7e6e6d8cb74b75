"""Rounding of float64 values onto binary16 / bfloat16 grids.

Written from the IEEE 754 definition of a binary format with p significant
bits, minimum normal exponent emin and maximum exponent emax: a finite value
is m * 2**(E-(p-1)) with integer |m| < 2**p and E >= emin.  Rounding picks
the integer m by round-to-nearest-even (``np.rint``), toward -inf
(``np.floor``) or toward +inf (``np.ceil``) on the value scaled by the grid
quantum at its exponent; the rescale is exact because the quantum is a
power of two.

binary16: p = 11, emin = -14, emax = 15.
bfloat16: p = 8,  emin = -126, emax = 127.

Meta values (fp16 scale and zero) use the directed modes: the zero rounds
down and the scale rounds up, so that every element of a group lands inside
the quantization range without a clamp (reading of the pages' "low-bit
quantization", which the episode notes of *FastKVComp: checking whether
high-throughput KV compression pays off* name but do not detail).
"""

import numpy as np

_FORMATS = {
    "fp16": (11, -14, 15),
    "bf16": (8, -126, 127),
}


def round_binary(x, fmt: str, mode: str = "rne") -> np.ndarray:
    """Round float64 ``x`` onto the grid of ``fmt``; returns float64 values.

    mode: "rne" (nearest, ties to even), "down" (toward -inf), "up"
    (toward +inf).  Overflow follows IEEE: RNE goes to +/-inf, directed
    modes go to inf only in their own direction and to +/-max otherwise.
    NaN propagates.
    """
    p, emin, emax = _FORMATS[fmt]
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    finite = np.isfinite(x)
    safe = np.where(finite & (ax > 0), ax, 1.0)
    _, e = np.frexp(safe)            # safe = f * 2**e, 0.5 <= f < 1
    E = np.maximum(e - 1, emin)      # 2**E <= |x| for normals; emin for subnormals
    quantum = np.ldexp(1.0, E - (p - 1))
    scaled = np.where(finite, x, 0.0) / quantum
    if mode == "rne":
        m = np.rint(scaled)
    elif mode == "down":
        m = np.floor(scaled)
    elif mode == "up":
        m = np.ceil(scaled)
    else:
        raise ValueError(mode)
    res = m * quantum
    # keep the sign of zero results (IEEE: the sign of the exact value)
    res = np.where(res == 0, np.copysign(0.0, x), res)
    big = np.ldexp(2.0 - 2.0 ** (1 - p), emax)
    if mode == "rne":
        res = np.where(res > big, np.inf, res)
        res = np.where(res < -big, -np.inf, res)
    elif mode == "down":
        res = np.where(res > big, big, res)
        res = np.where(res < -big, -np.inf, res)
    else:
        res = np.where(res > big, np.inf, res)
        res = np.where(res < -big, -big, res)
    res = np.where(finite, res, x)
    return res


def to_fp16(values_on_grid) -> np.ndarray:
    """Exact conversion of values already on the binary16 grid to float16."""
    v = np.asarray(values_on_grid, dtype=np.float64)
    h = v.astype(np.float16)
    ok = (h.astype(np.float64) == v) | np.isnan(v)
    if not np.all(ok):
        raise AssertionError("value not on the binary16 grid")
    return h


def rd16(x) -> np.ndarray:
    """float64 -> float16, rounding toward -inf."""
    return to_fp16(round_binary(x, "fp16", "down"))


def ru16(x) -> np.ndarray:
    """float64 -> float16, rounding toward +inf."""
    return to_fp16(round_binary(x, "fp16", "up"))


def rne_fp16(x) -> np.ndarray:
    """float64 -> float16 bit patterns (uint16), round to nearest even."""
    return to_fp16(round_binary(x, "fp16", "rne")).view(np.uint16)


def rne_bf16(x) -> np.ndarray:
    """float64 -> bfloat16 bit patterns (uint16), round to nearest even."""
    v = round_binary(x, "bf16", "rne")
    f = v.astype(np.float32)                     # exact: the bf16 grid is a subset
    if not np.all((f.astype(np.float64) == v) | np.isnan(v)):
        raise AssertionError("value not on the bfloat16 grid")
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def storage_to_f64(bits, dtype: str) -> np.ndarray:
    """uint16 storage of an fp16 / bf16 tensor -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16)
    if dtype == "fp16":
        return b.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        with np.errstate(invalid="ignore"):  # NaN patterns stay NaN; numpy flags their cast
            return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def f64_to_storage(x, dtype: str) -> np.ndarray:
    """float64 -> uint16 storage of ``dtype`` with round to nearest even."""
    if dtype == "fp16":
        return rne_fp16(x)
    if dtype == "bf16":
        return rne_bf16(x)
    raise ValueError(dtype)
