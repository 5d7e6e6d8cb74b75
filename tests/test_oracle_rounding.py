"""Pins of the fp16 / bf16 rounding: library conversions, exhaustive search, IEEE facts."""
import numpy as np
import torch

import oracle
from oracle import scalar
from conftest import golden_rows


def _samples(rng, n):
    # wide exponent range: subnormals, normals, overflow, exact grid points, midpoints
    mant = rng.uniform(-2, 2, n)
    expo = rng.integers(-30, 18, n)
    x = np.ldexp(mant, expo)
    grid = rng.integers(0, 0x7C00, n // 4).astype(np.uint16).view(np.float16).astype(np.float64)
    with np.errstate(over="ignore"):  # the largest finite value steps to inf on purpose
        nxt = np.nextafter(grid.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    mids = (grid + nxt) / 2
    return np.concatenate([x, grid, -grid, mids, -mids, [0.0, -0.0, 65504.0, 65520.0, -65520.0, 2.0**-25]])


def test_rne_fp16_matches_numpy_conversion():
    rng = np.random.default_rng(1)
    x = _samples(rng, 200000)
    ours = oracle.round_binary(x, "fp16", "rne")
    with np.errstate(over="ignore"):  # overflow to inf is part of what is compared
        ref = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(np.signbit(ours), np.signbit(ref))
    assert np.array_equal(ours, ref)


def test_rne_bf16_matches_torch_float32_conversion():
    rng = np.random.default_rng(2)
    bits = rng.integers(0, 2**32, 300000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ours = oracle.rne_bf16(f.astype(np.float64))
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_directed_rounding_matches_exhaustive_search():
    rng = np.random.default_rng(3)
    x = _samples(rng, 20000)
    x = x[np.abs(x) <= 65504.0]
    rd = oracle.round_binary(x, "fp16", "down")
    ru = oracle.round_binary(x, "fp16", "up")
    for v, a, b in zip(x, rd, ru):
        if v == 0.0:
            continue
        assert a == scalar.rd16_search(float(v))
        assert b == scalar.ru16_search(float(v))
    assert np.all(rd <= x) and np.all(ru >= x)


def test_ieee_binary16_facts():
    for row in golden_rows("fp16_rounding.txt"):
        expr, rd, ru, rne = row.split()
        x = float(eval(expr, {"__builtins__": {}}))
        assert int(oracle.rd16(x).view(np.uint16)) == int(rd, 16), expr
        assert int(oracle.ru16(x).view(np.uint16)) == int(ru, 16), expr
        assert int(oracle.rne_fp16(x)) == int(rne, 16), expr


def test_storage_round_trip():
    rng = np.random.default_rng(4)
    b = rng.integers(0, 65536, 50000).astype(np.uint16)
    for dt in ("fp16", "bf16"):
        v = oracle.storage_to_f64(b, dt)
        fin = np.isfinite(v)
        back = oracle.f64_to_storage(v[fin], dt)
        # -0 and +0 keep their patterns; every finite pattern maps to itself
        assert np.array_equal(back, b[fin])
