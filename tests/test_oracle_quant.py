"""Pins of quantization and packing: error bound, exact grids, constant groups,
brute force on tiny tensors, hand-worked packing."""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import scalar
from conftest import golden_rows


def _rotated_raw(rng, n, D, spread=1.0, offset=0.0):
    x = rng.normal(size=(n, D)) * spread + offset
    return oracle.rotate_raw(x, oracle.sign_vector(5, D))


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("G", [32, 64, 128])
def test_error_bound_and_code_range(bits, G):
    rng = np.random.default_rng(bits * 1000 + G)
    D = 128
    qmax = 2 ** bits - 1
    u = np.concatenate([_rotated_raw(rng, 2000, D), _rotated_raw(rng, 200, D, spread=30.0)])
    y = u / np.sqrt(D)
    scale, zero = oracle.group_meta(u, G, bits)
    q, t = oracle.quantize(u, scale, zero, G, bits)
    slack = 1e-6 * (qmax + 1)   # binary32 rounding of t: a few ulps of max(|t|, |zero/scale|)
    assert t.min() >= -slack and t.max() <= qmax + slack
    yhat = oracle.dequantize(q, scale, zero, G)
    sc = np.repeat(scale.astype(np.float64), G, axis=-1)
    assert np.all(np.abs(y - yhat) <= sc * (0.5 + slack))
    # the stored zero is a lower bound of its group (up to one binary32 rounding
    # of the normalized minimum), zero + (2^b-1)*scale an upper one
    yg = y.reshape(len(y), -1, G)
    lo = yg.min(-1)
    hi = yg.max(-1)
    assert np.all(zero.astype(np.float64) <= lo + 2.0 ** -22 * np.abs(lo))
    assert np.all(zero.astype(np.float64) + qmax * scale.astype(np.float64) >= hi - 2.0 ** -22 * np.abs(hi))


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_degenerate_groups_stay_in_range(bits):
    """Huge offset, tiny range: binary32 error in t is ~|y / scale| * 2^-23, the
    clamp keeps codes in [0, 2^b - 1], and the error bound holds up to it."""
    rng = np.random.default_rng(bits)
    D, G = 128, 32
    qmax = 2 ** bits - 1
    y = np.concatenate([1000.0 + 0.01 * rng.random((200, D)), -700.0 + 0.003 * rng.random((200, D)),
                        np.full((4, D), 3.0) + np.linspace(0, 1e-5, D)])
    u = y * np.sqrt(D)
    scale, zero = oracle.group_meta(u, G, bits)
    q, t = oracle.quantize(u, scale, zero, G, bits)
    assert q.max() <= qmax
    yhat = oracle.dequantize(q, scale, zero, G)
    sc = np.repeat(scale.astype(np.float64), G, axis=-1)
    slack = np.abs(y) * 2.0 ** -21
    assert np.all(np.abs(y - yhat) <= sc / 2 + slack)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_exact_grid_groups_round_trip(bits):
    """D = 64 (1/sqrt(D) = 1/8 exactly): y = zero + k * scale on fp16 grids."""
    rng = np.random.default_rng(bits)
    G, D = 32, 64
    rows = []
    codes = []
    for _ in range(50):
        row, crow = [], []
        for g in range(D // G):
            z = float(np.float16(rng.uniform(-8, 8)))
            s = float(np.float16(rng.uniform(0.01, 0.5)))
            k = rng.integers(0, 2 ** bits, G)
            k[0], k[1] = 0, 2 ** bits - 1
            rng.shuffle(k)
            row.extend(z + k * s)
            crow.extend(k)
        rows.append(row)
        codes.append(crow)
    y = np.array(rows)
    u = y * 8.0
    scale, zero = oracle.group_meta(u, G, bits)
    q, _ = oracle.quantize(u, scale, zero, G, bits)
    assert np.array_equal(q, np.array(codes, dtype=np.uint8))
    assert np.array_equal(oracle.dequantize(q, scale, zero, G), y)


def test_constant_groups():
    G, D = 64, 128
    u = np.zeros((3, D))
    u[1] = 0.375 * 8.0           # D=64 below: 1/sqrt(D) = 1/8
    u[2, :64] = -3.25 * 8.0
    u[2, 64:] = np.linspace(0, 8, 64)
    u = u[:, :64].copy(), u[:, 64:].copy()
    u = np.concatenate([u[0], u[1]], axis=1)[:, :64]
    uu = np.zeros((3, 64))
    uu[1] = 0.375 * 8.0
    uu[2, :32] = -3.25 * 8.0
    uu[2, 32:] = np.linspace(0, 8, 32)
    scale, zero = oracle.group_meta(uu, 32, 4)
    q, t = oracle.quantize(uu, scale, zero, 32, 4)
    assert scale[0, 0] == 0 and scale[1, 0] == 0 and scale[2, 0] == 0
    assert np.all(q[:2] == 0) and np.all(q[2, :32] == 0)
    assert np.array_equal(oracle.dequantize(q, scale, zero, 32)[:2], uu[:2] / 8.0)
    assert np.all(oracle.dequantize(q, scale, zero, 32)[2, :32] == -3.25)
    assert scale[2, 1] > 0


def test_binary32_helpers_are_exact():
    """fl / div_f32 / the fused multiply-add against exact rational rounding."""
    rng = np.random.default_rng(5)
    a = rng.normal(size=3000) * np.exp(rng.uniform(-20, 20, 3000))
    assert np.array_equal(oracle.fl(a), np.array([scalar.f32_round(float(v)) for v in a]))
    num = oracle.fl(rng.normal(size=3000) * 100)
    den = oracle.fl(np.abs(rng.normal(size=3000)) * 10 + 1e-3)
    den[:500] = np.float16(np.abs(rng.normal(size=500))).astype(np.float64) + 2.0 ** -10
    num[:500] = 1.0
    got = oracle.div_f32(num, den)
    want = [scalar.f32_round(Fraction(float(n)) / Fraction(float(d))) for n, d in zip(num, den)]
    assert np.array_equal(got, np.array(want))
    x, y, z = oracle.fl(rng.normal(size=(3, 3000)) * 50)
    fused = oracle.fl(x * y + z)
    want = [scalar.f32_round(Fraction(float(p)) * Fraction(float(q)) + Fraction(float(r)))
            for p, q, r in zip(x, y, z)]
    assert np.array_equal(fused, np.array(want))


def test_packing_worked_examples():
    for row in golden_rows("packing.txt"):
        b, codes, byts = (part.split() for part in row.split("|"))
        bits = int(b[0])
        q = np.array([[int(c) for c in codes]], dtype=np.uint8)
        want = np.array([[int(x, 16) for x in byts]], dtype=np.uint8)
        assert np.array_equal(oracle.pack_codes(q, bits), want)
        assert np.array_equal(oracle.unpack_codes(want, bits, q.shape[1]), q)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_every_byte_pattern_round_trips(bits):
    allb = np.arange(256, dtype=np.uint8).reshape(-1, 1).repeat(4, axis=1)
    D = 4 * 8 // bits
    q = oracle.unpack_codes(allb, bits, D)
    assert q.max() < 2 ** bits
    assert np.array_equal(oracle.pack_codes(q, bits), allb)


@pytest.mark.parametrize("bits,G,seed", list(itertools.product([2, 4, 8], [4, 8], [0, 1, 99])))
def test_brute_force_4x8(bits, G, seed):
    """4 rows x D=8: the numpy oracle equals the brute-force scalar twin."""
    rng = np.random.default_rng(bits * 100 + G * 10 + seed)
    for dt in ("bf16", "fp16"):
        xb = oracle.f64_to_storage(rng.normal(size=(4, 8)) * 3, dt)
        x = oracle.storage_to_f64(xb, dt)
        s = oracle.sign_vector(seed, 8)
        u = oracle.rotate_raw(x, s)
        scale, zero = oracle.group_meta(u, G, bits)
        q, _ = oracle.quantize(u, scale, zero, G, bits)
        packed = oracle.pack_codes(q, bits)
        sp, sm, sc = scalar.encode_rows(x.tolist(), 8, G, bits, seed)
        assert np.array_equal(packed, np.array(sp, dtype=np.uint8))
        assert np.array_equal(q, np.array(sc, dtype=np.uint8))
        assert np.array_equal(scale.view(np.uint16), np.array([[m[0] for m in r] for r in sm], dtype=np.uint16))
        assert np.array_equal(zero.view(np.uint16), np.array([[m[1] for m in r] for r in sm], dtype=np.uint16))
        yhat = oracle.dequantize(q, scale, zero, G)
        xhat = oracle.unrotate(yhat, s)
        ob, ov = scalar.decode_rows(sp, sm, 8, G, bits, seed, dt)
        assert np.array_equal(oracle.f64_to_storage(xhat, dt), np.array(ob, dtype=np.uint16))
        assert np.allclose(xhat, np.array(ov), rtol=0, atol=1e-12)


def test_reconstruction_error_equals_rotated_error():
    rng = np.random.default_rng(11)
    D, G, bits = 128, 64, 4
    x = rng.normal(size=(300, D))
    s = oracle.sign_vector(2, D)
    u = oracle.rotate_raw(x, s)
    y = u / np.sqrt(D)
    scale, zero = oracle.group_meta(u, G, bits)
    q, _ = oracle.quantize(u, scale, zero, G, bits)
    yhat = oracle.dequantize(q, scale, zero, G)
    xhat = oracle.unrotate(yhat, s)
    ex = np.linalg.norm(x - xhat, axis=1)
    ey = np.linalg.norm(y - yhat, axis=1)
    assert np.allclose(ex, ey, rtol=1e-12, atol=0)
    assert np.all(ey <= np.sqrt(D) * scale.astype(np.float64).max(axis=1) / 2)
