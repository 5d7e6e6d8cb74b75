"""Pins of quantization and packing: the exact definition of the meta and the
codes (brute force in exact arithmetic), error bound, exact grids, ties,
constant groups, degenerate groups, hand-worked packing."""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import scalar
from conftest import golden_rows


def _rotated(rng, n, D, spread=1.0, offset=0.0):
    x = rng.normal(size=(n, D)) * spread + offset
    return oracle.rotate(x, oracle.sign_vector(5, D))


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("G", [32, 64, 128])
def test_error_bound_and_code_range(bits, G):
    """The quantizer's invariant, exact in float64: 0 <= t <= 2^b - 1 and
    |y - yhat| <= scale / 2 for every element, zero <= min y and
    zero + (2^b - 1) scale >= max y for every group."""
    rng = np.random.default_rng(bits * 1000 + G)
    D = 128
    qmax = 2 ** bits - 1
    y = np.concatenate([_rotated(rng, 2000, D), _rotated(rng, 200, D, spread=30.0),
                        _rotated(rng, 200, D, spread=0.01, offset=3.0)])
    scale, zero = oracle.group_meta(y, G, bits)
    q, t = oracle.quantize(y, scale, zero, G, bits)
    eps = 1e-12
    assert t.min() >= -eps and t.max() <= qmax * (1 + eps)
    yhat = oracle.dequantize(q, scale, zero, G)
    sc = np.repeat(scale.astype(np.float64), G, axis=-1)
    assert np.all(np.abs(y - yhat) <= sc * (0.5 + eps))
    yg = y.reshape(len(y), -1, G)
    assert np.all(zero.astype(np.float64) <= yg.min(-1))
    assert np.all(zero.astype(np.float64) + qmax * scale.astype(np.float64) >= yg.max(-1))
    # and the meta is the tightest fp16 pair: one fp16 step up for zero, or
    # down for scale, breaks the bounds above
    z_up = np.nextafter(zero, np.float16(np.inf)).astype(np.float64)
    assert np.all(z_up > yg.min(-1))
    s_dn = np.nextafter(scale, np.float16(-np.inf)).astype(np.float64)
    pos = scale > 0
    assert np.all((zero.astype(np.float64) + qmax * s_dn < yg.max(-1))[pos])


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_codes_are_the_nearest_level(bits):
    """Against an argmin over every code level (float64 brute force): the code
    is the level nearest to y; equal distances only at exact midpoints."""
    rng = np.random.default_rng(40 + bits)
    G, D = 32, 64
    y = _rotated(rng, 300, D) * rng.uniform(0.1, 10, size=(300, 1))
    scale, zero = oracle.group_meta(y, G, bits)
    q, _ = oracle.quantize(y, scale, zero, G, bits)
    levels = zero.astype(np.float64)[..., None] + np.arange(2 ** bits) * scale.astype(np.float64)[..., None]
    dist = np.abs(y.reshape(300, -1, G)[..., None] - levels[..., None, :])      # [n, groups, G, codes]
    best = dist.argmin(-1).reshape(y.shape)
    assert np.array_equal(q, best.astype(np.uint8))


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_codes_match_exact_brute_force(bits):
    """Random y, meta and codes against the exact twin (y taken as exact
    rationals, D = 1): RD16 / RU16 by search over every fp16 value and the
    code by exact argmin over all 2^b levels."""
    rng = np.random.default_rng(70 + bits)
    G = 16
    y = rng.normal(size=(12, G)) * np.exp(rng.uniform(-6, 6, size=(12, 1))) + rng.normal(size=(12, 1))
    scale, zero = oracle.group_meta(y, G, bits)
    q, _ = oracle.quantize(y, scale, zero, G, bits)
    qmax = 2 ** bits - 1
    for r in range(len(y)):
        u = [Fraction(float(v)) for v in y[r]]
        z = scalar.rd16_exact(min(u), 1)
        s = scalar.ru16_scale(max(u), 1, z, qmax)
        assert z == Fraction(float(zero[r, 0])) and s == Fraction(float(scale[r, 0]))
        assert [scalar.nearest_code(v, 1, z, s, qmax) for v in u] == q[r].tolist()


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_exact_ties_go_to_the_even_code(bits):
    """y exactly halfway between two levels: both the numpy oracle and the twin
    pick the even code (round half to even)."""
    qmax = 2 ** bits - 1
    z, s = Fraction(-3, 4), Fraction(3, 64)          # both exact in fp16
    for k in range(qmax):
        mid = z + (k + Fraction(1, 2)) * s            # exact in float64 too
        want = k if k % 2 == 0 else k + 1
        assert scalar.nearest_code(mid, 1, z, s, qmax) == want
        t = oracle.code_values(np.array([[float(mid)]]), np.array([[np.float16(float(s))]]),
                               np.array([[np.float16(float(z))]]), 1)
        assert t[0, 0] == k + 0.5
        assert oracle.nearest_codes(t, bits)[0, 0] == want


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_degenerate_groups_stay_in_range(bits):
    """Huge offset, tiny range: the exact definition keeps every code in
    [0, 2^b - 1] and the error bound |y - yhat| <= scale / 2 holds."""
    rng = np.random.default_rng(bits)
    D, G = 128, 32
    qmax = 2 ** bits - 1
    y = np.concatenate([1000.0 + 0.01 * rng.random((200, D)), -700.0 + 0.003 * rng.random((200, D)),
                        np.full((4, D), 3.0) + np.linspace(0, 1e-5, D)])
    scale, zero = oracle.group_meta(y, G, bits)
    q, t = oracle.quantize(y, scale, zero, G, bits)
    assert q.max() <= qmax and t.min() >= -1e-9 and t.max() <= qmax + 1e-9
    yhat = oracle.dequantize(q, scale, zero, G)
    sc = np.repeat(scale.astype(np.float64), G, axis=-1)
    assert np.all(np.abs(y - yhat) <= sc / 2 + np.abs(y) * 2.0 ** -50)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_exact_grid_groups_round_trip(bits):
    """y = zero + k * scale on fp16 grids, with the extreme codes present:
    the meta is (scale, zero) again, the codes are k and yhat == y."""
    rng = np.random.default_rng(bits)
    G, D = 32, 64
    rows, codes, metas = [], [], []
    for _ in range(50):
        row, crow, mrow = [], [], []
        for g in range(D // G):
            z = float(np.float16(rng.uniform(-8, 8)))
            s = float(np.float16(rng.uniform(0.01, 0.5)))
            k = rng.integers(0, 2 ** bits, G)
            k[0], k[1] = 0, 2 ** bits - 1
            rng.shuffle(k)
            row.extend(z + k * s)
            crow.extend(k)
            mrow.append((s, z))
        rows.append(row)
        codes.append(crow)
        metas.append(mrow)
    y = np.array(rows)
    scale, zero = oracle.group_meta(y, G, bits)
    assert np.array_equal(scale.astype(np.float64), np.array([[m[0] for m in r] for r in metas]))
    assert np.array_equal(zero.astype(np.float64), np.array([[m[1] for m in r] for r in metas]))
    q, _ = oracle.quantize(y, scale, zero, G, bits)
    assert np.array_equal(q, np.array(codes, dtype=np.uint8))
    assert np.array_equal(oracle.dequantize(q, scale, zero, G), y)


def test_constant_groups():
    """Constant groups (all-zero vectors among them) get scale 0 and codes 0,
    and decode to the stored zero exactly; a zero minimum is stored as +0."""
    y = np.zeros((3, 64))
    y[1] = 0.375
    y[2, :32] = -3.25
    y[2, 32:] = np.linspace(0, 1, 32)
    scale, zero = oracle.group_meta(y, 32, 4)
    q, t = oracle.quantize(y, scale, zero, 32, 4)
    assert np.all(scale[:2] == 0) and scale[2, 0] == 0 and scale[2, 1] > 0
    assert np.all(q[:2] == 0) and np.all(q[2, :32] == 0)
    assert np.array_equal(oracle.dequantize(q, scale, zero, 32)[:2], y[:2])
    assert np.all(oracle.dequantize(q, scale, zero, 32)[2, :32] == -3.25)
    assert zero[0, 0].view(np.uint16) == 0 and zero[2, 1].view(np.uint16) == 0
    neg = oracle.group_meta(-np.zeros((1, 64)), 32, 4)[1]
    assert np.all(neg.view(np.uint16) == 0)


def test_overflowing_meta_raises():
    with pytest.raises(OverflowError):
        oracle.group_meta(np.full((1, 32), 70000.0), 32, 4)
    # inside the range the widest group still has a finite scale (131008 / 3)
    sc, ze = oracle.group_meta(np.concatenate([np.full((1, 16), -65504.0), np.full((1, 16), 65504.0)], 1), 32, 2)
    assert float(ze[0, 0]) == -65504.0 and float(sc[0, 0]) == float(np.float16(131008 / 3 + 16))


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
    """4 rows x D=8: the float64 oracle equals the exact brute-force twin --
    meta, codes, packed bytes and the decoded bit patterns."""
    rng = np.random.default_rng(bits * 100 + G * 10 + seed)
    for dt in ("bf16", "fp16"):
        xb = oracle.f64_to_storage(rng.normal(size=(4, 8)) * 3, dt)
        x = oracle.storage_to_f64(xb, dt)
        s = oracle.sign_vector(seed, 8)
        y = oracle.rotate(x, s)
        scale, zero = oracle.group_meta(y, G, bits)
        q, _ = oracle.quantize(y, scale, zero, G, bits)
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
    y = oracle.rotate(x, s)
    scale, zero = oracle.group_meta(y, G, bits)
    q, _ = oracle.quantize(y, scale, zero, G, bits)
    yhat = oracle.dequantize(q, scale, zero, G)
    xhat = oracle.unrotate(yhat, s)
    ex = np.linalg.norm(x - xhat, axis=1)
    ey = np.linalg.norm(y - yhat, axis=1)
    assert np.allclose(ex, ey, rtol=1e-12, atol=0)
    assert np.all(ey <= np.sqrt(D) * scale.astype(np.float64).max(axis=1) / 2)
