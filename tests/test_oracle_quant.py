"""Pins of quantization and packing: error bound, exact grids, constant groups,
brute force on tiny tensors, hand-worked packing."""
import itertools

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
    rng = np.random.default_rng(bits * 1000 + G)
    y = np.concatenate([
        _rotated(rng, 2000, 128),
        _rotated(rng, 200, 128, spread=30.0),
        # large offset with a tiny range: the fp16 ulp of the zero is far
        # larger than the group's spread (where round-to-nearest would clamp)
        1000.0 + 0.01 * rng.random((200, 128)),
        -700.0 + 0.003 * rng.random((200, 128)),
    ])
    scale, zero = oracle.group_meta(y, G, bits)
    q, t = oracle.quantize(y, scale, zero, G, bits)
    assert t.min() >= 0.0 and t.max() <= 2 ** bits - 1
    yhat = oracle.dequantize(q, scale, zero, G)
    bound = np.repeat(scale.astype(np.float64), G, axis=-1) / 2
    assert np.all(np.abs(y - yhat) <= bound)
    # the stored zero is a lower bound of its group, zero + (2^b-1)*scale an upper one
    yg = y.reshape(len(y), -1, G)
    assert np.all(zero.astype(np.float64) <= yg.min(-1))
    assert np.all(zero.astype(np.float64) + (2 ** bits - 1) * scale.astype(np.float64) >= yg.max(-1))


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_exact_grid_groups_round_trip(bits):
    rng = np.random.default_rng(bits)
    G, D = 32, 128
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
    scale, zero = oracle.group_meta(y, G, bits)
    q, _ = oracle.quantize(y, scale, zero, G, bits)
    assert np.array_equal(q, np.array(codes, dtype=np.uint8))
    assert np.array_equal(oracle.dequantize(q, scale, zero, G), y)


def test_constant_groups():
    G = 64
    y = np.zeros((3, 128))
    y[1] = 0.375          # on the fp16 grid
    y[2, :64] = -3.25
    y[2, 64:] = np.linspace(0, 1, 64)
    scale, zero = oracle.group_meta(y, G, 4)
    q, t = oracle.quantize(y, scale, zero, G, 4)
    assert scale[0, 0] == 0 and scale[1, 0] == 0 and scale[2, 0] == 0
    assert np.all(q[:2] == 0) and np.all(q[2, :64] == 0)
    assert np.array_equal(oracle.dequantize(q, scale, zero, G)[:2], y[:2])
    assert np.all(oracle.dequantize(q, scale, zero, G)[2, :64] == -3.25)


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
