"""Pins of the transform: Hadamard identities, scipy, closed forms, worked example."""
import numpy as np
import pytest
import scipy.linalg

import oracle
from conftest import golden_rows


@pytest.mark.parametrize("D", [2, 8, 64, 128])
def test_hadamard_orthogonal_and_equals_scipy(D):
    H = oracle.hadamard(D)
    assert np.array_equal(H @ H.T, D * np.eye(D))
    assert np.array_equal(H, scipy.linalg.hadamard(D).astype(np.float64))
    assert np.array_equal(H, H.T)


def test_worked_examples():
    for row in golden_rows("hadamard_worked.txt"):
        lhs, rhs = row.split("|")
        vals = [float(v) for v in lhs.split()]
        D, x = int(vals[0]), np.array(vals[1:])
        y = np.array([float(v) for v in rhs.split()])
        got = oracle.rotate(x[None, :], np.ones(D))[0]
        assert np.allclose(got, y, rtol=0, atol=1e-15)


@pytest.mark.parametrize("D", [64, 128])
def test_norm_preservation_and_round_trip(D):
    rng = np.random.default_rng(D)
    x = rng.normal(size=(500, D)) * rng.uniform(0.1, 30, size=(500, 1))
    s = oracle.sign_vector(7, D)
    y = oracle.rotate(x, s)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14, atol=0)
    back = oracle.unrotate(y, s)
    assert np.max(np.abs(back - x)) <= 1e-14 * np.max(np.abs(x))
    # only quantization loses information: the transform alone round-trips
    # bit-exactly once the result is rounded back to the storage format
    for dt in ("bf16", "fp16"):
        xb = oracle.f64_to_storage(x, dt)
        xv = oracle.storage_to_f64(xb, dt)
        rt = oracle.f64_to_storage(oracle.unrotate(oracle.rotate(xv, s), s), dt)
        assert np.array_equal(rt, xb)


@pytest.mark.parametrize("D", [8, 64, 128])
def test_closed_forms(D):
    ones = np.ones(D)
    s = oracle.sign_vector(3, D)
    for k in (0, 1, D // 2 - 1, D - 1):
        e = np.zeros(D)
        e[k] = 1.0
        expect = np.array([(-1.0) ** bin(i & k).count("1") for i in range(D)]) / np.sqrt(D)
        assert np.allclose(oracle.rotate(e[None], ones)[0], expect, rtol=0, atol=1e-15)
        assert np.allclose(oracle.rotate(e[None], s)[0], s[k] * expect, rtol=0, atol=1e-15)
    c = 2.5
    y = oracle.rotate(np.full((1, D), c), ones)[0]
    expect = np.zeros(D)
    expect[0] = c * np.sqrt(D)
    assert np.allclose(y, expect, rtol=0, atol=1e-12)


@pytest.mark.parametrize("D,G", [(64, 32), (64, 64), (128, 32), (128, 64), (128, 128)])
def test_group_factorization(D, G):
    """H_D = H_{D/G} (x) H_G in Sylvester order, and the decode's reordering:
    transforming zero + scale * q equals transforming the integer codes within
    each group, scaling, adding zero * G at each group's first element, then
    combining groups with H_{D/G} (x) I_G.  Exact in fp64 on these values."""
    H = oracle.hadamard(D)
    assert np.array_equal(H, np.kron(oracle.hadamard(D // G), oracle.hadamard(G)))
    rng = np.random.default_rng(D + G)
    for bits in (2, 4, 8):
        q = rng.integers(0, 2 ** bits, size=(5, D)).astype(np.float64)
        scale = rng.integers(1, 64, size=(5, D // G)) / 1024.0
        zero = rng.integers(-512, 512, size=(5, D // G)) / 256.0
        yhat = oracle.dequantize(q, scale, zero, G)
        direct = yhat @ H.T
        inner = (q.reshape(5, D // G, G) @ oracle.hadamard(G).T) * scale[..., None]
        inner[..., 0] += zero * G
        outer = np.kron(oracle.hadamard(D // G), np.eye(G))
        assert np.array_equal(direct, inner.reshape(5, D) @ outer.T)
