"""The 8-bit encode decides again, in float64, every code whose binary32 t
lies within a bound of a tie.  With the in-register butterfly as the
transform, the bound takes the error of the unnormalized rotated value u as
log2(D) * 2^-24 * S, S = sum |x_j| of the row: each butterfly stage adds one
round-to-nearest binary32 addition per element, whose error is at most 2^-24
times the magnitude of a partial sum over a block of the row, and the blocks
of one stage are disjoint.  This checks that bound on the binary32 model of
the kernel's butterfly against the exact transform (the oracle's float64
product with the explicit Hadamard matrix), over rows built to stress it."""
import numpy as np
import pytest

import oracle
from kernel_models import butterfly_model

W = 2.0 ** -24
SEED = 11


def _rows(kind, D, n, rng):
    if kind == "gaussian":
        x = rng.standard_normal((n, D))
    elif kind == "outliers":       # a few channels x20, as in the K caches of the workloads
        x = rng.standard_normal((n, D))
        x[:, rng.choice(D, 4, replace=False)] *= 20.0
    elif kind == "spikes":         # sparse x50 spikes
        x = rng.standard_normal((n, D))
        x *= np.where(rng.random((n, D)) < 0.01, 50.0, 1.0)
    elif kind == "offset":         # large offset, small spread (bf16 keeps 8 bits of each value)
        x = 1000.0 + rng.standard_normal((n, D)) * 8.0
    elif kind == "binades":        # magnitudes spread over many binades
        x = rng.standard_normal((n, D)) * 2.0 ** rng.integers(-30, 30, (n, D))
    elif kind == "cancel":         # rows equal to +-1 times a Hadamard row plus noise: one large output
        H = oracle.hadamard(D)
        x = H[rng.integers(0, D, n)] * oracle.sign_vector(SEED, D) * 3.0 + rng.standard_normal((n, D)) * 1e-3
    else:
        raise ValueError(kind)
    # values exact in bf16, as the kernel reads them
    return oracle.storage_to_f64(oracle.f64_to_storage(x, "bf16"), "bf16")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kind", ["gaussian", "outliers", "spikes", "offset", "binades", "cancel"])
def test_butterfly_error_within_its_bound(D, kind):
    rng = np.random.default_rng(D * 7 + len(kind))
    rows = _rows(kind, D, 4000, rng)
    u = butterfly_model(rows, SEED, D)
    exact = oracle.rotate_raw(rows, oracle.sign_vector(SEED, D))
    S = np.abs(rows).sum(axis=1)
    # second-order terms (the (1 + 2^-24)^k growth of the partial sums) and the
    # float64 reference's own rounding are far below the 1e-6 relative slack
    bound = np.log2(D) * W * S * (1.0 + 1e-6)
    err = np.abs(u - exact).max(axis=1)
    ratio = err / np.where(bound > 0, bound, 1.0)
    assert (err <= bound).all(), "butterfly error above log2(D) w S by %.3g" % ratio.max()


def test_butterfly_model_rounds_each_addition():
    """Planted check: a model that skipped the binary32 rounding (float64
    additions) would make u exact; the binary32 model must not be exact on
    rows whose sums need more than 24 bits."""
    rng = np.random.default_rng(3)
    rows = _rows("binades", 128, 200, rng)
    u = butterfly_model(rows, SEED, 128)
    exact = oracle.rotate_raw(rows, oracle.sign_vector(SEED, 128))
    assert (u != exact).any()
    assert np.array_equal(u, u.astype(np.float32).astype(np.float64)), "u must be binary32 values"
