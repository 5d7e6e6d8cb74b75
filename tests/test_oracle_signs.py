"""Pins of the sign generator: published SplitMix64 outputs and statistics."""
import numpy as np

import oracle
from conftest import golden_rows


def test_splitmix64_published_vectors():
    rows = [r.split() for r in golden_rows("splitmix64.txt")]
    for seed, idx, hexout in rows:
        outs = oracle.splitmix64_outputs(int(seed), int(idx) + 1)
        assert outs[int(idx)] == int(hexout, 16)


def test_signs_follow_bit63_and_are_counter_based():
    for seed in (0, 1, 2**63, 2**64 - 1, 12345):
        outs = oracle.splitmix64_outputs(seed, 128)
        s = oracle.sign_vector(seed, 128)
        assert np.array_equal(s, np.where([(z >> 63) & 1 for z in outs], -1.0, 1.0))
        assert np.array_equal(oracle.sign_vector(seed, 64), s[:64])
        mask = oracle.sign_bits_mask(seed, 128)
        assert all(((mask >> j) & 1) == (s[j] < 0) for j in range(128))


def test_sign_statistics():
    # number of -1 entries ~ Binomial(128, 1/2): mean 64, sd sqrt(32)
    counts = np.array([(oracle.sign_vector(seed, 128) < 0).sum() for seed in range(400)])
    assert abs(counts.mean() - 64) < 4 * np.sqrt(32) / np.sqrt(len(counts))
    assert counts.min() > 64 - 6 * np.sqrt(32) and counts.max() < 64 + 6 * np.sqrt(32)
    # per-coordinate balance across seeds
    S = np.array([oracle.sign_vector(seed, 64) for seed in range(400)])
    assert np.all(np.abs(S.mean(axis=0)) < 6 / np.sqrt(400))
