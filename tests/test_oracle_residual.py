"""Pins of the oracle's residual-stream step (post-norm of the block output,
depth-scaled residual)."""

import numpy as np
import pytest

import oracle
from oracle import residual


def test_step_weights_square_sum_to_one():
    for k in range(2, 106):
        keep, add = residual.step_weights(k)
        assert abs(keep * keep + add * add - 1.0) < 1e-15


def test_stream_is_the_scaled_sum_of_contributions():
    """Launch post, "Residual Stream" (and the model doc's sandwich-norm
    note): after k steps the stream is the sum of the k contributions divided
    by sqrt(k), every contribution with the same weight. Contributions here
    are already unit-RMS rows, so the post-norm leaves them unchanged."""
    rng = np.random.default_rng(0)
    H, K = 64, 105  # 52 layers x 2 sublayers + the embedding
    contrib = rng.normal(size=(K, 1, H))
    contrib /= np.sqrt(np.mean(contrib ** 2, axis=-1, keepdims=True))
    stream = contrib[0]
    for k in range(2, K + 1):
        stream = residual.residual_update(stream, contrib[k - 1], np.ones(H), 0.0, k)
    expected = contrib.sum(axis=0) / np.sqrt(K)
    assert np.allclose(stream, expected, rtol=1e-12, atol=1e-12)


def test_rms_norm_closed_forms():
    rng = np.random.default_rng(1)
    v = rng.normal(size=(5, 128)) * 3.0
    n = residual.rms_norm(v, np.ones(128), 0.0)
    assert np.allclose(np.mean(n * n, axis=-1), 1.0, rtol=1e-12)
    # scale invariance (eps = 0) and the gain acting per channel
    assert np.allclose(residual.rms_norm(7.5 * v, np.ones(128), 0.0), n, rtol=1e-12)
    g = rng.uniform(0.5, 2.0, size=128)
    assert np.allclose(residual.rms_norm(v, g, 0.0), n * g, rtol=1e-12)
    # eps: a zero row stays zero; a row of ones with eps gives 1 / sqrt(1 + eps)
    assert np.all(residual.rms_norm(np.zeros((1, 8)), np.ones(8), 1e-6) == 0.0)
    assert np.allclose(residual.rms_norm(np.ones((1, 8)), np.ones(8), 0.25), 1.0 / np.sqrt(1.25))


@pytest.mark.parametrize("k", [2, 3, 53, 105])
def test_update_matches_hand_formula(k):
    rng = np.random.default_rng(k)
    s = rng.normal(size=(3, 32))
    o = rng.normal(size=(3, 32))
    g = rng.uniform(0.5, 1.5, size=32)
    eps = 1e-6
    got = residual.residual_update(s, o, g, eps, k)
    ref = np.empty_like(s)
    for t in range(3):
        rms = np.sqrt(sum(x * x for x in o[t]) / 32 + eps)
        for c in range(32):
            ref[t, c] = s[t, c] * np.sqrt((k - 1) / k) + o[t, c] / rms * g[c] / np.sqrt(k)
    assert np.allclose(got, ref, rtol=1e-13)


def test_oracle_package_exports_residual():
    assert oracle.residual is residual
