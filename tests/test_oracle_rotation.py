"""Pins for the oracle's rotations: orthogonality, Hadamard identities,
Haar sign convention, and the Gaussianisation the blog measures ("TurboQuant
on a 16GB MacBook", section "Round 1, Part 1": per-vector excess kurtosis
51 -> -0.13 on real keys; here on synthetic heavy-tailed keys)."""

import numpy as np
import pytest

from oracle import rotation as rot
import tq_inputs


def test_dense_orthogonal():
    P = rot.dense_rotation(tq_inputs.rotation_draws(0, 128))
    assert np.max(np.abs(P.T @ P - np.eye(128))) < 1e-6
    assert np.max(np.abs(P @ P.T - np.eye(128))) < 1e-6


def test_dense_qr_sign_convention():
    """Pi^T G is upper triangular with a positive diagonal (unique QR)."""
    G = tq_inputs.rotation_draws(5, 16)
    q, r = np.linalg.qr(G)
    P = q * np.sign(np.diag(r))[None, :]
    R = P.T @ G
    assert np.max(np.abs(np.tril(R, -1))) < 1e-12
    assert np.all(np.diag(R) > 0)
    assert np.allclose(rot.dense_rotation(G), P.astype(np.float32), atol=0)


def test_dense_reconstructs_draws():
    """G = Pi R: the stored rotation is the Q factor of the draws."""
    G = tq_inputs.rotation_draws(1, 64)
    P = rot.dense_rotation(G)
    R = P.T @ G
    assert np.max(np.abs(P @ np.triu(R) - G)) < 1e-5


@pytest.mark.parametrize("d", [2, 8, 128])
def test_hadamard_identities(d):
    H = rot.sylvester_hadamard(d)
    assert np.array_equal(H @ H, d * np.eye(d))
    assert np.array_equal(H, H.T)
    i, j = np.indices((d, d))
    pc = np.vectorize(lambda v: bin(v).count("1"))(i & j)
    assert np.array_equal(H, (-1.0) ** pc)
    x = np.random.default_rng(0).standard_normal((5, d))
    assert np.allclose(rot.fwht(x), x @ H, atol=1e-12)


@pytest.mark.parametrize("kind", ["dense", "hadamard"])
def test_round_trip(kind):
    d = 128
    draws = tq_inputs.rotation_draws(0, d) if kind == "dense" else tq_inputs.hadamard_draws(0, d)
    R = rot.Rotation(kind, draws, d)
    x = np.random.default_rng(1).standard_normal((10, d))
    assert np.max(np.abs(R.inverse(R.forward(x)) - x)) < 1e-5
    assert np.allclose(R.forward(x), x @ R.matrix.T, atol=1e-12 if kind == "hadamard" else 1e-12)
    assert np.allclose(np.linalg.norm(R.forward(x), axis=1), np.linalg.norm(x, axis=1), rtol=1e-6)


def _excess_kurtosis(v):
    c = v - v.mean(axis=1, keepdims=True)
    m2 = np.mean(c ** 2, axis=1)
    m4 = np.mean(c ** 4, axis=1)
    return m4 / m2 ** 2 - 3.0


def test_gaussianisation_config0_keys(golden):
    """Synthetic config-0 keys: heavy tails before, near-Gaussian after a dense
    rotation (the page reports mean -0.13 after on real keys)."""
    d, T = 128, 1024
    k = tq_inputs.fp16(tq_inputs.keys(0, d, np.arange(T))).astype(np.float64)
    before = _excess_kurtosis(k)
    R = rot.Rotation("dense", tq_inputs.rotation_draws(0, d), d)
    after = _excess_kurtosis(R.forward(k))
    assert before.mean() > 10.0
    assert abs(after.mean()) < 0.3
    assert after.max() < 3.0
    assert golden["rotation_kurtosis"]["before_mean"] > 10 and abs(golden["rotation_kurtosis"]["after_mean"]) < 0.3
