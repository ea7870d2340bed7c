"""Pins of the oracle's rotation: Hadamard constructions and Pi."""

import itertools

import numpy as np
import pytest
from scipy import linalg

from oracle import (hadamard_sylvester, paley_hadamard_12, hadamard_matrix,
                    rotate, rotate_inverse, haar_rotation)


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 64, 128])
def test_sylvester_matches_library(d):
    # scipy builds H by the recursive Sylvester doubling; the oracle by popcount
    assert np.array_equal(hadamard_sylvester(d), linalg.hadamard(d).astype(float))


def test_brute_force_walsh_hadamard_tiny():
    d = 16
    x = np.random.default_rng(0).standard_normal(d)
    signs = np.array([1, -1] * 8)
    y = np.zeros(d)
    for i, j in itertools.product(range(d), range(d)):
        y[i] += (-1) ** bin(i & j).count("1") * signs[j] * x[j]
    assert np.allclose(rotate(x[None], signs)[0], y / 4.0, atol=1e-14)


def test_paley_12_is_hadamard():
    h = paley_hadamard_12()
    assert set(np.unique(h)) == {-1.0, 1.0}
    assert np.array_equal(h @ h.T, 12 * np.eye(12))


def test_kron_1536_orthogonal_and_chunk_structure():
    h = hadamard_matrix(1536)
    assert np.array_equal(h @ h.T, 1536 * np.eye(1536))
    # structure: order-128 transform inside each chunk, order-12 across chunks
    x = np.random.default_rng(1).standard_normal(1536)
    inner = x.reshape(12, 128) @ linalg.hadamard(128).T
    outer = paley_hadamard_12() @ inner
    assert np.allclose(h @ x, outer.ravel(), atol=1e-10)


@pytest.mark.parametrize("d", [8, 64, 128, 1536])
def test_rotation_orthogonal(d):
    rng = np.random.default_rng(d)
    signs = np.where(rng.random(d) < 0.5, -1, 1)
    x = rng.standard_normal((5, d))
    z = rotate(x, signs)
    assert np.allclose(np.linalg.norm(z, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14, atol=0)
    assert np.allclose(rotate_inverse(z, signs), x, atol=1e-13)
    # explicit matrix: Pi^T Pi = I
    pi = rotate(np.eye(d), signs).T
    assert np.allclose(pi.T @ pi, np.eye(d), atol=1e-13)
    # bool form of D (True = flipped) gives the same rotation
    assert np.array_equal(rotate(x, signs < 0), z)


def test_haar_orthogonal_and_isotropic():
    rng = np.random.default_rng(3)
    d = 16
    q = haar_rotation(d, rng)
    assert np.allclose(q.T @ q, np.eye(d), atol=1e-13)
    # the first row of Haar matrices: E[q_00^2] = 1/d, E[q_00] = 0
    s = np.array([haar_rotation(d, rng)[0, 0] for _ in range(4000)])
    assert abs(np.mean(s * s) - 1 / d) < 0.006
    assert abs(np.mean(s)) < 0.012
