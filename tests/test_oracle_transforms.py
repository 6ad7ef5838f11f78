"""Pins for oracle.transforms."""
import numpy as np

from oracle import transforms as tr
from tests.conftest import read_golden
from tq_inputs import haar_orthogonal, sign_vector


def test_sylvester_h8_matches_hand_typed():
    h8 = np.array([[float(v) for v in r] for r in read_golden("sylvester_h8.txt")])
    assert np.array_equal(tr.sylvester_hadamard(8), h8)


def test_hadamard_orthogonality():
    for n in (1, 2, 16, 128, 2048):
        h = tr.sylvester_hadamard(n)
        assert np.array_equal(h @ h.T, n * np.eye(n))
        assert np.array_equal(h, h.T)


def test_haar_generator_orthogonal_fp32():
    pi = haar_orthogonal(128, 0)
    assert pi.dtype == np.float32
    p = pi.astype(np.float64)
    assert np.max(np.abs(p.T @ p - np.eye(128))) < 1e-6


def test_dense_rotation_preserves_geometry():
    pi = haar_orthogonal(64, 3)
    rot = tr.DenseRotation(pi)
    rg = np.random.default_rng(0)
    a, b = rg.standard_normal((2, 5, 64))
    ya, yb = rot.forward(a), rot.forward(b)
    assert np.allclose(np.sum(ya * yb, 1), np.sum(a * b, 1), atol=1e-5)
    assert np.allclose(rot.inverse(ya), a, atol=1e-5)


def test_hadamard_rotation_matches_explicit_product_and_inverts():
    d, dr = 6, 8
    eps = sign_vector(dr, 1)
    rot = tr.HadamardRotation(eps, d)
    h8 = np.array([[float(v) for v in r] for r in read_golden("sylvester_h8.txt")])
    rg = np.random.default_rng(1)
    u = rg.standard_normal((4, d))
    pad = np.concatenate([u, np.zeros((4, dr - d))], axis=1)
    expect = (h8 @ (eps[None, :] * pad).T).T / np.sqrt(dr)
    assert np.allclose(rot.forward(u), expect, atol=1e-13)
    assert np.allclose(rot.inverse(rot.forward(u)), u, atol=1e-13)
    assert np.allclose(np.linalg.norm(rot.forward(u), axis=1), np.linalg.norm(u, axis=1))


def test_hadamard_spreads_a_spike():
    # a vector with all its mass on one coordinate becomes flat: every
    # coordinate has magnitude 1/sqrt(d') (explainer page section 3)
    eps = sign_vector(128, 2)
    rot = tr.HadamardRotation(eps, 128)
    y = rot.forward(np.eye(128)[:1])
    assert np.allclose(np.abs(y), 1 / np.sqrt(128))
