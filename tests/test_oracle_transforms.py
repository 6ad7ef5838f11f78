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


def _h8():
    return np.array([[float(v) for v in r] for r in read_golden("sylvester_h8.txt")])


def test_two_round_hadamard_matches_explicit_product_and_inverts():
    # (H D2 / sqrt 8)(H D1 / sqrt 8) pad(u) from the hand-typed H8: round 1 first
    d, dr = 6, 8
    eps = np.stack([sign_vector(dr, 3), sign_vector(dr, 4)])
    rot = tr.HadamardRotation(eps, d)
    h8 = _h8()
    m = (h8 @ np.diag(eps[1]) @ h8 @ np.diag(eps[0])) / 8.0
    rg = np.random.default_rng(2)
    u = rg.standard_normal((5, d))
    pad = np.concatenate([u, np.zeros((5, dr - d))], axis=1)
    assert np.allclose(rot.forward(u), pad @ m.T, atol=1e-13)
    assert not np.allclose(rot.forward(u), pad @ ((h8 @ np.diag(eps[0]) @ h8 @ np.diag(eps[1])) / 8.0).T)
    assert np.allclose(rot.inverse(rot.forward(u)), u, atol=1e-13)
    # orthogonal: lengths and inner products kept
    full = tr.HadamardRotation(eps, dr).forward(np.eye(dr))
    assert np.allclose(full @ full.T, np.eye(dr), atol=1e-13)


def _all_signs(n):
    return np.array([[1.0 if (i >> j) & 1 else -1.0 for j in range(n)] for i in range(1 << n)])


def test_multi_round_second_moment_is_one_over_d_exactly():
    # over the random signs, E[y_j^2] = ||u||^2 / d for any input and any
    # number of rounds (each round's signs decorrelate the coordinates):
    # exact average over every sign pattern of the last round at d = 8
    d = 8
    rg = np.random.default_rng(5)
    u = rg.standard_normal(d)
    u /= np.linalg.norm(u)
    first = sign_vector(d, 6)
    acc = np.zeros(d)
    signs = _all_signs(d)
    for e2 in signs:
        acc += tr.HadamardRotation(np.stack([first, e2]), d).forward(u[None, :])[0] ** 2
    assert np.allclose(acc / len(signs), 1.0 / d, atol=1e-14)


def test_two_round_fourth_moment_of_a_spike():
    # For u = e_1 one round gives |y_j| = 1/sqrt(d) exactly (E[y^4] = 1/d^2),
    # a third of the uniform rotation's 3 / (d (d + 2)) (blog notes, Lemma 1's
    # density).  Two rounds give y_j = +-(sum_k H_jk eps2_k) / d, and for a
    # sum of d independent signs E[(sum)^4] = 3 d^2 - 2 d, so
    # E[y_j^4] = (3 d - 2) / d^3: checked exactly over every sign pattern at d = 8.
    d = 8
    e1 = np.eye(d)[:1]
    signs = _all_signs(d)
    m4 = np.zeros(d)
    for e2 in signs:
        m4 += tr.HadamardRotation(np.stack([np.ones(d), e2]), d).forward(e1)[0] ** 4
    m4 /= len(signs)
    assert np.allclose(m4, (3 * d - 2) / d ** 3, atol=1e-15)
    one_round = tr.HadamardRotation(np.ones(d), d).forward(e1)[0] ** 4
    assert np.allclose(one_round, 1.0 / d ** 2)
    # both tend to 3 / d^2: at d = 128 two rounds are within 1.1% of the
    # uniform rotation's fourth moment, one round a factor of three away
    big = 128
    assert abs((3 * big - 2) / big ** 3 / (3.0 / (big * (big + 2))) - 1) < 0.011
    assert (3.0 / (big * (big + 2))) / (1.0 / big ** 2) > 2.9


def test_two_round_coordinates_follow_lemma_1():
    # a generic unit input at d = 128: the first coordinate over 4000 draws of
    # both rounds' signs is consistent with the uniform rotation's
    # coordinate law (Lemma 1 density, Kolmogorov-Smirnov at the 1% level)
    from scipy import stats
    from oracle import codebook as cb
    d = 128
    rg = np.random.default_rng(7)
    u = rg.standard_normal(d)
    u /= np.linalg.norm(u)
    ys = []
    for i in range(4000):
        eps = np.stack([sign_vector(d, 1000 + i), sign_vector(d, 9000 + i)])
        ys.append(tr.HadamardRotation(eps, d).forward(u[None, :])[0, 0])
    grid = np.linspace(-1, 1, 20001)
    cdf = np.cumsum(cb.pdf(grid, d)) * (grid[1] - grid[0])
    cdf /= cdf[-1]
    p = stats.kstest(ys, lambda x: np.interp(x, grid, cdf)).pvalue
    assert p > 0.01, p
