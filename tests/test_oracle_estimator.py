"""Pins for oracle.estimator: unbiasedness, shrinkage, QJL identity, invariants."""
import numpy as np
import pytest
from scipy import integrate

from oracle import codebook as cb
from oracle import estimator as est
from oracle import quantizer as qz
from oracle import transforms as tr
from tests.conftest import mean_se
from tq_inputs import gaussian_matrix, haar_orthogonal, sign_vector


def _pair(d, cos, seed=0):
    rg = np.random.default_rng(seed)
    x = rg.standard_normal(d)
    x /= np.linalg.norm(x)
    w = rg.standard_normal(d)
    w -= (w @ x) * x
    w /= np.linalg.norm(w)
    q = cos * x + np.sqrt(1 - cos ** 2) * w
    return x, q


def test_half_gaussian_identity_by_quadrature():
    # E[(s.y) sign(s.x)] = sqrt(2/pi) <x,y>/||x||  (explainer page section 8),
    # checked by integrating over the joint Gaussian of (s.x, s.y)
    nx, ny, rho = 1.7, 0.6, 0.35
    cov = rho * nx * ny

    def integrand(b, a):
        # density of (a, b) ~ N(0, [[nx^2, cov], [cov, ny^2]])
        det = nx ** 2 * ny ** 2 - cov ** 2
        qf = (ny ** 2 * a * a - 2 * cov * a * b + nx ** 2 * b * b) / det
        return b * np.sign(a) * np.exp(-0.5 * qf) / (2 * np.pi * np.sqrt(det))
    val, _ = integrate.dblquad(integrand, -12 * nx, 12 * nx, -12 * ny, 12 * ny, epsabs=1e-11)
    assert abs(val - np.sqrt(2 / np.pi) * cov / nx) < 1e-7


def test_qjl_unbiased_with_variance_bound():
    d, m = 16, 16
    x, q = _pair(d, 0.6)
    x = 2.5 * x
    ests = []
    for seed in range(20000):
        s = gaussian_matrix(m, d, seed)
        z = (s.astype(np.float64) @ x) >= 0
        ests.append(est.qjl_scores(q[None, :], z[None, :], np.array([np.linalg.norm(x)]), s)[0, 0])
    mu, se = mean_se(ests)
    assert abs(mu - q @ x) < 3 * se
    assert np.var(ests) <= np.pi / (2 * m) * (x @ x) * (q @ q) * 1.05


def test_qjl_unbiased_with_half_as_many_rows():
    # m = d / 2 projection rows (the first page's proj_dim = head_dim // 2):
    # the constant is sqrt(pi/2) / m, not / d (explainer page section 8,
    # Lemma 4).  A constant over d would centre the estimates on (m/d) <q, x>,
    # half the truth, about a hundred standard errors away.
    d, m = 16, 8
    x, q = _pair(d, 0.6, seed=21)
    x = 2.5 * x
    ests = []
    for seed in range(20000):
        s = gaussian_matrix(m, d, seed)
        z = (s.astype(np.float64) @ x) >= 0
        ests.append(est.qjl_scores(q[None, :], z[None, :], np.array([np.linalg.norm(x)]), s)[0, 0])
    mu, se = mean_se(ests)
    assert abs(mu - q @ x) < 3 * se
    assert abs(mu - (m / d) * (q @ x)) > 30 * se
    # the variance bound pi / (2 m) ||x||^2 ||q||^2 holds with m rows, and the
    # variance is larger than with m = d rows (fewer rows average less)
    var = np.var(ests)
    assert var <= np.pi / (2 * m) * (x @ x) * (q @ q) * 1.05
    assert var > np.pi / (2 * d) * (x @ x) * (q @ q)


@pytest.mark.parametrize("bits", [2, 3])
def test_prod_unbiased_with_half_as_many_rows(bits):
    # prod with an m x d QJL matrix, m = d / 2: still unbiased over (Pi, S),
    # and within the QJL variance bound applied to the residual,
    # Var <= pi / (2 m) n^2 E||r||^2 ||q||^2
    d, m = 32, 16
    c, b = cb.lloyd_max(d, bits - 1)
    x, q = _pair(d, 0.5, seed=30 + bits)
    x = 3.0 * x
    ests, r2 = [], []
    for seed in range(10000):
        rot = tr.DenseRotation(haar_orthogonal(d, seed))
        s = gaussian_matrix(m, d, seed)
        code = qz.encode_prod(x[None, :], rot, s, c, b, storage=False)
        assert code.z.shape == (1, m)
        ests.append(est.prod_scores(q[None, :], code.idx, code.z, code.n, code.gamma, rot, s, c)[0, 0])
        r2.append(code.gamma[0] ** 2)
    mu, se = mean_se(ests)
    assert abs(mu - q @ x) < 3 * se
    assert np.var(ests) <= np.pi / (2 * m) * 9.0 * np.mean(r2) * (q @ q) * 1.05


@pytest.mark.parametrize("bits", [2, 3])
def test_prod_estimator_unbiased_over_rotations(bits):
    # E over (Pi, S) of the prod estimate equals <q, x> (blog notes eq. (3))
    d = 32
    c, b = cb.lloyd_max(d, bits - 1)
    x, q = _pair(d, 0.5, seed=bits)
    x = 3.0 * x
    ests = []
    for seed in range(10000):
        rot = tr.DenseRotation(haar_orthogonal(d, seed))
        s = gaussian_matrix(d, d, seed)
        code = qz.encode_prod(x[None, :], rot, s, c, b, storage=False)
        ests.append(est.prod_scores(q[None, :], code.idx, code.z, code.n, code.gamma, rot, s, c)[0, 0])
    mu, se = mean_se(ests)
    assert abs(mu - q @ x) < 3 * se
    # and the MSE-only estimate is measurably shrunk by lambda = 1 - d D(b-1)
    assert se < 0.02


def test_prod_unbiased_over_projection_for_hadamard():
    # unbiased over S alone for a fixed rotation, so it holds for the Hadamard mode too
    d, bits = 24, 3
    dr = 32
    c, b = cb.lloyd_max(dr, bits - 1)
    x, q = _pair(d, -0.4, seed=5)
    rot = tr.HadamardRotation(sign_vector(dr, 9), d)
    ests = []
    for seed in range(10000):
        s = gaussian_matrix(dr, dr, seed)
        code = qz.encode_prod(x[None, :], rot, s, c, b, storage=False)
        ests.append(est.prod_scores(q[None, :], code.idx, code.z, code.n, code.gamma, rot, s, c)[0, 0])
    mu, se = mean_se(ests)
    assert abs(mu - q @ x) < 3 * se


@pytest.mark.parametrize("bits", [1, 2])
def test_mse_inner_product_shrinks_by_lambda(bits):
    # E over Pi of <q, x~_mse> = (1 - d D(b)) <q, x>  (explainer page section 7)
    d = 32
    c, b = cb.lloyd_max(d, bits)
    lam = 1 - d * cb.distortion(d, c, b)
    x, q = _pair(d, 0.8, seed=11)
    ests = []
    for seed in range(8000):
        rot = tr.DenseRotation(haar_orthogonal(d, seed))
        code = qz.encode_mse(x[None, :], rot, c, b, storage=False)
        ests.append(est.mse_scores(q[None, :], code.idx, code.n, rot, c)[0, 0])
    mu, se = mean_se(ests)
    assert abs(mu - lam * (q @ x)) < 3 * se
    assert abs(mu - q @ x) > 3 * se            # biased: the QJL stage is needed


def test_softmax_weighted_sum_invariants():
    rg = np.random.default_rng(0)
    s = rg.standard_normal((3, 9))
    v = rg.standard_normal((9, 5))
    o = est.softmax_weighted_sum(s, v, 0.7)
    # shift invariance per row
    assert np.allclose(est.softmax_weighted_sum(s + 5.0, v, 0.7), o)
    # scale 0 -> plain mean
    assert np.allclose(est.softmax_weighted_sum(s, v, 0.0), v.mean(0)[None, :].repeat(3, 0))
    # equal values -> that value
    vv = np.tile(v[:1], (9, 1))
    assert np.allclose(est.softmax_weighted_sum(s, vv, 0.7), vv[:3])
    # one dominant score -> its value
    s2 = s.copy()
    s2[:, 4] = 1e4
    assert np.allclose(est.softmax_weighted_sum(s2, v, 1.0), v[4][None, :].repeat(3, 0))
    # convex combination: within the per-coordinate hull
    assert np.all(o <= v.max(0) + 1e-12) and np.all(o >= v.min(0) - 1e-12)
    # the temperature multiplies the scores
    assert np.allclose(est.softmax_weighted_sum(s, v, 2.0), est.softmax_weighted_sum(2 * s, v, 1.0))
    # empty segment -> zeros
    assert np.array_equal(est.softmax_weighted_sum(np.zeros((2, 0)), np.zeros((0, 5)), 1.0), np.zeros((2, 5)))


def test_attend_single_token_returns_dequantized_value():
    d = 32
    ck, bk = cb.lloyd_max(d, 2)
    cv, bv = cb.lloyd_max(d, 3)
    rk = tr.DenseRotation(haar_orthogonal(d, 1))
    rv = tr.DenseRotation(haar_orthogonal(d, 2, 4))
    s = gaussian_matrix(d, d, 1)
    rg = np.random.default_rng(3)
    x, v, q = rg.standard_normal((3, 1, d))
    kc = qz.encode_prod(x, rk, s, ck, bk)
    vc = qz.encode_mse(v, rv, cv, bv)
    out = est.attend(q, (kc.idx, kc.z, kc.n, kc.gamma), (vc.idx, vc.n), rk, s, ck, rv, cv, 0.3)
    assert np.allclose(out, est.dequantize(vc.idx, vc.n, rv, cv))
    # and the dequantized value is close to v (MSE at 3 bits)
    assert np.sum((out - v) ** 2) / np.sum(v ** 2) < 0.2


def test_topk_ties_to_lower_index():
    s = np.array([[0.5, 2.0, 2.0, -1.0, 2.0, 0.7]])
    idx, val = est.topk(s, 4)
    expect = sorted(range(6), key=lambda i: (-s[0, i], i))[:4]
    assert idx[0].tolist() == expect == [1, 2, 4, 5]
    assert val[0].tolist() == [2.0, 2.0, 2.0, 0.7]
