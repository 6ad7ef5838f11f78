"""Pins for oracle.codebook: printed values, closed forms, invariants, brute force."""
import numpy as np
import pytest
from scipy import integrate, stats

from oracle import codebook as cb
from tests.conftest import read_golden


def test_gaussian_codebook_matches_printed_values():
    # explainer page: +-0.798 at 1 bit, +-0.453 / +-1.510 at 2 bits
    for row in read_golden("gaussian_codebook.txt"):
        bits = int(row[0])
        printed = np.array([float(v) for v in row[1:]])
        c, b = cb.lloyd_max(0, bits)
        assert np.allclose(c[len(c) // 2:], printed, atol=5e-4)
        assert np.allclose(c, -c[::-1], atol=0)


def test_one_bit_gaussian_is_half_normal_mean():
    c, b = cb.lloyd_max(0, 1)
    assert abs(c[1] - np.sqrt(2 / np.pi)) < 1e-12
    assert b.tolist() == [0.0]


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_d3_is_uniform_closed_form(bits):
    # d = 3: the coordinate is uniform on [-1, 1] (explainer page section 4);
    # Lloyd-Max for a uniform law is the uniform grid of cell midpoints, and the
    # unit-vector MSE 3 * w^2/12 equals 4^-b exactly (the Shannon lower bound).
    c, b = cb.lloyd_max(3, bits)
    K = 2 ** bits
    expect = -1 + (2 * np.arange(K) + 1) / K
    assert np.allclose(c, expect, atol=1e-10)
    assert np.allclose(b, expect[:-1] + 1.0 / K, atol=1e-10)
    assert abs(3 * cb.distortion(3, c, b) - 4.0 ** -bits) < 1e-9


def test_d2_one_bit_is_arcsine_mean():
    # d = 2: arcsine law 1/(pi sqrt(1 - x^2)); E[|X|] = 2/pi
    c, _ = cb.lloyd_max(2, 1)
    assert abs(c[1] - 2 / np.pi) < 1e-10


@pytest.mark.parametrize("d", [2, 3, 4, 8, 33, 128, 1000])
def test_density_normalised_with_variance_one_over_d(d):
    f = lambda x: float(cb.pdf(np.array([x]), d)[0])
    mass, _ = integrate.quad(f, -1, 1, limit=400, points=[0.0])
    var, _ = integrate.quad(lambda x: x * x * f(x), -1, 1, limit=400, points=[0.0])
    assert abs(mass - 1) < 1e-8
    assert abs(var - 1.0 / d) < 1e-9


def test_concentration_printed_values():
    for d, sd in read_golden("concentration.txt"):
        d = int(d)
        f = lambda x: float(cb.pdf(np.array([x]), d)[0])
        var, _ = integrate.quad(lambda x: x * x * f(x), -1, 1, limit=400, points=[0.0])
        assert abs(np.sqrt(var) - float(sd)) < 6e-4


def test_closed_form_moment_matches_quadrature():
    for d in (5, 128):
        a, b = 0.01, 0.2
        f = lambda x: x * float(cb.pdf(np.array([x]), d)[0])
        q, _ = integrate.quad(f, a, b, epsabs=1e-15)
        assert abs(cb.cell_first_moment(a, b, d) - q) < 1e-12
        m, _ = integrate.quad(lambda x: float(cb.pdf(np.array([x]), d)[0]), a, b, epsabs=1e-15)
        assert abs(cb.cell_mass(a, b, d) - m) < 1e-12


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_converges_to_gaussian_codebook(bits):
    # sqrt(d) * c_d -> N(0,1) codebook (Lemma 1's Gaussian limit)
    g, _ = cb.lloyd_max(0, bits)
    errs = []
    for d in (128, 2048):
        c, _ = cb.lloyd_max(d, bits)
        errs.append(np.max(np.abs(np.sqrt(d) * c - g)))
    assert errs[1] < errs[0]
    assert errs[1] < 3e-3


@pytest.mark.parametrize("bits", [1, 2])
def test_brute_force_grid_at_d8(bits):
    # The Lloyd-Max point minimises the distortion among symmetric codebooks:
    # search a fine grid of symmetric codebooks (1 free parameter at 1 bit, 2 at
    # 2 bits), scoring each by quadrature with midpoint boundaries.
    d = 8
    c_lm, b_lm = cb.lloyd_max(d, bits)
    best = cb.distortion(d, c_lm, b_lm)
    sd = 1 / np.sqrt(d)
    if bits == 1:
        for t in np.linspace(0.5, 1.2, 29) * sd:
            c = np.array([-t, t])
            assert cb.distortion(d, c, np.array([0.0])) >= best - 1e-12
    else:
        for t1 in np.linspace(0.3, 0.6, 7) * sd:
            for t2 in np.linspace(1.2, 1.7, 7) * sd:
                c = np.array([-t2, -t1, t1, t2])
                b = np.array([-(t1 + t2) / 2, 0.0, (t1 + t2) / 2])
                assert cb.distortion(d, c, b) >= best - 1e-12


def test_distortion_sandwich_and_rate():
    rows = {r[0]: float(r[1]) for r in read_golden("distortion_bounds.txt")}
    ds = []
    for bits in (1, 2, 3, 4):
        c, b = cb.lloyd_max(0, bits)
        D = cb.distortion(0, c, b)        # per coordinate in N(0,1) units = unit-vector MSE limit
        ds.append(D)
        assert D >= rows["lower_constant"] * 4.0 ** -bits
        assert D <= rows["upper_constant"] * 4.0 ** -bits
    assert abs(ds[0] / 4.0 ** -1 - rows["ratio_b1"]) < 0.01
    ratios = np.array(ds[:-1]) / np.array(ds[1:])
    assert np.all((ratios > 3.0) & (ratios < 4.2))   # "each extra bit cuts the MSE about 4x"


def test_shrinkage_factors_printed():
    for bits, lam in read_golden("shrinkage.txt"):
        bits = int(bits)
        c, b = cb.lloyd_max(0, bits)
        D = cb.distortion(0, c, b)
        ndig = len(lam.split(".")[1])
        # the page prints approximate values ("about"); 0.998 at b=5 is 0.99750
        assert abs((1 - D) - float(lam)) <= 0.6 * 10.0 ** -ndig
    c, b = cb.lloyd_max(0, 1)
    assert abs((1 - cb.distortion(0, c, b)) - 2 / np.pi) < 1e-10


@pytest.mark.parametrize("d", [2, 3, 8, 128])
def test_rotated_coordinate_follows_lemma1(d):
    # coordinates of a Haar-rotated e1 follow Lemma 1 (KS test); pins the
    # CDF used by the codebook and the Haar generator
    from tq_inputs import haar_orthogonal
    samples = np.array([haar_orthogonal(d, seed, 2)[0, 0] for seed in range(4000)], np.float64)

    def cdf(t):
        t = np.asarray(t, np.float64)
        up = cb._mass_upper(np.abs(t), d)
        return np.where(t >= 0, 1 - up, up)
    p = stats.kstest(samples, cdf).pvalue
    assert p > 1e-3


def test_monte_carlo_mse_matches_codebook():
    # unit vectors uniform on the sphere, coordinates quantized with the d=128
    # codebook: empirical MSE vs the analytic distortion, within 3 SE
    d, bits = 128, 2
    c, b = cb.lloyd_max(d, bits)
    rg = np.random.default_rng(123)
    u = rg.standard_normal((20000, d))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    err = ((u - c[np.searchsorted(b, u, side="right")]) ** 2).sum(axis=1)
    m, se = err.mean(), err.std(ddof=1) / np.sqrt(len(err))
    assert abs(m - d * cb.distortion(d, c, b)) < 3 * se
