"""Lloyd-Max codebooks for the coordinates of a randomly rotated unit vector.

After a uniform random rotation, one coordinate X of a unit vector in R^d has
the density (blog notes on the ICLR 2026 TurboQuant paper, Lemma 1)

    f_X(x) = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) * (1 - x^2)^((d-3)/2),  x in [-1, 1],

which tends to N(0, 1/d) as d grows (same lemma; explainer page section 4).
The optimal b-bit scalar quantizer of that density is the one-dimensional
continuous k-means problem of eq. (4) of the blog notes, solved by the
Lloyd-Max iteration (explainer page section 5; the Russian summary's
conditional-mean step): boundaries are midpoints of adjacent centroids, each
centroid is the conditional mean of its cell.

``d == 0`` stands for the Gaussian limit N(0, 1) itself (the normalised
codebook the explainer page quotes: +-0.798 at one bit, +-0.453 / +-1.510 at
two bits, section 0.9 and section 5).
"""
from __future__ import annotations

import numpy as np
from scipy import special


def _k(d: int) -> float:
    return (d - 3) / 2.0


def density_constant(d: int) -> float:
    """Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)), the normaliser of Lemma 1."""
    return float(np.exp(special.gammaln(d / 2.0) - 0.5 * np.log(np.pi) - special.gammaln((d - 1) / 2.0)))


def pdf(x, d: int):
    """Lemma 1 density on [-1, 1] (d >= 2); the N(0,1) density for d == 0."""
    x = np.asarray(x, dtype=np.float64)
    if d == 0:
        return np.exp(-0.5 * x * x) / np.sqrt(2 * np.pi)
    out = np.zeros_like(x)
    inside = np.abs(x) < 1
    out[inside] = density_constant(d) * (1.0 - x[inside] ** 2) ** _k(d)
    return out


def _mass_upper(a, d: int):
    """P(X >= a) for a >= 0."""
    a = np.asarray(a, dtype=np.float64)
    if d == 0:
        return special.ndtr(-a)
    # P(|X| >= a) = 1 - I_{a^2}(1/2, (d-1)/2); half of it by symmetry
    return 0.5 * special.betaincc(0.5, (d - 1) / 2.0, np.minimum(a * a, 1.0))


def cell_mass(a, b, d: int):
    """P(a <= X < b) for 0 <= a <= b (upper half line; the density is even)."""
    return _mass_upper(a, d) - _mass_upper(b, d)


def cell_first_moment(a, b, d: int):
    """Integral of x f_X(x) over [a, b], in closed form.

    For Lemma 1: C_d [(1-a^2)^(k+1) - (1-b^2)^(k+1)] / (2(k+1)), k = (d-3)/2.
    For the Gaussian: phi(a) - phi(b).
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if d == 0:
        return (np.exp(-0.5 * a * a) - np.exp(-0.5 * b * b)) / np.sqrt(2 * np.pi)
    k1 = _k(d) + 1.0
    ta = np.clip(1.0 - a * a, 0.0, None) ** k1
    tb = np.clip(1.0 - b * b, 0.0, None) ** k1
    return density_constant(d) * (ta - tb) / (2.0 * k1)


def _sd(d: int) -> float:
    return 1.0 if d == 0 else 1.0 / np.sqrt(d)


def lloyd_max(d: int, bits: int, tol: float = 1e-12, max_iter: int = 200000):
    """Lloyd-Max codebook for Lemma 1's density (or N(0,1) if d == 0).

    Returns (centroids [2^bits] ascending, boundaries [2^bits - 1]), float64,
    in unit-sphere units (N(0,1) units when d == 0).  The codebook is exactly
    odd-symmetric: the density is even, the iteration starts symmetric, and the
    upper half is solved with the middle boundary held at 0 and mirrored.

    Iteration (explainer page section 5; blog notes eq. (4)):
      boundaries  beta_i = (c_i + c_{i+1}) / 2
      centroids   c_i = E[X | beta_{i-1} <= X < beta_i],  outer edges at +-1 (+-inf)
    starting from the Gaussian quantiles (i + 1/2)/2^bits scaled by the
    coordinate standard deviation, until the largest centroid move (in units
    of that standard deviation) is below ``tol``.  (In float64 the closed-form
    moments carry a noise floor near 1e-13 of the standard deviation at
    d = 2048, which sets the default tolerance.)
    """
    if bits < 1:
        raise ValueError("bits must be >= 1")
    if d != 0 and d < 2:
        raise ValueError("d must be >= 2 (or 0 for the Gaussian limit)")
    K = 2 ** bits
    half = K // 2
    sd = _sd(d)
    top = np.inf if d == 0 else 1.0
    # upper-half centroids, ascending
    p = (np.arange(half) + half + 0.5) / K
    c = special.ndtri(p) * sd
    if d != 0:
        c = np.minimum(c, 1.0 - 1e-12)
    for _ in range(max_iter):
        edges = np.concatenate([[0.0], 0.5 * (c[:-1] + c[1:]), [top]])
        mass = cell_mass(edges[:-1], edges[1:], d)
        mom = cell_first_moment(edges[:-1], edges[1:], d)
        c_new = mom / mass
        move = np.max(np.abs(c_new - c)) / sd
        c = c_new
        if move < tol:
            break
    centroids = np.concatenate([-c[::-1], c])
    upper_b = 0.5 * (c[:-1] + c[1:])
    boundaries = np.concatenate([-upper_b[::-1], [0.0], upper_b])
    return centroids, boundaries


def distortion(d: int, centroids, boundaries) -> float:
    """Per-coordinate mean squared error of the scalar quantizer, E[(X - Q(X))^2].

    Computed by adaptive quadrature of (x - c_i)^2 f_X(x) over each cell,
    without using the centroid condition, so it can check a codebook that is
    not the Lloyd-Max fixed point.  Multiply by d for the MSE of a unit vector
    (D_mse of eq. (1) of the blog notes).
    """
    from scipy import integrate
    lo = -np.inf if d == 0 else -1.0
    hi = np.inf if d == 0 else 1.0
    edges = np.concatenate([[lo], np.asarray(boundaries, np.float64), [hi]])
    total = 0.0
    sd = _sd(d)
    for i, ci in enumerate(np.asarray(centroids, np.float64)):
        a, b = edges[i], edges[i + 1]
        # keep quad away from an infinite interval where the integrand is ~0
        a = max(a, -40 * sd) if d == 0 else a
        b = min(b, 40 * sd) if d == 0 else b
        val, _ = integrate.quad(lambda x: (x - ci) ** 2 * float(pdf(np.array([x]), d)[0]), a, b,
                                limit=200, epsabs=1e-15, epsrel=1e-12,
                                points=[0.0] if a < 0 < b else None)
        total += val
    return total
