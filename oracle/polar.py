"""PolarQuant as stage 1: the recursive polar transform of a rotated unit
vector and Lloyd-Max quantization of its angles, float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources.  The FastVQ README, "PolarQuant Algorithm": a random rotation, a
polar transform, Lloyd-Max quantization of the angles, and storage of the
norm with the angle indices and no per-block scales.  Its "Implementation
Notes" say the package uses a pairwise transform in place of the paper's full
recursive one; this module implements the recursive one.  Its "TurboQuant
Combination": normalise, PolarQuant, the residual against the dequantized
vector, QJL signs of the residual, and the record (||x||, polar codes, QJL
bits).

Readings (the pages leave these steps open; the plainest form the rest
supports):

* Transform, for d = 2^L and y the rotated unit vector.  Level 1 pairs the
  coordinates (y_{2j}, y_{2j+1}) (0-based): angle psi = atan2(y_{2j+1}, y_{2j})
  in (-pi, pi], radius the pair's length.  Level l >= 2 pairs the radii of
  level l-1 the same way: psi = atan2(rho_{2j+1}, rho_{2j}) in [0, pi/2].
  Level L leaves one radius, ||y|| = 1, so the only stored radius is n = ||x||
  (float16, as for the other records).  d - 1 angles in all.
* Angle laws after a uniform rotation (y uniform on the sphere; the angles
  are those of a standard Gaussian vector, since they do not depend on its
  length): level 1 uniform on (-pi, pi]; at level l >= 2 the two children are
  lengths of independent Gaussian blocks of 2^(l-1) coordinates, so
  sin^2 psi ~ Beta(a, a) with a = 2^(l-2), i.e. the density
      f_l(psi) = sin^(2a-1)(2 psi) / (2^(2a-2) B(a, a))   on [0, pi/2];
  all angles are independent.
* Codebooks: Lloyd-Max (explainer page section 5: midpoint boundaries,
  conditional-mean centroids) per level on that level's law.  Level 1's law is
  uniform, whose Lloyd-Max quantizer is the uniform grid: K1 = 2^b1 cells of
  width 2 pi / K1 from -pi, centroids at the cell middles.  Levels >= 2 use
  one width b; level 1 its own width b1.  A code is the number of boundaries
  at or below the angle (ties to the upper cell), as for the coordinates.
* Reconstruction: the unit top radius is split level by level with the
  centroid angles (rho cos, rho sin), so the reconstruction y~ has norm 1
  exactly whatever the codes are; x~ = n Pi^T y~.
* Stage 2 (optional, the FastVQ combination): residual r = y - y~ in the
  rotated domain, gamma = ||r|| stored as for TurboQuant-prod keys (the page's
  record lists ||x|| and the two code sets; the estimator of the prod keys
  needs ||r|| as well), z = [S r >= 0], and the score estimate
      s(q, x) = n (<Pi q, y~> + gamma sqrt(pi/2)/m <S Pi q, 2 z - 1>).
* A zero vector has u = 0, so every angle is atan2(0, 0) = 0; it is stored
  with n = 0 and contributes nothing.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
from scipy import integrate, special

from .quantizer import normalise


def n_levels(d: int) -> int:
    L = int(d).bit_length() - 1
    if d < 2 or (1 << L) != d:
        raise ValueError("d must be a power of two >= 2")
    return L


def polar_transform(y):
    """Rows of y [N, 2^L] -> (angles, radius): angles[l-1] is [N, d / 2^l], radius [N]."""
    y = np.asarray(y, np.float64)
    L = n_levels(y.shape[1])
    angles = []
    rho = y
    for _ in range(L):
        a, b = rho[:, 0::2], rho[:, 1::2]
        angles.append(np.arctan2(b, a))
        rho = np.hypot(a, b)
    return angles, rho[:, 0]


def polar_inverse(angles, radius):
    """Inverse of polar_transform: split each radius down the levels."""
    rho = np.asarray(radius, np.float64)[:, None]
    for psi in reversed(angles):
        psi = np.asarray(psi, np.float64)
        out = np.empty((rho.shape[0], 2 * rho.shape[1]))
        out[:, 0::2] = rho * np.cos(psi)
        out[:, 1::2] = rho * np.sin(psi)
        rho = out
    return rho


def _shape(level: int) -> float:
    return float(2 ** (level - 2))


def angle_pdf(psi, level: int):
    """Density of a level's angle for a uniformly rotated vector."""
    psi = np.asarray(psi, np.float64)
    if level == 1:
        return np.where((psi > -np.pi) & (psi <= np.pi), 1.0 / (2 * np.pi), 0.0)
    a = _shape(level)
    inside = (psi >= 0) & (psi <= np.pi / 2)
    logc = -(2 * a - 2) * np.log(2.0) - special.betaln(a, a)
    s = np.clip(np.sin(2 * np.where(inside, psi, 0.0)), 0.0, None)
    return np.where(inside, np.exp(logc) * s ** (2 * a - 1), 0.0)


def angle_cdf(psi, level: int):
    """P(angle <= psi): uniform at level 1, I_{sin^2 psi}(a, a) above."""
    psi = np.asarray(psi, np.float64)
    if level == 1:
        return np.clip((psi + np.pi) / (2 * np.pi), 0.0, 1.0)
    a = _shape(level)
    t = np.clip(psi, 0.0, np.pi / 2)
    return special.betainc(a, a, np.sin(t) ** 2)


def uniform_codebook(bits: int):
    """Level 1: K uniform cells of (-pi, pi], centroids at their middles."""
    K = 2 ** bits
    w = 2 * np.pi / K
    c = -np.pi + (np.arange(K) + 0.5) * w
    b = -np.pi + np.arange(1, K) * w
    return c, b


def _cell_mean(lo, hi, level):
    mass = angle_cdf(hi, level) - angle_cdf(lo, level)
    if mass <= 0:
        return 0.5 * (lo + hi)
    mom, _ = integrate.quad(lambda t: t * angle_pdf(t, level), lo, hi, epsabs=0, epsrel=1e-13, limit=200)
    return mom / mass


def angle_codebook(level: int, bits: int, tol: float = 1e-13, max_iter: int = 100000):
    """Lloyd-Max codebook (centroids [2^bits], boundaries [2^bits - 1]) of a level's angle."""
    if level == 1:
        return uniform_codebook(bits)
    K = 2 ** bits
    a = _shape(level)
    sd = 0.5 / np.sqrt(2 * a + 1)          # sd of psi near pi/4 (sin^2 psi has variance 1/(4(2a+1)))
    lo_edge, hi_edge = 0.0, np.pi / 2
    c = np.pi / 4 + np.clip(np.linspace(-2.0, 2.0, K) * sd, -np.pi / 4 + 1e-9, np.pi / 4 - 1e-9)
    for _ in range(max_iter):
        b = 0.5 * (c[:-1] + c[1:])
        edges = np.concatenate([[lo_edge], b, [hi_edge]])
        cn = np.array([_cell_mean(edges[i], edges[i + 1], level) for i in range(K)])
        move = np.max(np.abs(cn - c))
        c = cn
        if move < tol:
            break
    return c, 0.5 * (c[:-1] + c[1:])


def level_codebooks(d: int, bits1: int, bits: int):
    """[(centroids, boundaries)] for levels 1 .. L (level 1 uniform at bits1)."""
    L = n_levels(d)
    return [uniform_codebook(bits1)] + [angle_codebook(l, bits) for l in range(2, L + 1)]


@dataclass
class PolarCode:
    codes: list          # codes[l-1]: [N, d / 2^l] int64 angle cells of level l
    n: np.ndarray        # [N] ||x|| (float16 values as float64 in storage mode)
    y: np.ndarray        # [N, d] rotated unit vectors (diagnostic)
    angles: list         # the exact angles (diagnostic)
    y_hat: np.ndarray    # [N, d] reconstruction on the unit sphere
    z: np.ndarray = None       # [N, m] QJL bits (stage 2 only)
    gamma: np.ndarray = None   # [N] ||y - y_hat|| (stage 2 only)
    proj: np.ndarray = None    # [N, m] S r (diagnostic)


def _store(v, storage):
    return v.astype(np.float16).astype(np.float64) if storage else v


def reconstruct(codes, codebooks):
    """y~ on the unit sphere from the cells of every level (centroid angles)."""
    angles = [np.asarray(cb[0], np.float64)[np.asarray(c)] for c, cb in zip(codes, codebooks)]
    n = np.asarray(codes[0]).shape[0]
    return polar_inverse(angles, np.ones(n))


def encode_polar(x, rot, codebooks, s_matrix=None, storage: bool = True) -> PolarCode:
    """Normalise, rotate, transform, code every angle against its level's boundaries.

    ``codebooks`` as level_codebooks gives them (the caller may round them to
    float32 first: the decisions use whatever values it passes).  With
    ``s_matrix`` the QJL stage follows on the residual y - y~.
    """
    n, u = normalise(x)
    y = rot.forward(u)
    angles, _ = polar_transform(y)
    codes = [np.searchsorted(np.asarray(cb[1], np.float64), psi, side="right").astype(np.int64)
             for psi, cb in zip(angles, codebooks)]
    y_hat = reconstruct(codes, codebooks)
    out = PolarCode(codes=codes, n=_store(n, storage), y=y, angles=angles, y_hat=y_hat)
    if s_matrix is not None:
        r = y - y_hat
        out.gamma = _store(np.sqrt(np.sum(r * r, axis=1)), storage)
        out.proj = r @ np.asarray(s_matrix, np.float64).T
        out.z = out.proj >= 0
    return out


def decode_polar(code: PolarCode, rot):
    """x~ = n Pi^T y~ (rows)."""
    return np.asarray(code.n)[:, None] * rot.inverse(code.y_hat)


def polar_scores(q, code: PolarCode, rot, s_matrix=None):
    """Estimated <q_h, x_t> for query rows q [H, d] -> [H, T] (see the module docstring)."""
    q_rot = rot.forward(np.asarray(q, np.float64))
    est = q_rot @ code.y_hat.T
    if s_matrix is not None:
        s = np.asarray(s_matrix, np.float64)
        m = s.shape[0]
        est = est + np.sqrt(np.pi / 2) / m * np.asarray(code.gamma)[None, :] * (
            (q_rot @ s.T) @ (2.0 * np.asarray(code.z, np.float64) - 1.0).T)
    return np.asarray(code.n)[None, :] * est
