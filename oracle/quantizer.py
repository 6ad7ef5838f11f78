"""TurboQuant-MSE and TurboQuant-prod encoders, float64.

Notation follows the blog notes on the ICLR 2026 paper (Q_mse, Q_prod
definitions) and the explainer page (sections 6 and 8):

* normalise: the method assumes ||x|| = 1; otherwise the L2 norm is stored
  and the vector rescaled (blog notes, the assumption before Lemma 1).
  Here n = ||x||_2 and u = x / n (u = 0 when n = 0).
* Q_mse: y = Pi u, then every coordinate goes to the index of its cell,
  idx_j = #{k : beta_k <= y_j} (ties go to the upper cell).
* Q_prod with a b-bit budget: Q_mse at b-1 bits, the residual in the rotated
  domain r = y - c[idx] (explainer page section 8: r = Pi x - y~_mse), its
  norm gamma = ||r||_2 (the one stored side scale), and the QJL bits
  z_i = [(S r)_i >= 0] with S an iid N(0,1) matrix shared by encoder and
  decoder (explainer page section 8, the QJL encoder).  With b = 1 there is
  no MSE stage and r = y.

* EDEN's per-vector scale (explainer page, section 0.9, the prior-work map:
  EDEN stores S = ||x||^2 / <R x, Q(R x)> with its quantized rotated vector,
  which makes the reconstruction S R^T Q unbiased; DRIVE's one-bit scale
  ||x||^2 / ||R x||_1 is the same formula with Q = sign).  In this module's
  unit-sphere notation, with y = Pi u and codebook c, the reconstruction is
  S Pi^T c[idx] with S = n / <y, c[idx]> (0 for a zero vector).

Storage mode rounds n, gamma and S to float16 (round to nearest even), the
record format's precision; exact mode keeps them in float64.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class MseCode:
    idx: np.ndarray      # [N, d_rot] int64 cell indices
    n: np.ndarray        # [N] norms (float16 values as float64 in storage mode)
    y: np.ndarray        # [N, d_rot] rotated unit vectors (diagnostic)


@dataclass
class ProdCode:
    idx: np.ndarray      # [N, d_rot] int64 (b-1)-bit indices (empty columns if b == 1)
    z: np.ndarray        # [N, m] bool, True <=> (S r)_i >= 0
    n: np.ndarray        # [N] ||x||
    gamma: np.ndarray    # [N] ||r||
    y: np.ndarray        # [N, d_rot] rotated unit vectors (diagnostic)
    proj: np.ndarray     # [N, m] S r (diagnostic)


def _store(v: np.ndarray, storage: bool) -> np.ndarray:
    return v.astype(np.float16).astype(np.float64) if storage else v


def normalise(x):
    """n = ||x||_2 and u = x / n, with u = 0 for a zero vector."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=1))
    u = np.zeros_like(x)
    nz = n > 0
    u[nz] = x[nz] / n[nz, None]
    return n, u


def cell_index(y, boundaries):
    """idx_j = number of boundaries <= y_j (searchsorted, side='right')."""
    return np.searchsorted(np.asarray(boundaries, np.float64), y, side="right").astype(np.int64)


def encode_mse(x, rot, centroids, boundaries, storage: bool = True) -> MseCode:
    n, u = normalise(x)
    y = rot.forward(u)
    idx = cell_index(y, boundaries)
    return MseCode(idx=idx, n=_store(n, storage), y=y)


def encode_eden(x, rot, centroids, boundaries, storage: bool = True) -> MseCode:
    """Q_mse codes with EDEN's scale in place of the norm: n = S = ||x|| / <y, c[idx]>."""
    nrm, u = normalise(x)
    y = rot.forward(u)
    idx = cell_index(y, boundaries)
    yc = np.sum(y * np.asarray(centroids, np.float64)[idx], axis=1)
    scale = np.zeros_like(nrm)
    ok = (nrm > 0) & (yc > 0)
    scale[ok] = nrm[ok] / yc[ok]
    return MseCode(idx=idx, n=_store(scale, storage), y=y)


def encode_prod(x, rot, s_matrix, centroids, boundaries, storage: bool = True) -> ProdCode:
    """Q_prod: (b-1)-bit Q_mse, then QJL signs of the residual and its norm.

    ``centroids``/``boundaries`` are the (b-1)-bit codebook; pass ``None`` for
    b = 1 (pure QJL on y).
    """
    n, u = normalise(x)
    y = rot.forward(u)
    if centroids is None:
        idx = np.zeros((y.shape[0], 0), dtype=np.int64)
        r = y
    else:
        idx = cell_index(y, boundaries)
        r = y - np.asarray(centroids, np.float64)[idx]
    gamma = np.sqrt(np.sum(r * r, axis=1))
    proj = r @ np.asarray(s_matrix, np.float64).T
    z = proj >= 0
    return ProdCode(idx=idx, z=z, n=_store(n, storage), gamma=_store(gamma, storage), y=y, proj=proj)
