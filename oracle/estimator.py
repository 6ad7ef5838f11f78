"""Decoders: the asymmetric inner-product estimator, dequantization, attention.

* QJL decoder (explainer page section 8): with the query y kept in full
  precision, <S y, sign(S x)> scaled by sqrt(pi/2)/m and by ||x|| estimates
  <x, y> without bias (Lemma 4), with variance at most pi/(2m) ||x||^2 ||y||^2.
* TurboQuant-prod estimator (blog notes, the estimator after Q_prod's
  definition, read with the stored L2 norm ||r||_2; explainer page section 8):
  <y, x> ~= <y, x~_mse> + ||r|| * <y, Q_qjl^-1(Q_qjl(r))>.
  With the residual in the rotated domain, y enters as Pi y, and a record's
  stored norm n rescales the estimate of a non-unit x:

    s(q, t) = n_t * ( <Pi q, c[idx_t]> + gamma_t * sqrt(pi/2)/m * <S Pi q, 2 z_t - 1> ).

* MSE dequantization (blog notes, Q_mse^-1): x~ = n * Pi^T c[idx].
* Attention over a compressed cache (first page, pattern 1): scores from the
  compressed keys, softmax over the tokens, weighted sum of the dequantized
  values; a softmax temperature ``scale`` multiplies the scores first.
"""
from __future__ import annotations

import numpy as np


def kappa(m: int) -> float:
    return float(np.sqrt(np.pi / 2.0) / m)


def prepare_query(q, rot, s_matrix):
    """(Pi q, S Pi q) for rows of q."""
    q_rot = rot.forward(np.asarray(q, np.float64))
    q_proj = q_rot @ np.asarray(s_matrix, np.float64).T
    return q_rot, q_proj


def prod_scores(q, idx, z, n, gamma, rot, s_matrix, centroids):
    """Estimated <q_h, x_t> for query rows q [H, d] against T encoded keys -> [H, T]."""
    q_rot, q_proj = prepare_query(q, rot, s_matrix)
    m = np.asarray(s_matrix).shape[0]
    if idx.shape[1]:
        mse_part = q_rot @ np.asarray(centroids, np.float64)[idx].T
    else:
        mse_part = np.zeros((q_rot.shape[0], idx.shape[0]))
    qjl_part = q_proj @ (2.0 * np.asarray(z, np.float64) - 1.0).T
    return np.asarray(n)[None, :] * (mse_part + np.asarray(gamma)[None, :] * kappa(m) * qjl_part)


def mse_scores(q, idx, n, rot, centroids):
    """<q, x~_mse>: the (biased) inner product with the MSE reconstruction."""
    q_rot = rot.forward(np.asarray(q, np.float64))
    return np.asarray(n)[None, :] * (q_rot @ np.asarray(centroids, np.float64)[idx].T)


def qjl_scores(q, z, norm_x, s_matrix):
    """Pure QJL estimate of <q, x> from z = [S x >= 0] and ||x|| (no rotation)."""
    m = np.asarray(s_matrix).shape[0]
    q_proj = np.asarray(q, np.float64) @ np.asarray(s_matrix, np.float64).T
    return kappa(m) * np.asarray(norm_x)[None, :] * (q_proj @ (2.0 * np.asarray(z, np.float64) - 1.0).T)


def dequantize(idx, n, rot, centroids):
    """x~ = n * Pi^T c[idx] (rows)."""
    return np.asarray(n)[:, None] * rot.inverse(np.asarray(centroids, np.float64)[idx])


def softmax_weighted_sum(scores, values, scale: float):
    """o_h = sum_t softmax_t(scale * s_h)_t v_t for scores [H, T], values [T, d].

    With T == 0 the output is zero.
    """
    scores = np.asarray(scores, np.float64)
    values = np.asarray(values, np.float64)
    if scores.shape[1] == 0:
        return np.zeros((scores.shape[0], values.shape[1]))
    a = scale * scores
    a = a - a.max(axis=1, keepdims=True)
    w = np.exp(a)
    w /= w.sum(axis=1, keepdims=True)
    return w @ values


def attend(q, key_code, val_code, rot_k, s_matrix, cent_k, rot_v, cent_v, scale: float):
    """Softmax attention of queries q [H, d] over one compressed segment.

    key_code = (idx, z, n, gamma); val_code = (idx, n).
    """
    kidx, z, kn, kg = key_code
    vidx, vn = val_code
    s = prod_scores(q, kidx, z, kn, kg, rot_k, s_matrix, cent_k)
    v = dequantize(vidx, vn, rot_v, cent_v)
    return softmax_weighted_sum(s, v, scale)


def topk(scores, k: int):
    """Per row, the k largest scores; equal scores go to the lower index.

    Returns (indices [H, k] int64, values [H, k])."""
    scores = np.asarray(scores, np.float64)
    order = np.lexsort((np.broadcast_to(np.arange(scores.shape[1]), scores.shape), -scores), axis=1)
    idx = order[:, :k]
    return idx, np.take_along_axis(scores, idx, axis=1)
