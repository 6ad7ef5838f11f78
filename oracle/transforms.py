"""Rotations: the dense random orthogonal Pi and the sign-flipped Hadamard.

Dense (explainer page section 3; blog notes, Q_mse): y = Pi u, and the inverse
is Pi^T (Pi orthogonal keeps lengths and inner products).

Hadamard (explainer page section 0.9: a randomised Hadamard transform may
replace the uniform rotation at O(d log d) cost; the FastVQ README's
"sign-flipped Hadamard" backend with block padding):
    y = H_{d'} (eps * pad(u)) / sqrt(d'),
with H_{d'} the Sylvester Hadamard matrix of order d' = 2^k >= d (natural
order, H[i, j] = (-1)^popcount(i & j)), eps in {+1, -1}^{d'} and pad() zero
padding at the end.  Since H H^T = d' I and H is symmetric, the inverse is
u = (eps * (H y) / sqrt(d'))[:d].

The oracle builds H explicitly and multiplies; it never uses a fast
transform.
"""
from __future__ import annotations

import numpy as np


def sylvester_hadamard(n: int) -> np.ndarray:
    """Sylvester-ordered Hadamard matrix of order n (a power of two), float64."""
    if n < 1 or (n & (n - 1)):
        raise ValueError("order must be a power of two")
    i = np.arange(n)
    parity = np.zeros((n, n), dtype=np.int64)
    x = i[:, None] & i[None, :]
    while np.any(x):
        parity ^= x & 1
        x = x >> 1
    return np.where(parity == 1, -1.0, 1.0)


class DenseRotation:
    """y = Pi u with Pi given (float32 values taken exactly)."""

    kind = "dense"

    def __init__(self, pi):
        self.pi = np.asarray(pi, dtype=np.float64)
        self.d = self.pi.shape[1]
        self.d_rot = self.pi.shape[0]

    def forward(self, u):
        """Rows of u are vectors: returns rows of Pi u."""
        return np.asarray(u, np.float64) @ self.pi.T

    def inverse(self, y):
        return np.asarray(y, np.float64) @ self.pi


class HadamardRotation:
    """y = H (eps * pad(u)) / sqrt(d_rot), or with several rounds

        y = (H D_R / sqrt(d_rot)) ... (H D_1 / sqrt(d_rot)) pad(u),   D_r = diag(eps[r]),

    the randomised Hadamard transform applied R times with independent sign
    vectors, round 1 first (explainer page section 0.9: the randomised
    Hadamard transform as a cheap stand-in for a uniform rotation; more rounds
    bring the coordinates of any input closer to the uniform rotation's law).
    ``eps`` is [d_rot] for one round or [R, d_rot]."""

    kind = "hadamard"

    def __init__(self, eps, d: int):
        eps = np.asarray(eps, dtype=np.float64)
        self.eps_rounds = eps[None, :] if eps.ndim == 1 else eps
        self.eps = self.eps_rounds[0]
        self.rounds = self.eps_rounds.shape[0]
        self.d_rot = self.eps_rounds.shape[1]
        self.d = d
        if d > self.d_rot:
            raise ValueError("d must not exceed the padded order")
        self.h = sylvester_hadamard(self.d_rot)

    def forward(self, u):
        u = np.asarray(u, np.float64)
        v = np.zeros((u.shape[0], self.d_rot))
        v[:, : self.d] = u
        for r in range(self.rounds):
            v = ((v * self.eps_rounds[r][None, :]) @ self.h.T) / np.sqrt(self.d_rot)
        return v

    def inverse(self, y):
        v = np.asarray(y, np.float64)
        for r in reversed(range(self.rounds)):
            v = (v @ self.h.T) / np.sqrt(self.d_rot) * self.eps_rounds[r][None, :]
        return v[:, : self.d]
