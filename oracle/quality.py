"""Quality statistics of an estimated score matrix against the exact one.

TEST INFRASTRUCTURE ONLY (like the rest of this package): the GPU harness
computes the same statistics on device from the library's outputs, and the
tests compare the two.

* Attention fidelity ("turboquant-pytorch" page, the attention-fidelity usage
  pattern): per query, the softmax distribution over the keys from the exact
  scores and the one from the estimated scores; the statistic is the cosine
  of the two distributions, and top-1 agreement is whether their argmax is
  the same key.  A softmax temperature ``scale`` multiplies both score rows
  (the page uses 1).
* Needle in a haystack (same page, the needle usage pattern): per trial,
  whether the argmax of the estimated scores is the argmax of the exact ones.
* Output fidelity: cosine between attention outputs (exact and from the
  compressed cache), per query head.

Ties in an argmax go to the lower key index.
"""
from __future__ import annotations

import numpy as np


def softmax_rows(scores, scale: float = 1.0):
    """softmax(scale * s) along the last axis, float64."""
    a = scale * np.asarray(scores, np.float64)
    a = a - a.max(axis=-1, keepdims=True)
    w = np.exp(a)
    return w / w.sum(axis=-1, keepdims=True)


def row_cosine(a, b):
    """Cosine of corresponding rows of a and b, float64."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return (a * b).sum(-1) / (np.linalg.norm(a, axis=-1) * np.linalg.norm(b, axis=-1))


def argmax_rows(scores):
    """Index of the largest entry of each row; the lowest index among equals."""
    return np.argmax(np.asarray(scores, np.float64), axis=-1)


def attention_fidelity(true_scores, est_scores, scale: float = 1.0):
    """(cosine [Q], top-1 agreement [Q] bool) of the two score matrices [Q, N]."""
    cos = row_cosine(softmax_rows(true_scores, scale), softmax_rows(est_scores, scale))
    top1 = argmax_rows(true_scores) == argmax_rows(est_scores)
    return cos, top1


def needle_found(true_scores, est_scores):
    """Per trial (rows [trials, N]): the estimated argmax is the exact argmax."""
    return argmax_rows(true_scores) == argmax_rows(est_scores)
