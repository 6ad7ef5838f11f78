"""Pins for oracle.quality (attention-fidelity and needle statistics of the
"turboquant-pytorch" page's usage patterns): closed forms, an independent
expression of the cosine, and invariants."""
import numpy as np

from oracle import quality as ql


def test_two_key_closed_form():
    # exact scores equal -> softmax (1/2, 1/2); estimate (a, 0) at temperature t
    # gives (p, 1 - p), p = 1 / (1 + e^(-t a)).  cos = 1 / (sqrt(2) sqrt(p^2 + (1-p)^2)).
    # With t = 1/2 and a = 2 ln 3: p = 3/4, cos = 2 / sqrt(5).
    cos, top1 = ql.attention_fidelity(np.array([[0.0, 0.0]]), np.array([[2 * np.log(3.0), 0.0]]), scale=0.5)
    assert abs(cos[0] - 2 / np.sqrt(5)) < 1e-14
    assert top1[0]          # both argmax are key 0 (the tie goes to the lower index)


def test_cosine_matches_an_expression_without_softmax_normalisation():
    # p = softmax(t s), p^ = softmax(t (s + e)); the normalisers cancel in the
    # cosine, so cos = E_pi[w] / sqrt(E_pi[w^2]) with w = exp(t e) and
    # pi proportional to p^2 (i.e. to exp(2 t s)).
    rg = np.random.default_rng(3)
    s = rg.standard_normal((6, 50))
    e = 0.3 * rg.standard_normal((6, 50))
    t = 0.7
    cos, _ = ql.attention_fidelity(s, s + e, scale=t)
    pi = np.exp(2 * t * (s - s.max(axis=1, keepdims=True)))
    pi /= pi.sum(axis=1, keepdims=True)
    w = np.exp(t * e)
    ref = (pi * w).sum(1) / np.sqrt((pi * w * w).sum(1))
    np.testing.assert_allclose(cos, ref, rtol=1e-13)


def test_small_error_second_order():
    # 1 - cos ~= Var_pi(t e) / 2 for small e (pi as above)
    rg = np.random.default_rng(4)
    s = rg.standard_normal((4, 200))
    e = 1e-3 * rg.standard_normal((4, 200))
    cos, _ = ql.attention_fidelity(s, s + e, scale=1.0)
    pi = np.exp(2 * s)
    pi /= pi.sum(axis=1, keepdims=True)
    var = (pi * e * e).sum(1) - (pi * e).sum(1) ** 2
    np.testing.assert_allclose(1 - cos, var / 2, rtol=2e-2)


def test_shift_invariance_and_identity():
    rg = np.random.default_rng(5)
    s = rg.standard_normal((5, 30))
    cos, top1 = ql.attention_fidelity(s, s + rg.standard_normal((5, 1)) * 10, scale=1.3)
    np.testing.assert_allclose(cos, 1.0, atol=1e-13)
    assert top1.all()


def test_top1_and_needle():
    true = np.array([[0.1, 0.9, 0.3], [0.5, 0.2, 0.5], [1.0, 2.0, 3.0]])
    est = np.array([[0.1, 0.8, 0.85], [0.5, 0.5, 0.1], [3.0, 2.0, 1.0]])
    _, top1 = ql.attention_fidelity(true, est)
    # row 0: 1 vs 2; row 1: ties -> 0 vs 0; row 2: 2 vs 0
    assert top1.tolist() == [False, True, False]
    assert ql.needle_found(true, est).tolist() == [False, True, False]
    assert ql.argmax_rows(np.array([[2.0, 2.0, 1.0]])).tolist() == [0]
