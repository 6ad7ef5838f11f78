"""Plain CPU oracle of the TurboQuant encode / score / attend path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the tests, the smoke check's comparison and the
bench's CPU-baseline leg use it.  It shares no code with the HIP library.

Everything is written for clarity, in float64, with NumPy/SciPy primitives,
following the method as the pages state it (citations name the page title and
its section or equation):

* ``codebook``   -- Lloyd-Max scalar quantizer for the coordinate density of a
  uniformly rotated unit vector (blog notes on the ICLR 2026 paper, Lemma 1 and
  eq. (4); explainer page sections 4-5).
* ``transforms`` -- the random rotation Pi (dense) and the sign-flipped
  Sylvester Hadamard transform (explainer page sections 0.9 and 3).
* ``quantizer``  -- TurboQuant-MSE and TurboQuant-prod encoders (blog notes,
  Q_mse and Q_prod definitions; explainer page sections 6 and 8).
* ``packing``    -- the bit-plane record layout both sides agree on.
* ``estimator``  -- the asymmetric inner-product estimator, MSE dequantization,
  softmax attention over the compressed cache and top-k retrieval.
* ``polar``      -- PolarQuant as stage 1: the recursive polar transform of
  the rotated vector, Lloyd-Max codebooks of each level's angle law, the
  reconstruction and the score estimate with the optional QJL stage (FastVQ
  README, "PolarQuant Algorithm" and "TurboQuant Combination").
* ``quality``    -- attention-fidelity and needle statistics of an estimated
  score matrix against the exact one (the first page's usage patterns).

Parity pins: every function is pinned in ``tests/test_oracle_*.py`` to values
the pages print, closed forms, invariants or brute force.  Functions without
such a pin say "parity unpinned" in their docstring.
"""
from . import codebook, transforms, quantizer, packing, estimator, quality, polar  # noqa: F401
