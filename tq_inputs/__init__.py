"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module only draws random numbers and shapes them into the workloads the
pages describe (KV caches of small decoder models, retrieval embeddings).  It
holds none of the quantizer's arithmetic: no norms, no codebooks, no
quantization, no packing.  The random objects the method itself draws (the
Haar rotation, the Gaussian projection, the Hadamard sign flips) are produced
here and passed to both the oracle and the library as plain inputs.

Seeding: every array comes from ``numpy.random.default_rng(SeedSequence([seed,
purpose]))`` so that each (seed, purpose) pair is an independent stream.
"""
from __future__ import annotations

import numpy as np

# purpose codes of the independent random streams
DATA = 0
OUTLIER_CHANNELS = 1
PI_K = 2
S_K = 3
PI_V = 4
EPS_K = 5
EPS_V = 6
QUERIES = 7
CHANNEL_SCALES = 8
MIXTURE_MEANS = 9
MIXTURE_LABELS = 10
DATA_V = 11
OUTLIER_CHANNELS_V = 12
CHANNEL_SCALES_V = 13
NEEDLE_POSITIONS = 14
NEEDLE_NOISE = 15
RANDOM_RECORDS = 16


def rng(seed: int, purpose: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(purpose)]))


def haar_orthogonal(d: int, seed: int, purpose: int = PI_K) -> np.ndarray:
    """A d x d orthogonal matrix drawn uniformly from O(d), returned as float32.

    Drawn as the Q factor of the QR factorisation of an iid N(0,1) matrix, with
    the columns' signs fixed by the signs of diag(R) so that the law is exactly
    Haar (turboquant explainer page, section 3: QR of a Gaussian matrix gives a
    uniform orthogonal matrix).  The float32 values are the definition every
    consumer uses.
    """
    g = rng(seed, purpose).standard_normal((d, d))
    q, r = np.linalg.qr(g)
    q = q * np.sign(np.diag(r))[None, :]
    return np.ascontiguousarray(q.astype(np.float32))


def gaussian_matrix(m: int, d: int, seed: int, purpose: int = S_K) -> np.ndarray:
    """An m x d matrix of iid N(0,1) entries (the QJL projection), float32."""
    return np.ascontiguousarray(rng(seed, purpose).standard_normal((m, d)).astype(np.float32))


def sign_vector(d: int, seed: int, purpose: int = EPS_K) -> np.ndarray:
    """d iid Rademacher signs (+1/-1) as float32 (randomised Hadamard flips)."""
    return np.where(rng(seed, purpose).integers(0, 2, size=d) == 1, 1.0, -1.0).astype(np.float32)


def gaussian_queries(n: int, d: int, seed: int, purpose: int = QUERIES) -> np.ndarray:
    return np.ascontiguousarray(rng(seed, purpose).standard_normal((n, d)).astype(np.float32))


def unit_gaussian(n: int, d: int, seed: int, purpose: int = DATA) -> np.ndarray:
    """n rows drawn from N(0, I_d) and scaled to unit length, float32 (random unit keys and queries)."""
    z = rng(seed, purpose).standard_normal((n, d))
    return np.ascontiguousarray((z / np.linalg.norm(z, axis=1, keepdims=True)).astype(np.float32))


def needle_haystacks(trials: int, seq_len: int, d: int, seed: int, noise: float = 0.1):
    """Needle-in-a-haystack trials: (haystacks [trials, seq_len, d], queries [trials, d], position [trials]).

    Each haystack is seq_len random unit vectors; each query is a random unit
    vector; at a seeded position per trial the haystack row is replaced by the
    unit vector along query + noise * N(0, I_d), a key close to the query.
    """
    hay = unit_gaussian(trials * seq_len, d, seed, DATA).reshape(trials, seq_len, d)
    q = unit_gaussian(trials, d, seed, QUERIES)
    pos = rng(seed, NEEDLE_POSITIONS).integers(0, seq_len, size=trials)
    nz = rng(seed, NEEDLE_NOISE).standard_normal((trials, d))
    needle = q.astype(np.float64) + noise * nz
    needle /= np.linalg.norm(needle, axis=1, keepdims=True)
    hay[np.arange(trials), pos] = needle.astype(np.float32)
    return np.ascontiguousarray(hay), q, pos.astype(np.int64)


def tiny_vectors(n: int = 4096, d: int = 128, seed: int = 0, n_outliers: int = 4,
                 factor: float = 20.0) -> np.ndarray:
    """float32 N(0,1) vectors with a few outlier channels scaled up.

    The outlier channels are a seeded choice of ``n_outliers`` distinct columns.
    """
    x = rng(seed, DATA).standard_normal((n, d)).astype(np.float32)
    ch = rng(seed, OUTLIER_CHANNELS).choice(d, size=n_outliers, replace=False)
    x[:, ch] *= np.float32(factor)
    return np.ascontiguousarray(x)


def kv_tensor(layers: int, heads: int, tokens: int, d: int, seed: int, value: bool = False,
              outlier_frac: float = 0.02, outlier_factor: float = 10.0,
              sigma: float = 0.5) -> np.ndarray:
    """A [layers, heads, tokens, d] float16 KV tensor with real-model-like channels.

    Each (layer, head, channel) gets a scale exp(sigma * N(0,1)) (lognormal(0, sigma));
    round(outlier_frac * d) channels per (layer, head), a seeded choice, are
    multiplied by ``outlier_factor``.  Entries are N(0,1) times the channel scale.
    Keys and values use disjoint random streams (``value``).
    """
    p_data, p_out, p_scale = (DATA_V, OUTLIER_CHANNELS_V, CHANNEL_SCALES_V) if value else \
        (DATA, OUTLIER_CHANNELS, CHANNEL_SCALES)
    scales = np.exp(sigma * rng(seed, p_scale).standard_normal((layers, heads, d)))
    n_out = int(round(outlier_frac * d))
    ro = rng(seed, p_out)
    for l in range(layers):
        for h in range(heads):
            ch = ro.choice(d, size=n_out, replace=False)
            scales[l, h, ch] *= outlier_factor
    scales = scales.astype(np.float32)
    out = np.empty((layers, heads, tokens, d), dtype=np.float16)
    rd = rng(seed, p_data)
    for l in range(layers):
        z = rd.standard_normal((heads, tokens, d), dtype=np.float32)
        out[l] = (z * scales[l][:, None, :]).astype(np.float16)
    return out


def mixture_database(n: int, d: int, n_components: int = 64, seed: int = 4,
                     n_queries: int = 0):
    """Unit-norm vectors from a Gaussian mixture (retrieval embeddings stand-in).

    Component means mu_k ~ N(0, I); a point is normalize(mu_k + xi), xi ~ N(0, I),
    with k uniform.  Returns (database [n, d] float32, queries [n_queries, d]
    float32), queries drawn fresh from the same mixture.
    """
    mu = rng(seed, MIXTURE_MEANS).standard_normal((n_components, d)).astype(np.float32)

    def draw(count, purpose_lab, purpose_noise):
        lab = rng(seed, purpose_lab).integers(0, n_components, size=count)
        out = np.empty((count, d), dtype=np.float32)
        rn = rng(seed, purpose_noise)
        step = 65536
        for s in range(0, count, step):
            e = min(count, s + step)
            v = mu[lab[s:e]] + rn.standard_normal((e - s, d), dtype=np.float32)
            v /= np.linalg.norm(v, axis=1, keepdims=True)
            out[s:e] = v
        return out

    db = draw(n, MIXTURE_LABELS, DATA)
    qs = draw(n_queries, MIXTURE_LABELS + 100, QUERIES) if n_queries else np.zeros((0, d), np.float32)
    return db, qs


def random_record_words(n: int, words_per_record: int, seed: int, scalar_ranges=((0.0, 1.0),)):
    """n records of uniformly random 32-bit plane words and float16 scalars.

    Every bit pattern is a valid code (uniformly random cell indices and sign
    bits), so these fill a packed cache at full size without encoding
    anything.  Returns (words [n, words_per_record] uint32, scalars [n, k]
    float16), scalar column j uniform on scalar_ranges[j]."""
    r = rng(seed, RANDOM_RECORDS)
    words = r.integers(0, 1 << 32, size=(n, words_per_record), dtype=np.uint64).astype(np.uint32)
    lo = np.array([a for a, _ in scalar_ranges])
    hi = np.array([b for _, b in scalar_ranges])
    sc = (lo[None, :] + (hi - lo)[None, :] * r.random((n, len(scalar_ranges)))).astype(np.float16)
    return words, sc
