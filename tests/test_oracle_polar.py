"""Pins for oracle.polar (PolarQuant as stage 1, recursive form) and its record
packing: hand-worked transforms, the d = 2 case (ordinary polar coordinates),
exact inverses, the angle laws against sampled uniform vectors, the closed-form
one-bit codebook of level 2, brute-force Lloyd-Max optima, nearest-centroid
codes, unbiasedness of the two-stage estimate over QJL matrices, and hand-built
record words."""
import numpy as np
import pytest
from scipy import integrate, stats

from oracle import packing as pk
from oracle import polar as pq
from oracle import transforms as tr
from tests.conftest import mean_se
from tq_inputs import gaussian_matrix, haar_orthogonal, rng


def _angles(y):
    a, r = pq.polar_transform(np.asarray(y, np.float64)[None])
    return [x[0].tolist() for x in a], float(r[0])


def test_worked_examples():
    q = np.pi / 4
    # all four coordinates equal: every pair and every pair of radii sits at 45 degrees
    a, r = _angles([0.5, 0.5, 0.5, 0.5])
    assert np.allclose(a[0], [q, q]) and np.allclose(a[1], [q]) and abs(r - 1) < 1e-15
    # the last axis: the first pair is empty (atan2(0, 0) = 0), the second points up,
    # and the first pair's radius is 0, so the level-2 angle is 90 degrees
    a, r = _angles([0, 0, 0, 1])
    assert np.allclose(a[0], [0, np.pi / 2]) and np.allclose(a[1], [np.pi / 2])
    # the negative first axis: angle pi at level 1, and 0 above (all length in block 0)
    a, r = _angles([-1, 0, 0, 0])
    assert np.allclose(a[0], [np.pi, 0]) and np.allclose(a[1], [0])
    # a 3-4-5 pair in d = 8: one nonzero level-1 angle, zeros above
    a, r = _angles([0.6, 0.8, 0, 0, 0, 0, 0, 0])
    assert np.allclose(a[0], [np.arctan(4 / 3), 0, 0, 0])
    assert np.allclose(a[1], [0, 0]) and np.allclose(a[2], [0]) and abs(r - 1) < 1e-15
    # the level-3 angle between the halves of (1,0,0,0, 0,0,1,1)/sqrt(3): tan = sqrt(2)
    a, r = _angles(np.array([1, 0, 0, 0, 0, 0, 1, 1]) / np.sqrt(3))
    assert np.allclose(a[2], [np.arctan(np.sqrt(2))]) and np.allclose(a[1], [0, np.pi / 2])
    assert np.allclose(a[0], [0, 0, 0, q])


def test_d2_is_ordinary_polar_coordinates():
    phi = np.linspace(-np.pi + 1e-3, np.pi, 41)
    r = np.linspace(0.1, 3.0, 41)
    y = np.stack([r * np.cos(phi), r * np.sin(phi)], axis=1)
    a, rad = pq.polar_transform(y)
    assert len(a) == 1
    assert np.allclose(a[0][:, 0], phi, atol=1e-13) and np.allclose(rad, r, atol=1e-13)


@pytest.mark.parametrize("d", [2, 4, 64, 128, 256])
def test_inverse_is_exact(d):
    y = rng(0, d).standard_normal((50, d))
    a, r = pq.polar_transform(y)
    assert [x.shape[1] for x in a] == [d >> l for l in range(1, pq.n_levels(d) + 1)]
    assert np.allclose(pq.polar_inverse(a, r), y, atol=1e-12)
    assert np.allclose(r, np.linalg.norm(y, axis=1), atol=1e-12)
    for l, x in enumerate(a, start=1):
        lo = -np.pi if l == 1 else 0.0
        hi = np.pi if l == 1 else np.pi / 2
        assert np.all((x >= lo) & (x <= hi))


@pytest.mark.parametrize("level", [2, 3, 5, 7])
def test_cdf_is_integral_of_pdf(level):
    assert abs(integrate.quad(lambda t: pq.angle_pdf(t, level), 0, np.pi / 2)[0] - 1) < 1e-10
    for t in (0.2, 0.6, np.pi / 4, 1.1, 1.4):
        v = integrate.quad(lambda s: pq.angle_pdf(s, level), 0, t, epsabs=1e-14)[0]
        assert abs(v - pq.angle_cdf(t, level)) < 1e-10
    # symmetric about pi/4
    assert abs(pq.angle_cdf(np.pi / 4, level) - 0.5) < 1e-14


def test_angle_laws_of_uniform_vectors():
    # the angles of a uniformly rotated vector (a uniform point on the sphere)
    d = 128
    y = rng(1, 77).standard_normal((6000, d))
    y /= np.linalg.norm(y, axis=1, keepdims=True)
    a, _ = pq.polar_transform(y)
    for l, x in enumerate(a, start=1):
        sample = x[:, 0] if l < 7 else x[:, 0]
        p = stats.kstest(sample, lambda t: pq.angle_cdf(t, l)).pvalue
        assert p > 1e-3, (l, p)
        if l >= 2:
            # sin^2 psi ~ Beta(a, a): mean 1/2, variance 1/(4 (2a + 1)), a = 2^(l-2)
            s2 = np.sin(x.ravel()) ** 2
            av = 2.0 ** (l - 2)
            assert abs(s2.mean() - 0.5) < 5 * np.sqrt(0.25 / (2 * av + 1) / s2.size)
            assert abs(s2.var() / (0.25 / (2 * av + 1)) - 1) < 0.08
    # independent levels: the level-1 and level-2 angles of one block are uncorrelated
    c = np.corrcoef(a[0][:, 0], a[1][:, 0])[0, 1]
    assert abs(c) < 4 / np.sqrt(6000)


def test_level2_one_bit_closed_form():
    # density sin(2 psi) on [0, pi/2]: the 1-bit cells split at pi/4, and the lower
    # centroid is 2 * int_0^{pi/4} psi sin(2 psi) dpsi = 1/2
    c, b = pq.angle_codebook(2, 1)
    assert abs(b[0] - np.pi / 4) < 1e-12
    assert np.allclose(c, [0.5, np.pi / 2 - 0.5], atol=1e-11)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_level1_uniform_grid(bits):
    c, b = pq.uniform_codebook(bits)
    K = 2 ** bits
    w = 2 * np.pi / K
    assert np.allclose(np.diff(c), w) and abs(c[0] + np.pi - w / 2) < 1e-15
    assert np.allclose(b, 0.5 * (c[1:] + c[:-1]))
    # the mean squared angle error of a uniform angle is w^2 / 12
    psi = rng(2, bits).uniform(-np.pi, np.pi, 200000)
    err = psi - c[np.searchsorted(b, psi, side="right")]
    assert abs(np.mean(err ** 2) / (w * w / 12) - 1) < 0.02


def _mse(level, c, b, grid):
    t = grid
    w = pq.angle_pdf(t, level)
    idx = np.searchsorted(b, t, side="right")
    return np.sum(w * (t - c[idx]) ** 2) * (t[1] - t[0])


def _grid_cell_means(level, b, grid):
    w = pq.angle_pdf(grid, level)
    idx = np.searchsorted(b, grid, side="right")
    return np.array([np.sum(w[idx == k] * grid[idx == k]) / np.sum(w[idx == k]) for k in range(len(b) + 1)])


@pytest.mark.parametrize("level,bits", [(2, 2), (3, 2), (4, 1), (6, 2)])
def test_lloyd_matches_brute_force(level, bits):
    grid = np.linspace(0, np.pi / 2, 200001)
    c, b = pq.angle_codebook(level, bits)
    # fixed point, with the means taken by a plain Riemann sum instead of quadrature
    assert np.allclose(_grid_cell_means(level, b, grid), c, atol=2e-6)
    # no symmetric boundary placement on a search grid does better
    best = _mse(level, c, b, grid)
    if bits == 1:
        for t in np.linspace(0.3, 1.2, 91):
            bb = np.array([t])
            cc = _grid_cell_means(level, bb, grid)
            assert _mse(level, cc, bb, grid) >= best - 1e-12
    else:
        for t in np.linspace(0.01, np.pi / 4 - 0.01, 157):
            bb = np.array([np.pi / 4 - t, np.pi / 4, np.pi / 4 + t])
            cc = _grid_cell_means(level, bb, grid)
            assert _mse(level, cc, bb, grid) >= best - 1e-12


def _setup(d=128, seed=3, bits1=3, bits=2, m=None):
    pi = haar_orthogonal(d, seed)
    rot = tr.DenseRotation(pi)
    cbs = pq.level_codebooks(d, bits1, bits)
    s = gaussian_matrix(m, d, seed) if m else None
    return rot, cbs, s


def test_codes_are_nearest_centroids():
    rot, cbs, _ = _setup()
    x = rng(4, 1).standard_normal((300, 128))
    code = pq.encode_polar(x, rot, cbs, storage=False)
    for l, (cells, psi, (c, b)) in enumerate(zip(code.codes, code.angles, cbs), start=1):
        dist = np.abs(psi[..., None] - np.asarray(c)[None, None, :])
        near = np.argmin(dist, axis=-1)
        srt = np.sort(dist, axis=-1)
        clear = srt[..., 1] - srt[..., 0] > 1e-12
        assert np.array_equal(cells[clear], near[clear]), l


def test_reconstruction_on_the_sphere_and_decode_norm():
    rot, cbs, _ = _setup(bits1=2, bits=1)
    x = rng(5, 1).standard_normal((200, 128)) * 3.0
    code = pq.encode_polar(x, rot, cbs, storage=False)
    assert np.allclose(np.linalg.norm(code.y_hat, axis=1), 1.0, atol=1e-13)
    assert np.allclose(np.linalg.norm(pq.decode_polar(code, rot), axis=1), np.linalg.norm(x, axis=1), atol=1e-12)
    # arbitrary cells reconstruct on the sphere too
    codes = [rng(6, l).integers(0, len(cb[0]), c.shape) for l, (c, cb) in enumerate(zip(code.codes, cbs))]
    assert np.allclose(np.linalg.norm(pq.reconstruct(codes, cbs), axis=1), 1.0, atol=1e-13)


def test_zero_vector():
    rot, cbs, s = _setup(m=128)
    code = pq.encode_polar(np.zeros((1, 128)), rot, cbs, s, storage=False)
    assert code.n[0] == 0.0
    assert all(np.all(psi == 0.0) for psi in code.angles)
    # level 1 angle 0 lies in the cell starting at 0; angle 0 sits below every upper boundary
    assert np.all(code.codes[0] == len(cbs[0][0]) // 2) and all(np.all(c == 0) for c in code.codes[1:])
    assert np.all(pq.polar_scores(rng(7, 1).standard_normal((2, 128)), code, rot, s) == 0.0)


def test_scores_without_stage2_equal_decoded_inner_products():
    # <Pi q, y~> n against <q, n Pi^T y~>: a transposed rotation fails this
    rot, cbs, _ = _setup()
    x = rng(8, 1).standard_normal((40, 128))
    q = rng(8, 2).standard_normal((3, 128))
    code = pq.encode_polar(x, rot, cbs, storage=True)
    assert np.allclose(pq.polar_scores(q, code, rot), q @ pq.decode_polar(code, rot).T, atol=1e-11)


def test_two_stage_estimate_is_unbiased_over_qjl_matrices():
    d = 16
    rot = tr.DenseRotation(haar_orthogonal(d, 9))
    cbs = pq.level_codebooks(d, 2, 1)
    x = rng(9, 1).standard_normal((1, d))
    q = rng(9, 2).standard_normal((1, d))
    est = []
    for k in range(4000):
        s = rng(100 + k, 3).standard_normal((d, d))
        est.append(pq.polar_scores(q, pq.encode_polar(x, rot, cbs, s, storage=False), rot, s)[0, 0])
    mu, se = mean_se(est)
    assert abs(mu - float(q[0] @ x[0])) < 4 * se
    # the polar stage alone is biased for this x (the check above is not vacuous)
    alone = pq.polar_scores(q, pq.encode_polar(x, rot, cbs, storage=False), rot)[0, 0]
    assert abs(alone - float(q[0] @ x[0])) > 4 * se


def test_stream_packing_hand_built():
    # d = 8, b1 = 3, b = 2: level-1 cells 5, 1, 7, 2 -> stream bits 101 100 111 010
    # (least significant first) = word 1 + 4 + 8 + 64 + 128 + 256 + 1024 = 1485;
    # upper cells (level 2: 3, 0; level 3: 2) -> bits 11 00 01 = 1 + 2 + 32 = 35
    code = pq.PolarCode(codes=[np.array([[5, 1, 7, 2]]), np.array([[3, 0]]), np.array([[2]])],
                        n=np.array([1.5]), y=None, angles=None, y_hat=None)
    w, s = pk.pack_polar(code, 3, 2)
    assert w.tolist() == [[1485, 35]] and s.tolist() == [[1.5]]
    codes, z, n, g = pk.unpack_polar(w, s, 8, 3, 2, 0)
    assert [c.tolist() for c in codes] == [[[5, 1, 7, 2]], [[3, 0]], [[2]]] and z is None and n[0] == 1.5


def test_stream_packing_straddles_words():
    # b = 3 at d = 128: level-1 cell 10 (value 5 = 101b) occupies bits 30, 31 of word 0
    # and bit 0 of word 1
    cells = np.zeros((1, 64), np.int64)
    cells[0, 10] = 5
    w = pk.pack_stream(cells, 3)
    assert w.shape == (1, 6) and w[0, 0] == (1 << 30) and w[0, 1] == 1 and not np.any(w[0, 2:])


@pytest.mark.parametrize("bits1,bits,m", [(1, 1, 0), (2, 3, 128), (3, 2, 128), (4, 4, 0), (4, 2, 128)])
def test_record_round_trip(bits1, bits, m):
    rot, cbs, s = _setup(bits1=bits1, bits=bits, m=m)
    x = rng(10, bits1 * 8 + bits).standard_normal((64, 128))
    code = pq.encode_polar(x, rot, cbs, s)
    w, sc = pk.pack_polar(code, bits1, bits)
    assert w.shape[1] == pk.polar_record_words(128, bits1, bits, m) == 2 * bits1 + 2 * bits + m // 32
    codes, z, n, g = pk.unpack_polar(w, sc, 128, bits1, bits, m)
    assert all(np.array_equal(a, b) for a, b in zip(codes, code.codes))
    assert np.array_equal(n, code.n)
    if m:
        assert np.array_equal(z, code.z) and np.array_equal(g, code.gamma)
