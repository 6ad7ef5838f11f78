"""Pins for oracle.quantizer and oracle.packing."""
import itertools

import numpy as np
import pytest

from oracle import codebook as cb
from oracle import packing as pk
from oracle import quantizer as qz
from oracle import transforms as tr
from tests.conftest import read_golden
from tq_inputs import gaussian_matrix, haar_orthogonal


@pytest.mark.parametrize("bits", [1, 2])
def test_brute_force_nearest_codeword_d8(bits):
    # over all 2^(8b) product codewords, the nearest one is the per-coordinate
    # cell index (the product codebook of section 6 of the explainer page)
    d = 8
    c, b = cb.lloyd_max(d, bits)
    rg = np.random.default_rng(7)
    y = rg.standard_normal((25, d))
    y /= np.linalg.norm(y, axis=1, keepdims=True)
    words = np.array(list(itertools.product(range(2 ** bits), repeat=d)))
    cw = c[words]                                   # [K^d, d]
    for v in y:
        best = words[np.argmin(((cw - v) ** 2).sum(axis=1))]
        assert np.array_equal(qz.cell_index(v[None, :], b)[0], best)


def test_cell_index_ties_go_up():
    b = np.array([-0.5, 0.0, 0.5])
    assert qz.cell_index(np.array([[-0.5, 0.0, 0.5, -0.6, 0.7]]), b).tolist() == [[1, 2, 3, 0, 3]]


def test_zero_vector():
    d = 32
    c, b = cb.lloyd_max(d, 2)
    rot = tr.DenseRotation(haar_orthogonal(d, 0))
    code = qz.encode_prod(np.zeros((1, d)), rot, gaussian_matrix(d, d, 0), c, b)
    assert code.n[0] == 0
    assert np.all(code.idx == 2)
    assert abs(code.gamma[0] - np.float16(np.sqrt(d) * c[2])) < 1e-3


def test_mse_falls_about_4x_per_bit_and_matches_distortion():
    d = 128
    rg = np.random.default_rng(5)
    x = rg.standard_normal((3000, d)) * np.exp(rg.standard_normal(d))[None, :]
    rot = tr.DenseRotation(haar_orthogonal(d, 11))
    from oracle.estimator import dequantize
    errs = []
    for bits in (1, 2, 3, 4):
        c, b = cb.lloyd_max(d, bits)
        code = qz.encode_mse(x, rot, c, b, storage=False)
        xt = dequantize(code.idx, code.n, rot, c)
        e = ((x - xt) ** 2).sum(1) / (x ** 2).sum(1)
        m, se = e.mean(), e.std(ddof=1) / np.sqrt(len(e))
        # the random rotation makes any fixed input look uniform on the sphere
        assert abs(m - d * cb.distortion(d, c, b)) < 4 * se + 1e-4
        errs.append(m)
    ratios = np.array(errs[:-1]) / np.array(errs[1:])
    assert np.all((ratios > 2.9) & (ratios < 4.2))


def test_residual_energy_is_b_minus_1_distortion():
    # E||r||^2 = d * D(b-1) for the prod residual
    d, bits = 64, 3
    c, b = cb.lloyd_max(d, bits - 1)
    rg = np.random.default_rng(9)
    x = rg.standard_normal((4000, d))
    rot = tr.DenseRotation(haar_orthogonal(d, 4))
    code = qz.encode_prod(x, rot, gaussian_matrix(d, d, 4), c, b, storage=False)
    g2 = code.gamma ** 2
    assert abs(g2.mean() - d * cb.distortion(d, c, b)) < 4 * g2.std() / np.sqrt(len(g2))


def test_float16_storage_rounds_to_nearest_even():
    one = 1.0
    ulp = 2.0 ** -10
    v = np.array([one + ulp / 2, one + 1.5 * ulp, one + ulp / 2 + 1e-9, 65519.0, 2.0 ** -25 * 1.0000001])
    out = qz._store(v, True)
    assert out[0] == 1.0                 # midpoint -> even
    assert out[1] == 1.0 + 2 * ulp       # midpoint -> even (up)
    assert out[2] == 1.0 + ulp           # above midpoint -> up
    assert out[3] == 65504.0
    assert out[4] == 2.0 ** -24          # subnormal range, above the midpoint


def test_pack_hand_built_words():
    idx = np.zeros((1, 64), np.int64)
    idx[0, 0] = 1          # plane 0, word 0, bit 0
    idx[0, 33] = 2         # plane 1, word 1, bit 1
    idx[0, 31] = 3         # both planes, word 0, bit 31
    planes = pk.index_planes(idx, 2)
    assert planes.shape == (1, 2, 2)
    assert planes[0, 0].tolist() == [1 | (1 << 31), 0]
    assert planes[0, 1].tolist() == [1 << 31, 2]
    assert np.array_equal(pk.planes_to_index(planes), idx)
    # record order interleaves the planes word by word: w0p0 w0p1 w1p0 w1p1
    rec = pk.interleave(planes).reshape(1, -1)
    assert rec[0].tolist() == [1 | (1 << 31), 1 << 31, 0, 2]


def test_pack_roundtrip_random():
    rg = np.random.default_rng(2)
    idx = rg.integers(0, 8, size=(7, 128))
    z = rg.integers(0, 2, size=(7, 128)).astype(bool)
    code = qz.ProdCode(idx=idx, z=z, n=rg.random(7) * 10, gamma=rg.random(7), y=None, proj=None)
    planes, scal = pk.pack_key(code, 3)
    assert planes.shape == (7, 4, 4)
    # word w of plane p sits at w * P + p of the record
    pm = pk.index_planes(idx, 3)
    assert np.array_equal(planes.reshape(7, -1)[:, 1 * 4 + 2], pm[:, 2, 1])
    assert np.array_equal(planes.reshape(7, -1)[:, 3 * 4 + 3], pk.pack_bits(z)[:, 3])
    i2, z2, n2, g2 = pk.unpack_key(planes, scal, 3)
    assert np.array_equal(i2, idx) and np.array_equal(z2, z)
    assert np.allclose(n2, code.n, rtol=1e-3) and np.allclose(g2, code.gamma, rtol=1e-3, atol=1e-4)


def test_record_sizes_reproduce_printed_compression_ratios():
    # key = (b-1) d index bits + d sign bits + 2 float16; value = b d bits + 1 float16,
    # against 2 float16 vectors of d = 128 per token-head
    for bits, ratio in read_golden("compression.txt"):
        bits = int(bits)
        r = (2 * 128 * 2) / (pk.key_record_bytes(128, 128, bits) + pk.value_record_bytes(128, bits))
        assert round(r, 1) == float(ratio)
    assert pk.key_record_bytes(128, 128, 3) == 52 and pk.value_record_bytes(128, 3) == 50


def test_value_blocks_hand_built_and_roundtrip():
    idx = np.zeros((40, 64), np.int64)
    idx[0, 0] = 1          # block 0, coord 0, plane 0, bit 0
    idx[5, 3] = 2          # block 0, coord 3, plane 1, bit 5
    idx[33, 63] = 3        # block 1, coord 63, planes 0 and 1, bit 1
    w = pk.pack_value_blocks(idx, 2)
    assert w.shape == (2, 64, 2)
    assert w[0, 0, 0] == 1 and w[0, 0, 1] == 0
    assert w[0, 3, 1] == 1 << 5 and w[0, 3, 0] == 0
    assert w[1, 63, 0] == 2 and w[1, 63, 1] == 2
    assert np.count_nonzero(w) == 4
    rg = np.random.default_rng(4)
    r = rg.integers(0, 8, size=(77, 128))
    assert np.array_equal(pk.unpack_value_blocks(pk.pack_value_blocks(r, 3), 77), r)


def _eden_recon(code, rot, c):
    return code.n[:, None] * rot.inverse(np.asarray(c, np.float64)[code.idx])


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_eden_reconstruction_has_exact_projection_on_x(bits):
    # <x, S Pi^T c[idx]> = S <Pi x, c[idx]> = ||x||^2 (the scale's definition,
    # explainer page section 0.9, EDEN), for every vector and rotation
    d = 64
    rg = np.random.default_rng(bits)
    x = rg.standard_normal((50, d)) * rg.uniform(0.1, 10, size=(50, 1))
    rot = tr.DenseRotation(haar_orthogonal(d, 3, 2))
    c, b = cb.lloyd_max(d, bits)
    code = qz.encode_eden(x, rot, c, b, storage=False)
    xh = _eden_recon(code, rot, c)
    np.testing.assert_allclose(np.sum(x * xh, axis=1), np.sum(x * x, axis=1), rtol=1e-12)


def test_eden_one_bit_is_drive_unbiased_scale():
    # at one bit c[idx] = +-c1 sign(y): S c1 = ||x||^2 / ||Pi x||_1 (DRIVE's unbiased scale)
    d = 32
    x = np.random.default_rng(5).standard_normal((20, d)) * 3.0
    rot = tr.DenseRotation(haar_orthogonal(d, 4, 2))
    c, b = cb.lloyd_max(d, 1)
    code = qz.encode_eden(x, rot, c, b, storage=False)
    drive = np.sum(x * x, axis=1) / np.sum(np.abs(x @ haar_orthogonal(d, 4, 2).astype(np.float64).T), axis=1)
    np.testing.assert_allclose(code.n * c[1], drive, rtol=1e-12)


def test_eden_reconstruction_unbiased_over_rotations():
    # E over uniformly random rotations of S Pi^T c[idx] is x (EDEN's
    # unbiasedness); 3000 Haar rotations at d = 16, b = 2: each coordinate of
    # the mean within 4 standard errors of x
    d, trials = 16, 3000
    x = np.random.default_rng(7).standard_normal((1, d))
    c, b = cb.lloyd_max(d, 2)
    recs = []
    for t in range(trials):
        rot = tr.DenseRotation(haar_orthogonal(d, 1000 + t, 2))
        recs.append(_eden_recon(qz.encode_eden(x, rot, c, b, storage=False), rot, c)[0])
    recs = np.array(recs)
    mean, se = recs.mean(0), recs.std(0, ddof=1) / np.sqrt(trials)
    assert np.all(np.abs(mean - x[0]) < 4 * se), np.max(np.abs(mean - x[0]) / se)
    # the plain MSE reconstruction n Pi^T c[idx] is shrunk: its mean falls short of x
    mse = np.array([_eden_recon(qz.encode_mse(x, tr.DenseRotation(haar_orthogonal(d, 1000 + t, 2)), c, b,
                                              storage=False), tr.DenseRotation(haar_orthogonal(d, 1000 + t, 2)), c)[0]
                    for t in range(200)])
    assert mse.mean(0) @ x[0] < 0.97 * (x[0] @ x[0])


def test_eden_zero_vector():
    rot = tr.DenseRotation(haar_orthogonal(8, 1, 2))
    c, b = cb.lloyd_max(8, 2)
    code = qz.encode_eden(np.zeros((1, 8)), rot, c, b)
    assert code.n[0] == 0.0


def test_pack_key_half_projection_hand_built_and_roundtrip():
    # m = 64 QJL rows at d = 128, b - 1 = 2 index bits: group w holds index
    # words (plane 0, plane 1), then sign word w for w < 2
    rg = np.random.default_rng(9)
    idx = rg.integers(0, 4, size=(3, 128))
    z = rg.integers(0, 2, size=(3, 64)).astype(bool)
    code = qz.ProdCode(idx=idx, z=z, n=np.ones(3), gamma=np.ones(3), y=None, proj=None)
    words, scal = pk.pack_key(code, 2)
    assert words.shape == (3, 10)
    for v in range(3):
        for w in range(4):
            off = 2 * w + min(w, 2)
            for p in range(2):
                want = sum(int((idx[v, 32 * w + j] >> p) & 1) << j for j in range(32))
                assert int(words[v, off + p]) == want
            if w < 2:
                want = sum(int(z[v, 32 * w + j]) << j for j in range(32))
                assert int(words[v, off + 2]) == want
    i2, z2, _, _ = pk.unpack_key(words, scal, 2, d=128)
    assert np.array_equal(i2, idx) and np.array_equal(z2, z)
    assert pk.key_record_bytes(128, 64, 3) == 44
