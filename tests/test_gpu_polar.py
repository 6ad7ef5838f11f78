"""GPU parity of the PolarQuant stage-1 path (tq_polar_encode / _decode /
_scores) against oracle.polar.

Encode: the GPU's cells must equal the oracle's except for an angle within
1e-5 rad of one of its level's boundaries (float32 decisions against float64
ones), at most 1e-4 of the angles; n exact in float16 (one ulp only at a
rounding midpoint); gamma and the QJL signs on every vector whose cells all
agree, the signs exact except where |S r| < 1e-5.  Decode and scores run on
records the oracle encoded and packed, so both sides see the same cells; the
float32 results must lie within 1e-5 (decode) and 2e-5 (scores) of the scale
the inputs set (n ||q|| per token, n per vector), a bound taken from the
inputs, never from the output under test."""
import numpy as np
import pytest

import kv_cache_vector_02_amd as tq
from oracle import packing as pk
from oracle import polar as pq
from oracle import transforms as tr
from tests.gpu_util import _f16_ulp_apart, _near_midpoint_f16, torch
from tq_inputs import gaussian_matrix, gaussian_queries, haar_orthogonal, kv_tensor, sign_vector, tiny_vectors

pytestmark = pytest.mark.gpu
ANGLE_EPS = 1e-5
MAX_FLIP_FRAC = 1e-4


def _log(msg):
    print(msg, flush=True)


class PolarSetup:
    """Seeded rotation, QJL matrix and float32 level codebooks, on host and device."""

    def __init__(self, bits1=3, bits=2, m=128, rot="dense", seed=0):
        T = torch()
        self.bits1, self.bits, self.m = bits1, bits, m
        books = pq.level_codebooks(128, bits1, bits)
        self.books32 = [(c.astype(np.float32), b.astype(np.float32)) for c, b in books]
        cat_c = np.concatenate([c for c, _ in self.books32])
        cat_b = np.concatenate([b for _, b in self.books32])
        dev = lambda a: None if a is None else T.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
        if rot == "dense":
            self.pi = haar_orthogonal(128, seed, 2)
            self.rot = tr.DenseRotation(self.pi)
            self.eps = None
            kind = tq.TQ_ROT_DENSE
        else:
            self.eps = sign_vector(128, seed, 5)
            self.rot = tr.HadamardRotation(self.eps, 128)
            self.pi = None
            kind = tq.TQ_ROT_HADAMARD
        self.s = gaussian_matrix(128, 128, seed, 3) if m else None
        self.params = tq.PolarParams(d=128, rot=kind, bits1=bits1, bits=bits, centroids=cat_c, boundaries=cat_b,
                                     pi=dev(self.pi), eps=dev(self.eps), s=dev(self.s), m=m)

    def oracle(self, x, storage=True):
        return pq.encode_polar(x, self.rot, self.books32, self.s, storage=storage)

    def packed_cache(self, code, seg_stride=0):
        T = torch()
        words, scal = pk.pack_polar(code, self.bits1, self.bits)
        return tq.Cache(T.from_numpy(words.view(np.int32)).cuda(), T.from_numpy(scal).cuda(), seg_stride)

    def encode_gpu(self, x, records=None, slot=None):
        T = torch()
        xd = T.from_numpy(np.ascontiguousarray(x)).cuda()
        cache = tq.alloc_polar_cache(self.params, records or x.shape[0])
        sl = None if slot is None else T.from_numpy(np.asarray(slot, np.int64)).cuda()
        tq.polar_encode(self.params, xd, cache, slot=sl)
        T.cuda.synchronize()
        return cache.planes.cpu().numpy().view(np.uint32), cache.scalars.cpu().numpy()


def compare_encode(st: PolarSetup, words, scal, code):
    """Check GPU records against the oracle's exact-mode code; returns statistics."""
    cells, z, n, g = pk.unpack_polar(words, scal, 128, st.bits1, st.bits, st.m)
    vec_ok = np.ones(words.shape[0], bool)
    flips = 0
    for l, (got, want, psi, (_, b)) in enumerate(zip(cells, code.codes, code.angles, st.books32), start=1):
        mism = got != want
        if np.any(mism):
            dist = np.min(np.abs(psi[..., None] - np.asarray(b, np.float64)[None, None, :]), axis=-1)
            assert np.all(dist[mism] < ANGLE_EPS), f"level {l}: cell flips away from a boundary {dist[mism].max()}"
        flips += int(mism.sum())
        vec_ok &= ~np.any(mism, axis=1)
    assert flips <= max(1, MAX_FLIP_FRAC * 127 * words.shape[0]), flips
    dn = _f16_ulp_apart(scal[:, 0], code.n.astype(np.float16))
    assert not np.any((dn > 1) | ((dn == 1) & ~_near_midpoint_f16(code.n))), "norm mismatch"
    stats = {"cell_flips": flips}
    if st.m:
        zm = (z != code.z) & vec_ok[:, None]
        if np.any(zm):
            assert np.all(np.abs(code.proj[zm]) < 1e-5), f"sign flips away from zero {np.abs(code.proj[zm]).max()}"
        assert zm.sum() <= max(1, MAX_FLIP_FRAC * zm.size)
        dg = _f16_ulp_apart(scal[:, 1], code.gamma.astype(np.float16))
        bad = vec_ok & ((dg > 1) | ((dg == 1) & ~_near_midpoint_f16(code.gamma)))
        assert not np.any(bad), f"gamma mismatch at {np.nonzero(bad)[0][:5]}"
        stats["sign_flips"] = int(zm.sum())
    return stats


@pytest.mark.parametrize("bits1,bits,m,rot,dtype", [
    (3, 2, 128, "dense", np.float32), (4, 2, 128, "dense", np.float16), (1, 1, 0, "dense", np.float32),
    (2, 3, 0, "hadamard", np.float16), (4, 4, 128, "hadamard", np.float32), (3, 3, 128, "dense", np.float16),
    (2, 4, 0, "dense", np.float32), (4, 1, 128, "hadamard", np.float16)])
def test_encode(bits1, bits, m, rot, dtype):
    _log(f"polar encode b1={bits1} b={bits} m={m} {rot} {np.dtype(dtype).name}")
    st = PolarSetup(bits1, bits, m, rot, seed=bits1 * 10 + bits)
    x = tiny_vectors(3000, 128, seed=bits1 + 7 * bits).astype(dtype)     # ragged last tile of 32
    words, scal = st.encode_gpu(x)
    stats = compare_encode(st, words, scal, st.oracle(x.astype(np.float64), storage=False))
    _log(f"  {stats}")


def test_encode_large_batch_eight_wave_workgroups():
    # > 2 tiles per compute unit: the eight-wave launch shape, with a ragged tail
    st = PolarSetup(4, 2, 128, "dense", seed=3)
    x = kv_tensor(1, 8, 20001, 128, seed=3).reshape(-1, 128)[:160003]
    _log(f"polar encode {x.shape[0]} vectors")
    words, scal = st.encode_gpu(x)
    _log(f"  {compare_encode(st, words, scal, st.oracle(x.astype(np.float64), storage=False))}")


def test_encode_zero_vectors_slots_and_capacity():
    st = PolarSetup(3, 2, 128, "dense", seed=4)
    rg = np.random.default_rng(4)
    x = rg.standard_normal((70, 128)).astype(np.float32)
    x[[0, 33, 69]] = 0.0
    slot = rg.permutation(100)[:70]
    slot[5] = 100          # outside the capacity: not written
    slot[6] = -1
    words, scal = st.encode_gpu(x, records=100, slot=slot)
    keep = (slot >= 0) & (slot < 100)
    code = st.oracle(x[keep].astype(np.float64), storage=False)
    compare_encode(st, words[slot[keep]], scal[slot[keep]], code)
    untouched = np.setdiff1d(np.arange(100), slot[keep])
    assert not np.any(words[untouched]) and not np.any(scal[untouched].view(np.uint16))
    zero_rows = slot[[0, 33, 69]]
    assert np.all(scal[zero_rows, 0] == 0)


def _decode_gpu(st, cache, n):
    T = torch()
    out = T.full((n, 130), float("nan"), dtype=T.float32, device="cuda")
    tq.polar_decode(st.params, cache, n, out)
    T.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("bits1,bits,m,rot", [(3, 2, 128, "dense"), (4, 4, 0, "hadamard"), (1, 3, 0, "dense"),
                                              (2, 1, 128, "hadamard")])
def test_decode(bits1, bits, m, rot):
    _log(f"polar decode b1={bits1} b={bits} m={m} {rot}")
    st = PolarSetup(bits1, bits, m, rot, seed=5)
    x = tiny_vectors(1000, 128, seed=5)
    code = st.oracle(x)                       # storage mode: float16 n, as the record holds it
    got = _decode_gpu(st, st.packed_cache(code), 1000)
    want = pq.decode_polar(code, st.rot)
    assert np.all(np.isnan(got[:, 128:]))     # nothing written past d
    err = np.abs(got[:, :128] - want)
    assert np.all(err <= 1e-5 * np.maximum(code.n, 1e-30)[:, None]), err.max()


def _scores_gpu(st, q, segs, group, cache, T_, length=None):
    T = torch()
    qd = T.from_numpy(np.ascontiguousarray(q, np.float32)).cuda()
    out = T.full((segs * group, T_), float("nan"), dtype=T.float32, device="cuda")
    ln = None if length is None else T.from_numpy(np.asarray(length, np.int32)).cuda()
    tq.polar_scores(st.params, qd, segs, group, cache, T_, out, length=ln)
    T.cuda.synchronize()
    return out.cpu().numpy()


def _check_scores(got, q, code, st, segs, group, stride, T_, length):
    for s in range(segs):
        ln = T_ if length is None else length[s]
        sub = pq.PolarCode(codes=[c[s * stride:s * stride + ln] for c in code.codes], n=code.n[s * stride:s * stride + ln],
                           y=None, angles=None, y_hat=code.y_hat[s * stride:s * stride + ln],
                           z=None if code.z is None else code.z[s * stride:s * stride + ln],
                           gamma=None if code.gamma is None else code.gamma[s * stride:s * stride + ln])
        qs = q[s * group:(s + 1) * group]
        want = pq.polar_scores(qs, sub, st.rot, st.s)
        rows = got[s * group:(s + 1) * group]
        scale = np.linalg.norm(qs, axis=1)[:, None] * np.max(sub.n, initial=0.0)
        assert np.all(np.abs(rows[:, :ln] - want) <= 2e-5 * scale), (s, np.max(np.abs(rows[:, :ln] - want)))
        assert np.all(np.isnan(rows[:, ln:])), "tokens at or past len written"


@pytest.mark.parametrize("bits1,bits,m,rot,group", [
    (3, 2, 128, "dense", 4), (4, 2, 128, "dense", 8), (4, 4, 0, "hadamard", 16), (1, 1, 0, "dense", 1),
    (2, 3, 128, "hadamard", 5), (3, 4, 0, "dense", 12)])
def test_scores_segments(bits1, bits, m, rot, group):
    # several segments with a stride past T, ragged lengths, several workgroups
    # per segment (T spans several 256-token passes) and every head-quad count
    segs, T_, stride = 6, 1300, 1400
    _log(f"polar scores b1={bits1} b={bits} m={m} {rot} G={group}")
    st = PolarSetup(bits1, bits, m, rot, seed=6 + group)
    x = kv_tensor(1, segs, stride, 128, seed=6).reshape(-1, 128)
    code = st.oracle(x)
    q = gaussian_queries(segs * group, 128, seed=6)
    length = [1300, 0, 257, 1, 1299, 640]
    got = _scores_gpu(st, q, segs, group, st.packed_cache(code, stride), T_, length)
    _check_scores(got, q, code, st, segs, group, stride, T_, length)


def test_scores_many_segments_full_launch():
    # 64 segments x 8192 tokens, GQA group 4: the launch shape of a long cache
    segs, T_, group = 64, 8192, 4
    _log(f"polar scores {segs} x {T_} x G{group}")
    st = PolarSetup(4, 2, 128, "dense", seed=9)
    x = kv_tensor(4, 16, T_, 128, seed=9).reshape(-1, 128)
    code = st.oracle(x)
    q = gaussian_queries(segs * group, 128, seed=9)
    got = _scores_gpu(st, q, segs, group, st.packed_cache(code, T_), T_)
    _check_scores(got, q, code, st, segs, group, T_, T_, None)
