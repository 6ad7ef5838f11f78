"""GPU parity of prod keys with m = d / 2 = 64 QJL rows at d = 128: the first
page's default proj_dim = head_dim / 2 (its compressor examples and its rule
of thumb for the projection dimension).  The estimator is the same with
kappa = sqrt(pi/2) / 64; the record holds, per 32-coordinate group, the index
words and then the group's sign word for the first two groups only.

Acceptance as for m = d: index and sign bits exact except within 1e-5 of a
boundary; scores within 1e-3 of each row's largest magnitude; attention
outputs within 1e-3 of each head's largest magnitude."""
import numpy as np
import pytest

import kv_cache_vector_02_amd as tq
from oracle import estimator as est
from oracle import packing as pk
from tests.gpu_util import Setup, compare_encode, torch
from tests.test_gpu_attend import check_heads, gpu_attend, oracle_value_cache
from tests.test_gpu_scores import check_ragged, check_rows, gpu_scores, long_pass_lengths, oracle_key_cache
from tq_inputs import gaussian_queries, kv_tensor, tiny_vectors

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def test_record_words():
    for bits, words in ((2, 6), (3, 10), (4, 14)):
        st = Setup(bits=bits, m=64, seed=40)
        assert tq.key_record_words(st.params) == words
        assert tq.key_record_words(Setup(bits=bits, seed=40).params) == 4 * bits


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("rot", ["dense", "hadamard"])
def test_encode(bits, rot):
    _log(f"m=64 encode b{bits} {rot}: 1500 fp32 vectors with outlier channels")
    x = tiny_vectors(1500, 128, seed=41)
    st = Setup(bits=bits, rot=rot, seed=41, m=64)
    planes, scal = st.encode_gpu(x)
    assert planes.shape == (1500, tq.key_record_words(st.params))
    _log(f"  {compare_encode(st, planes, scal, st.encode_oracle(x))}")


@pytest.mark.parametrize("n", [7, 2000])
def test_encode_f16_slots(n):
    _log(f"m=64 encode f16, {n} vectors through slots")
    x = kv_tensor(1, 1, n, 128, seed=42)[0, 0]
    st = Setup(bits=3, seed=42, m=64)
    slot = np.random.default_rng(42).permutation(n + 30)[:n]
    planes, scal = st.encode_gpu(x, slot=slot, records=n + 30)
    _log(f"  {compare_encode(st, planes[slot], scal[slot], st.encode_oracle(x.astype(np.float64)))}")


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("group", [1, 8, 16])
def test_scores(bits, group):
    _log(f"m=64 scores b{bits} G{group}")
    segs, T_ = 3, 1000
    x = kv_tensor(1, segs, T_, 128, seed=43)[0].reshape(-1, 128)
    st = Setup(bits=bits, seed=43, m=64)
    cache, (idx, z, n, g) = oracle_key_cache(st, x, seg_stride=T_)
    assert z.shape[1] == 64
    q = gaussian_queries(segs * group, 128, seed=43)
    length = [1000, 401, 0]
    got = gpu_scores(st, q, segs, group, cache, T_, length=length)
    worst = 0.0
    for s in range(segs):
        L = length[s]
        rows = slice(s * group, (s + 1) * group)
        if L:
            sl = slice(s * T_, s * T_ + L)
            ref = est.prod_scores(q[rows], idx[sl], z[sl], n[sl], g[sl], st.rot, st.s, st.c32)
            worst = max(worst, check_rows(got[rows, :L], ref))
        assert np.all(np.isnan(got[rows, L:]))
    _log(f"  worst rel {worst:.2e}")


def test_scores_hadamard_prepared_and_gpu_encode():
    # the two-phase form, on records the GPU encoded (compared with the
    # oracle's estimator on the oracle's reading of those same records)
    Tt = torch()
    _log("m=64 scores hadamard b3, GPU encode, prepare + prepared")
    x = kv_tensor(1, 2, 512, 128, seed=44)[0].reshape(-1, 128)
    st = Setup(bits=3, rot="hadamard", seed=44, m=64)
    cache = st.alloc(1024, seg_stride=512)
    tq.encode_prod(st.params, Tt.from_numpy(x).cuda(), cache)
    Tt.cuda.synchronize()
    idx, z, n, g = pk.unpack_key(cache.planes.cpu().numpy().view(np.uint32), cache.scalars.cpu().numpy(), 2, d=128)
    q = gaussian_queries(8, 128, seed=44)
    out = Tt.full((8, 512), float("nan"), dtype=Tt.float32, device="cuda")
    ws = tq.alloc_workspace(tq.scores_workspace(st.params, 2, 4))
    tq.scores_prepare(st.params, Tt.from_numpy(q).cuda(), 2, 4, ws)
    tq.scores_prepared(st.params, 2, 4, cache, 512, out, ws)
    Tt.cuda.synchronize()
    got = out.cpu().numpy()
    for s in range(2):
        sl = slice(512 * s, 512 * (s + 1))
        check_rows(got[4 * s:4 * s + 4], est.prod_scores(q[4 * s:4 * s + 4], idx[sl], z[sl], n[sl], g[sl],
                                                         st.rot, st.s, st.c32))


@pytest.mark.parametrize("bk,bv", [(3, 3), (2, 4), (4, 2)])
@pytest.mark.parametrize("group", [1, 8, 16])
def test_attend(bk, bv, group):
    _log(f"m=64 attend bk{bk} bv{bv} G{group}")
    segs, T_, stride = 3, 700, 704
    scale = 1 / np.sqrt(128)
    xk = kv_tensor(1, segs, stride, 128, seed=45)[0].reshape(-1, 128)
    xv = kv_tensor(1, segs, stride, 128, seed=45, value=True)[0].reshape(-1, 128)
    sk = Setup(bits=bk, seed=45, m=64)
    sv = Setup(bits=bv, prod=False, seed=45, purpose_pi=4, purpose_eps=6)
    kc, (kidx, kz, kn, kg) = oracle_key_cache(sk, xk, seg_stride=stride)
    vc, vidx, vn = oracle_value_cache(sv, xv, stride)
    q = gaussian_queries(segs * group, 128, seed=45)
    length = [700, 257, 0]
    got = gpu_attend(sk, sv, q, segs, group, kc, vc, T_, scale, length=length)
    worst = 0.0
    for s in range(segs):
        L = length[s]
        rows = slice(s * group, (s + 1) * group)
        if L == 0:
            assert np.all(got[rows] == 0.0)
            continue
        sl = slice(s * stride, s * stride + L)
        ref = est.attend(q[rows], (kidx[sl], kz[sl], kn[sl], kg[sl]), (vidx[sl], vn[sl]), sk.rot, sk.s, sk.c32,
                         sv.rot, sv.c32, scale)
        worst = max(worst, check_heads(got[rows], ref))
    _log(f"  worst rel {worst:.2e}")


def test_attend_hadamard():
    # sign-flipped Hadamard keys and values, m = 64
    _log("m=64 attend hadamard b3")
    segs, T_ = 2, 640
    scale = 1 / np.sqrt(128)
    xk = kv_tensor(1, segs, T_, 128, seed=46)[0].reshape(-1, 128)
    xv = kv_tensor(1, segs, T_, 128, seed=46, value=True)[0].reshape(-1, 128)
    sk = Setup(bits=3, rot="hadamard", seed=46, m=64)
    sv = Setup(bits=3, prod=False, rot="hadamard", seed=46, purpose_pi=4, purpose_eps=6)
    kc, (kidx, kz, kn, kg) = oracle_key_cache(sk, xk, seg_stride=T_)
    vc, vidx, vn = oracle_value_cache(sv, xv, T_)
    q = gaussian_queries(segs * 4, 128, seed=46)
    got = gpu_attend(sk, sv, q, segs, 4, kc, vc, T_, scale)
    for s in range(segs):
        sl = slice(s * T_, (s + 1) * T_)
        ref = est.attend(q[4 * s:4 * s + 4], (kidx[sl], kz[sl], kn[sl], kg[sl]), (vidx[sl], vn[sl]), sk.rot, sk.s,
                         sk.c32, sv.rot, sv.c32, scale)
        check_heads(got[4 * s:4 * s + 4], ref)


def test_qwen_shaped_full_size():
    # 36 layers x 2 KV heads x 8192 tokens, G = 8, b = 3, m = 64: the score
    # pass bench.py times, every segment in one launch; every token of every
    # segment against the oracle, to 1e-3 of the oracle's row maximum
    _log("m=64 scores qwen-shaped full size (every token)")
    L_, H_, T_ = 36, 2, 8192
    x = kv_tensor(L_, H_, T_, 128, seed=1).reshape(-1, 128)
    st = Setup(bits=3, seed=1, m=64)
    cache, (idx, z, n, g) = oracle_key_cache(st, x, seg_stride=T_)
    segs, group = L_ * H_, 8
    q = gaussian_queries(segs * group, 128, seed=1)
    got = gpu_scores(st, q, segs, group, cache, T_)
    worst = 0.0
    for s in range(segs):
        sl = slice(s * T_, (s + 1) * T_)
        rows = slice(s * group, (s + 1) * group)
        ref = est.prod_scores(q[rows], idx[sl], z[sl], n[sl], g[sl], st.rot, st.s, st.c32)
        worst = max(worst, check_rows(got[rows], ref))
    _log(f"  worst rel {worst:.2e}")


def test_long_pass_ragged_lengths():
    # prod b = 3 keys with m = 64 QJL rows through the 4-wave pass of a long
    # call (80 segments x 24576 tokens, G = 4) with ragged lengths, every valid
    # token against the oracle
    _log("m=64 scores: long pass, ragged lengths (80 x 24576 tokens)")
    segs, T_, G = 80, 24576, 4
    x = kv_tensor(1, segs, T_, 128, seed=19)[0].reshape(-1, 128)
    st = Setup(bits=3, seed=19, m=64)
    cache, (idx, z, n, g) = oracle_key_cache(st, x, seg_stride=T_)
    q = gaussian_queries(segs * G, 128, seed=19)
    ln = long_pass_lengths(segs, T_, 19)
    got = gpu_scores(st, q, segs, G, cache, T_, length=ln)
    ref = np.empty((segs * G, T_))
    for s in range(segs):
        sl = slice(s * T_, (s + 1) * T_)
        rows = slice(s * G, (s + 1) * G)
        ref[rows] = est.prod_scores(q[rows], idx[sl], z[sl], n[sl], g[sl], st.rot, st.s, st.c32)
    _log(f"  worst rel {check_ragged(got, ref, ln, G):.2e}")
