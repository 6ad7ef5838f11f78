"""GPU parity of MSE-only keys at d = 128: TurboQuant-MSE applied to keys, with
no QJL stage (blog notes on the paper, Q_mse; explainer page section 8, whose
QJL stage exists to remove the bias this estimator keeps).

* tq_encode_mse_keys: b index bits per coordinate in the per-record key
  layout, one fp16 norm, against the oracle's MSE encoder (indices exact
  except within 1e-5 of a boundary; norms exact except at an fp16 midpoint).
* tq_scores with a key quantizer that has no QJL matrix: the biased MSE
  inner product n <Pi q, c[idx]>, against the oracle's mse_scores on
  oracle-packed records, to 1e-3 of each row's largest magnitude.
* tq_attend with MSE-only keys: softmax of those scores over MSE values,
  against the oracle, to 1e-3 of each head's largest output magnitude."""
import numpy as np
import pytest

import kv_cache_vector_02_amd as tq
from oracle import estimator as est
from oracle import packing as pk
from tests.gpu_util import Setup, compare_encode, torch
from tests.test_gpu_attend import check_heads, gpu_attend, oracle_value_cache
from tests.test_gpu_scores import check_ragged, check_rows, gpu_scores, long_pass_lengths
from tq_inputs import gaussian_queries, kv_tensor, tiny_vectors

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _setup(bits, rot="dense", seed=0):
    # a key quantizer without a QJL matrix (the keys' rotation stream)
    return Setup(bits=bits, prod=False, rot=rot, seed=seed)


def gpu_encode_keys(st, x, slot=None, records=None):
    T = torch()
    xd = x if hasattr(x, "data_ptr") else T.from_numpy(np.ascontiguousarray(x)).cuda()
    n = xd.shape[0]
    cache = tq.alloc_cache(tq.key_layout(st.params), records or n)
    sl = None if slot is None else T.from_numpy(np.asarray(slot, np.int64)).cuda()
    tq.encode_mse_keys(st.params, xd, cache, slot=sl)
    T.cuda.synchronize()
    return cache.planes.cpu().numpy().view(np.uint32), cache.scalars.cpu().numpy()


def oracle_mse_key_cache(st, x, seg_stride):
    """Oracle-encoded MSE records in the key layout -> (device Cache, idx, n)."""
    T = torch()
    code = st.encode_oracle(x)
    n16 = code.n.astype(np.float16)
    code.n = n16.astype(np.float64)
    planes, scal = pk.pack_value(code, st.bq)
    cache = tq.Cache(T.from_numpy(planes.view(np.int32)).cuda(), T.from_numpy(scal).cuda(), seg_stride)
    return cache, code.idx, code.n


def test_layout():
    st = _setup(3)
    assert tq.key_layout(st.params) == (3, 4, 1)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("rot", ["dense", "hadamard"])
def test_encode(bits, rot):
    _log(f"mse keys encode b{bits} {rot}: 2000 fp32 vectors with outlier channels")
    x = tiny_vectors(2000, 128, seed=21)
    st = _setup(bits, rot=rot, seed=21)
    planes, scal = gpu_encode_keys(st, x)
    assert planes.shape == (2000, 4, bits) and scal.shape == (2000, 1)
    idx = pk.unpack_value(planes, scal, bits)[0]
    _log(f"  {compare_encode(st, idx, scal, st.encode_oracle(x))}")


@pytest.mark.parametrize("n", [5, 1000])
def test_encode_f16_slots(n):
    # float16 rows with a row stride, records scattered through a slot map;
    # n = 5 takes the one-wave launch shape
    T = torch()
    _log(f"mse keys encode f16, {n} vectors through slots")
    x = kv_tensor(1, 1, n, 128, seed=22)[0, 0]
    st = _setup(4, seed=22)
    wide = T.zeros((n, 192), dtype=T.float16, device="cuda")
    wide[:, :128] = T.from_numpy(x).cuda()
    slot = np.random.default_rng(22).permutation(n + 40)[:n]
    planes, scal = gpu_encode_keys(st, wide[:, :128], slot=slot, records=n + 40)
    idx = pk.unpack_value(planes[slot], scal[slot], 4)[0]
    _log(f"  {compare_encode(st, idx, scal[slot], st.encode_oracle(x.astype(np.float64)))}")


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("group", [1, 8, 16])
def test_scores(bits, group):
    _log(f"mse keys scores b{bits} G{group}")
    segs, T_ = 3, 1000
    x = kv_tensor(1, segs, T_, 128, seed=23)[0].reshape(-1, 128)
    st = _setup(bits, seed=23)
    cache, idx, n = oracle_mse_key_cache(st, x, T_)
    q = gaussian_queries(segs * group, 128, seed=23)
    length = [1000, 333, 0]
    got = gpu_scores(st, q, segs, group, cache, T_, length=length)
    worst = 0.0
    for s in range(segs):
        L = length[s]
        rows = slice(s * group, (s + 1) * group)
        if L:
            sl = slice(s * T_, s * T_ + L)
            worst = max(worst, check_rows(got[rows, :L], est.mse_scores(q[rows], idx[sl], n[sl], st.rot, st.c32)))
        assert np.all(np.isnan(got[rows, L:])), "entries past len are not written"
    _log(f"  worst rel {worst:.2e}")


@pytest.mark.parametrize("bits", [2, 4])
def test_scores_hadamard_prepared(bits):
    # the two-phase form on Hadamard-rotated keys
    Tt = torch()
    _log(f"mse keys scores hadamard b{bits}, prepare + prepared")
    x = kv_tensor(1, 2, 640, 128, seed=24)[0].reshape(-1, 128)
    st = _setup(bits, rot="hadamard", seed=24)
    cache, idx, n = oracle_mse_key_cache(st, x, 640)
    q = gaussian_queries(8, 128, seed=24)
    qd = Tt.from_numpy(q).cuda()
    out = Tt.full((8, 640), float("nan"), dtype=Tt.float32, device="cuda")
    ws = tq.alloc_workspace(tq.scores_workspace(st.params, 2, 4))
    tq.scores_prepare(st.params, qd, 2, 4, ws)
    tq.scores_prepared(st.params, 2, 4, cache, 640, out, ws)
    Tt.cuda.synchronize()
    got = out.cpu().numpy()
    for s in range(2):
        sl = slice(s * 640, (s + 1) * 640)
        check_rows(got[4 * s:4 * s + 4], est.mse_scores(q[4 * s:4 * s + 4], idx[sl], n[sl], st.rot, st.c32))


@pytest.mark.parametrize("bk,bv", [(2, 2), (3, 3), (4, 4), (2, 4), (4, 2), (3, 2)])
@pytest.mark.parametrize("group", [1, 8, 12, 16])
def test_attend(bk, bv, group):
    # 4-bit keys with more than 8 heads run as two halves of the segment's heads
    _log(f"mse keys attend bk{bk} bv{bv} G{group}")
    segs, T_, stride = 3, 700, 704
    scale = 1 / np.sqrt(128)
    xk = kv_tensor(1, segs, stride, 128, seed=25)[0].reshape(-1, 128)
    xv = kv_tensor(1, segs, stride, 128, seed=25, value=True)[0].reshape(-1, 128)
    sk = _setup(bk, seed=25)
    sv = Setup(bits=bv, prod=False, seed=25, purpose_pi=4, purpose_eps=6)
    kc, kidx, kn = oracle_mse_key_cache(sk, xk, stride)
    vc, vidx, vn = oracle_value_cache(sv, xv, stride)
    q = gaussian_queries(segs * group, 128, seed=25)
    length = [700, 129, 0]
    got = gpu_attend(sk, sv, q, segs, group, kc, vc, T_, scale, length=length)
    worst = 0.0
    for s in range(segs):
        L = length[s]
        rows = slice(s * group, (s + 1) * group)
        if L == 0:
            assert np.all(got[rows] == 0.0)
            continue
        sl = slice(s * stride, s * stride + L)
        scores = est.mse_scores(q[rows], kidx[sl], kn[sl], sk.rot, sk.c32)
        ref = est.softmax_weighted_sum(scores, est.dequantize(vidx[sl], vn[sl], sv.rot, sv.c32), scale)
        worst = max(worst, check_heads(got[rows], ref))
    _log(f"  worst rel {worst:.2e}")


def test_attend_4bit_keys_reject_odd_groups_over_8():
    sk = _setup(4, seed=26)
    sv = Setup(bits=3, prod=False, seed=26, purpose_pi=4, purpose_eps=6)
    T = torch()
    q = T.zeros((15, 128), dtype=T.float32, device="cuda")
    kc = tq.alloc_cache(tq.key_layout(sk.params), 64)
    vc = tq.alloc_value_cache(tq.value_layout(sv.params), 64)
    out = T.zeros((15, 128), dtype=T.float32, device="cuda")
    ws = tq.alloc_workspace(tq.attend_workspace(sk.params, sv.params, 1, 15, 64))
    with pytest.raises(tq.TQError, match="UNSUPPORTED"):
        tq.attend(sk.params, sv.params, q, 1, 15, kc, vc, 64, 1.0, out, ws)


def test_qwen_shaped_full_size():
    # 36 layers x 2 KV heads x 8192 tokens, G = 8, MSE-only b = 3 keys: the
    # score pass bench.py times, every segment in one launch; every token of
    # every segment against the oracle, to 1e-3 of the oracle's row maximum
    _log("mse keys scores qwen-shaped full size (every token)")
    L_, H_, T_ = 36, 2, 8192
    x = kv_tensor(L_, H_, T_, 128, seed=1).reshape(-1, 128)
    st = _setup(3, seed=1)
    cache, idx, n = oracle_mse_key_cache(st, x, T_)
    segs, group = L_ * H_, 8
    q = gaussian_queries(segs * group, 128, seed=1)
    got = gpu_scores(st, q, segs, group, cache, T_)
    worst = 0.0
    for s in range(segs):
        sl = slice(s * T_, (s + 1) * T_)
        rows = slice(s * group, (s + 1) * group)
        worst = max(worst, check_rows(got[rows], est.mse_scores(q[rows], idx[sl], n[sl], st.rot, st.c32)))
    _log(f"  worst rel {worst:.2e}")


def test_long_pass_ragged_lengths():
    # MSE-only b = 3 keys through the 4-wave pass of a long call (80 segments
    # x 24576 tokens, G = 8) with ragged lengths, every valid token against the
    # oracle's MSE inner product
    _log("mse keys scores: long pass, ragged lengths (80 x 24576 tokens)")
    segs, T_, G = 80, 24576, 8
    x = kv_tensor(1, segs, T_, 128, seed=18)[0].reshape(-1, 128)
    st = _setup(3, seed=18)
    cache, idx, n = oracle_mse_key_cache(st, x, T_)
    q = gaussian_queries(segs * G, 128, seed=18)
    ln = long_pass_lengths(segs, T_, 18)
    got = gpu_scores(st, q, segs, G, cache, T_, length=ln)
    ref = np.empty((segs * G, T_))
    for s in range(segs):
        sl = slice(s * T_, (s + 1) * T_)
        rows = slice(s * G, (s + 1) * G)
        ref[rows] = est.mse_scores(q[rows], idx[sl], n[sl], st.rot, st.c32)
    _log(f"  worst rel {check_ragged(got, ref, ln, G):.2e}")
