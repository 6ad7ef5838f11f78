"""GPU parity of tq_attend against the oracle on identical packed keys and
values, both made by the oracle's encoder and packing."""
import numpy as np
import pytest

import kv_cache_vector_02_amd as tq
from oracle import estimator as est
from oracle import packing as pk
from tests.gpu_util import Setup, compare_encode, torch
from tests.test_gpu_scores import oracle_key_cache
from tq_inputs import gaussian_queries, kv_tensor

pytestmark = pytest.mark.gpu
REL_TOL = 1e-3


def _log(msg):
    print(msg, flush=True)


def oracle_value_cache(st: Setup, x, seg_stride):
    """Oracle-encoded values in the block layout -> (device Cache, idx, n)."""
    T = torch()
    code = st.encode_oracle(x)
    n16 = code.n.astype(np.float16)
    words = pk.pack_value_blocks(code.idx, st.bq)
    cache = tq.Cache(T.from_numpy(words.view(np.int32)).cuda(), T.from_numpy(n16[:, None]).cuda(), seg_stride)
    return cache, code.idx, n16.astype(np.float64)


def gpu_attend(sk, sv, q, segs, group, kc, vc, T_, scale, length=None):
    Tt = torch()
    qd = Tt.from_numpy(np.ascontiguousarray(q, np.float32)).cuda()
    out = Tt.full((segs * group, 128), float("nan"), dtype=Tt.float32, device="cuda")
    ws = Tt.zeros(tq.attend_workspace(sk.params, sv.params, segs, group, T_), dtype=Tt.uint8, device="cuda")
    ln = None if length is None else Tt.from_numpy(np.asarray(length, np.int32)).cuda()
    tq.attend(sk.params, sv.params, qd, segs, group, kc, vc, T_, scale, out, ws, length=ln)
    Tt.cuda.synchronize()
    return out.cpu().numpy()


def oracle_attend(sk, sv, q, kf, vidx, vn, sl, scale):
    idx, z, n, g = kf
    return est.attend(q, (idx[sl], z[sl], n[sl], g[sl]), (vidx[sl], vn[sl]), sk.rot, sk.s, sk.c32,
                      sv.rot, sv.c32, scale)


def check_heads(got, ref):
    """||got_h - ref_h||_inf <= 1e-3 ||ref_h||_inf for every head."""
    err = np.max(np.abs(got - ref), axis=1)
    scale = np.max(np.abs(ref), axis=1)
    worst = float(np.max(err / np.maximum(scale, 1e-30)))
    assert np.all(err <= REL_TOL * scale + 1e-30), f"worst relative head error {worst:.3e}"
    return worst


def _setups(bk, bv, rot="dense", seed=5):
    sk = Setup(bits=bk, prod=True, seed=seed, rot=rot)
    sv = Setup(bits=bv, prod=False, seed=seed, rot=rot, purpose_pi=4, purpose_eps=6)
    return sk, sv


@pytest.mark.parametrize("bk,bv", [(3, 3), (2, 2), (4, 3), (3, 1), (2, 3), (4, 4), (2, 4)])
@pytest.mark.parametrize("group", [1, 4, 8, 16])
def test_segments_groups_bits_lengths(bk, bv, group):
    _log(f"attend bk{bk} bv{bv} G{group}")
    segs, T_, stride = 3, 1000, 1024
    sk, sv = _setups(bk, bv)
    xk = kv_tensor(1, segs, stride, 128, seed=5)[0].reshape(-1, 128)
    xv = kv_tensor(1, segs, stride, 128, seed=5, value=True)[0].reshape(-1, 128)
    kc, kf = oracle_key_cache(sk, xk, seg_stride=stride)
    vc, vidx, vn = oracle_value_cache(sv, xv, stride)
    q = gaussian_queries(segs * group, 128, seed=5)
    length = [1000, 517, 0]
    scale = 1 / np.sqrt(128)
    got = gpu_attend(sk, sv, q, segs, group, kc, vc, T_, scale, length=length)
    for s in range(segs):
        rows = slice(s * group, (s + 1) * group)
        L = length[s]
        if L == 0:
            assert np.all(got[rows] == 0.0), "an empty segment gives zeros"
            continue
        sl = slice(s * stride, s * stride + L)
        ref = oracle_attend(sk, sv, q[rows], kf, vidx, vn, sl, scale)
        check_heads(got[rows], ref)


@pytest.mark.parametrize("scale", [1.0, 1 / np.sqrt(128), 0.0])
def test_temperatures(scale):
    _log(f"attend scale {scale}")
    segs, T_ = 2, 700
    stride = 704
    sk, sv = _setups(3, 3, seed=6)
    xk = kv_tensor(1, segs, stride, 128, seed=6)[0].reshape(-1, 128)
    xv = kv_tensor(1, segs, stride, 128, seed=6, value=True)[0].reshape(-1, 128)
    kc, kf = oracle_key_cache(sk, xk, seg_stride=stride)
    vc, vidx, vn = oracle_value_cache(sv, xv, stride)
    q = gaussian_queries(segs * 8, 128, seed=6)
    got = gpu_attend(sk, sv, q, segs, 8, kc, vc, T_, scale)
    for s in range(segs):
        sl = slice(s * stride, s * stride + T_)
        check_heads(got[s * 8:(s + 1) * 8], oracle_attend(sk, sv, q[s * 8:(s + 1) * 8], kf, vidx, vn, sl, scale))


def test_hadamard_rotations():
    # sign-flipped Hadamard on keys and values (query prep and the final
    # inverse rotation take the Hadamard paths)
    _log("attend hadamard")
    segs, T_ = 2, 640
    sk, sv = _setups(3, 3, rot="hadamard", seed=7)
    xk = kv_tensor(1, segs, T_, 128, seed=7)[0].reshape(-1, 128)
    xv = kv_tensor(1, segs, T_, 128, seed=7, value=True)[0].reshape(-1, 128)
    kc, kf = oracle_key_cache(sk, xk, seg_stride=T_)
    vc, vidx, vn = oracle_value_cache(sv, xv, T_)
    q = gaussian_queries(segs * 4, 128, seed=7)
    got = gpu_attend(sk, sv, q, segs, 4, kc, vc, T_, 1 / np.sqrt(128))
    for s in range(segs):
        sl = slice(s * T_, (s + 1) * T_)
        check_heads(got[s * 4:(s + 1) * 4],
                    oracle_attend(sk, sv, q[s * 4:(s + 1) * 4], kf, vidx, vn, sl, 1 / np.sqrt(128)))


@pytest.mark.parametrize("rot,group", [("dense", 1), ("dense", 4), ("dense", 8), ("dense", 16), ("hadamard", 4)])
def test_single_workgroup_segments(rot, group):
    # T <= 512: one workgroup per segment, which normalises its heads and
    # applies the inverse value rotation itself (no combine launch); lengths
    # include a full segment, a ragged one, an empty one and a single token
    _log(f"attend, one workgroup per segment, {rot} G{group}")
    segs, T_, stride = 4, 512, 512
    sk, sv = _setups(3, 3, rot=rot, seed=9)
    xk = kv_tensor(1, segs, stride, 128, seed=9)[0].reshape(-1, 128)
    xv = kv_tensor(1, segs, stride, 128, seed=9, value=True)[0].reshape(-1, 128)
    kc, kf = oracle_key_cache(sk, xk, seg_stride=stride)
    vc, vidx, vn = oracle_value_cache(sv, xv, stride)
    q = gaussian_queries(segs * group, 128, seed=9)
    length = [512, 300, 0, 1]
    scale = 1 / np.sqrt(128)
    got = gpu_attend(sk, sv, q, segs, group, kc, vc, T_, scale, length=length)
    for s in range(segs):
        rows = slice(s * group, (s + 1) * group)
        if length[s] == 0:
            assert np.all(got[rows] == 0.0), "an empty segment gives zeros"
            continue
        sl = slice(s * stride, s * stride + length[s])
        check_heads(got[rows], oracle_attend(sk, sv, q[rows], kf, vidx, vn, sl, scale))


def test_many_segments_one_workgroup_each():
    # more segments than the device holds workgroups at once: each 768-token
    # segment gets a single workgroup (the batched-decode launch shape);
    # sampled segments against the oracle
    _log("attend, 1024 segments x 768 tokens, one workgroup each")
    segs, T_, group = 1024, 768, 4
    sk, sv = _setups(3, 3, seed=10)
    xk = kv_tensor(1, segs, T_, 128, seed=10)[0].reshape(-1, 128)
    xv = kv_tensor(1, segs, T_, 128, seed=10, value=True)[0].reshape(-1, 128)
    kc, kf = oracle_key_cache(sk, xk, seg_stride=T_)
    vc, vidx, vn = oracle_value_cache(sv, xv, T_)
    q = gaussian_queries(segs * group, 128, seed=10)
    scale = 1 / np.sqrt(128)
    got = gpu_attend(sk, sv, q, segs, group, kc, vc, T_, scale)
    for s in [0, 1, 511, 777, 1023]:
        rows = slice(s * group, (s + 1) * group)
        sl = slice(s * T_, (s + 1) * T_)
        check_heads(got[rows], oracle_attend(sk, sv, q[rows], kf, vidx, vn, sl, scale))


@pytest.mark.parametrize("T_", [512, 1500])
def test_prepare_then_prepared_equals_attend(T_):
    # tq_attend_prepare on a second stream, then tq_attend_prepared twice on
    # the pack (one workgroup per segment at T = 512, several at 1500): both
    # equal tq_attend bit for bit
    _log(f"attend prepare / prepared, T = {T_}")
    Tt = torch()
    segs, group = 3, 4
    sk, sv = _setups(3, 3, seed=11)
    xk = kv_tensor(1, segs, T_, 128, seed=11)[0].reshape(-1, 128)
    xv = kv_tensor(1, segs, (T_ + 31) // 32 * 32, 128, seed=11, value=True)[0].reshape(-1, 128)
    kc, _ = oracle_key_cache(sk, xk, seg_stride=T_)
    vc, _, _ = oracle_value_cache(sv, xv, (T_ + 31) // 32 * 32)
    q = Tt.from_numpy(gaussian_queries(segs * group, 128, seed=11)).cuda()
    scale = 1 / np.sqrt(128)
    ref = gpu_attend(sk, sv, q.cpu().numpy(), segs, group, kc, vc, T_, scale)
    ws = Tt.zeros(tq.attend_workspace(sk.params, sv.params, segs, group, T_), dtype=Tt.uint8, device="cuda")
    side = Tt.cuda.Stream()
    side.wait_stream(Tt.cuda.current_stream())
    tq.attend_prepare(sk.params, q, segs, group, ws, stream=side)
    Tt.cuda.current_stream().wait_stream(side)
    for _ in range(2):
        out = Tt.full((segs * group, 128), float("nan"), dtype=Tt.float32, device="cuda")
        tq.attend_prepared(sk.params, sv.params, segs, group, kc, vc, T_, scale, out, ws)
        Tt.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref)


def test_qwen_shaped_full_size():
    # 36 layers x 2 KV heads x 8192 tokens, 16 query heads per layer (G=8),
    # keys prod b=3, values mse b=3, one launch; every segment against the oracle
    _log("attend qwen-shaped full size (every segment)")
    L_, H_, T_ = 36, 2, 8192
    sk, sv = _setups(3, 3, seed=1)
    xk = kv_tensor(L_, H_, T_, 128, seed=1).reshape(-1, 128)
    xv = kv_tensor(L_, H_, T_, 128, seed=1, value=True).reshape(-1, 128)
    kc, kf = oracle_key_cache(sk, xk, seg_stride=T_)
    vc, vidx, vn = oracle_value_cache(sv, xv, T_)
    segs, group = L_ * H_, 8
    q = gaussian_queries(segs * group, 128, seed=1)
    scale = 1 / np.sqrt(128)
    got = gpu_attend(sk, sv, q, segs, group, kc, vc, T_, scale)
    worst = 0.0
    for s in range(segs):
        sl = slice(s * T_, (s + 1) * T_)
        rows = slice(s * group, (s + 1) * group)
        worst = max(worst, check_heads(got[rows], oracle_attend(sk, sv, q[rows], kf, vidx, vn, sl, scale)))
    _log(f"  worst rel {worst:.2e}")


def _flip_allowance(sk, sv, q, kcode, vcode, scale, k_idx, k_z, v_idx):
    """Per head, how far the output may move because the encoder took the
    other side of a decision inside the 1e-5 band (the encode tests'
    allowance), to first order in the softmax.  k_idx / k_z / v_idx are the
    encoder's key indices, key signs and value indices; where they differ from
    the oracle's (each such coordinate is first checked to lie in the band),
    the oracle re-encodes that record with the encoder's decision and takes
    the change it makes:
      value (t, j): o moves by at most p_t n_t |c_v[idx'] - c_v[idx]| max_i |Pi_v^T[i, j]|
      key t: its score moves by delta_t = |s'(q, t) - s(q, t)| (neighbouring
      cell: new residual, gamma and signs from the oracle; a flipped sign: that
      sign), so o moves by at most |scale| p_t delta_t ||v_t - o||_inf."""
    band = 1e-5
    ck = np.asarray(sk.c32, np.float64)
    cv = np.asarray(sv.c32, np.float64)
    smat = np.asarray(sk.s, np.float64)
    kn = kcode.n.astype(np.float16).astype(np.float64)
    kg = kcode.gamma.astype(np.float16).astype(np.float64)
    vn = vcode.n.astype(np.float16).astype(np.float64)
    s = est.prod_scores(q, kcode.idx, kcode.z, kn, kg, sk.rot, sk.s, sk.c32)
    a = scale * s
    p = np.exp(a - a.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    v = est.dequantize(vcode.idx, vn, sv.rot, sv.c32)
    o = p @ v
    q_rot, q_proj = est.prepare_query(q, sk.rot, sk.s)
    kap = est.kappa(sk.m)
    bound = np.zeros(q.shape[0])
    # the inverse value rotation's largest entry per rotated coordinate
    spread = np.max(np.abs(sv.rot.inverse(np.eye(sv.d_rot))), axis=1)
    for t, j in zip(*np.nonzero(v_idx != vcode.idx)):
        assert np.min(np.abs(vcode.y[t, j] - np.asarray(sv.b32, np.float64))) < band
        bound += p[:, t] * vn[t] * abs(cv[v_idx[t, j]] - cv[vcode.idx[t, j]]) * spread[j]
    for t in np.nonzero(np.any(k_idx != kcode.idx, axis=1) | np.any(k_z != kcode.z, axis=1))[0]:
        if np.any(k_idx[t] != kcode.idx[t]):
            alt = k_idx[t]
            r = kcode.y[t] - ck[alt]
            g = np.float64(np.float16(np.sqrt(r @ r)))
            z = (smat @ r) >= 0
        else:
            alt, g, z = kcode.idx[t], kg[t], k_z[t]
        s_alt = kn[t] * (q_rot @ ck[alt] + g * kap * (q_proj @ (2.0 * z - 1.0)))
        bound += abs(scale) * p[:, t] * np.abs(s_alt - s[:, t]) * np.max(np.abs(v[t][None, :] - o), axis=1)
    return 2.0 * bound


def test_end_to_end_gpu_encode_then_attend():
    # GPU encode + GPU attend against oracle encode + oracle attend.  The
    # encoder may take the other side of a decision within 1e-5 of a boundary
    # (checked record by record first); the tolerance is 1e-3 of the head's
    # largest output magnitude plus the oracle's bound on what those decisions
    # move (zero when the encodes agree bit for bit).
    _log("attend end to end")
    Tt = torch()
    segs, T_ = 2, 1024
    sk, sv = _setups(3, 3, seed=8)
    xk = kv_tensor(1, segs, T_, 128, seed=8)[0].reshape(-1, 128)
    xv = kv_tensor(1, segs, T_, 128, seed=8, value=True)[0].reshape(-1, 128)
    kc = tq.alloc_cache(sk.layout(), segs * T_, seg_stride=T_)
    vc = tq.alloc_value_cache(sv.layout(), segs * T_, seg_stride=T_)
    tq.encode_prod(sk.params, Tt.from_numpy(xk).cuda(), kc)
    tq.encode_mse(sv.params, Tt.from_numpy(xv).cuda(), vc)
    q = gaussian_queries(segs * 8, 128, seed=8)
    scale = 1 / np.sqrt(128)
    got = gpu_attend(sk, sv, q, segs, 8, kc, vc, T_, scale)
    kcode = sk.encode_oracle(xk)
    vcode = sv.encode_oracle(xv)
    kplanes, kscal = kc.planes.cpu().numpy().view(np.uint32), kc.scalars.cpu().numpy()
    vidx_gpu = pk.unpack_value_blocks(vc.planes.cpu().numpy().view(np.uint32), segs * T_)
    ks = compare_encode(sk, kplanes, kscal, kcode)
    vs = compare_encode(sv, vidx_gpu, vc.scalars.cpu().numpy(), vcode)
    _log(f"  encode flips: keys {ks}, values {vs}")
    kidx_gpu, kz_gpu, _, _ = pk.unpack_key(kplanes, kscal, sk.bq, d=128)
    kf = (kcode.idx, kcode.z, kcode.n.astype(np.float16).astype(np.float64),
          kcode.gamma.astype(np.float16).astype(np.float64))
    vn = vcode.n.astype(np.float16).astype(np.float64)
    for s in range(segs):
        sl = slice(s * T_, (s + 1) * T_)
        rows = slice(s * 8, (s + 1) * 8)
        ref = oracle_attend(sk, sv, q[rows], kf, vcode.idx, vn, sl, scale)
        sub_k = type(kcode)(idx=kcode.idx[sl], z=kcode.z[sl], n=kcode.n[sl], gamma=kcode.gamma[sl],
                            y=kcode.y[sl], proj=kcode.proj[sl])
        sub_v = type(vcode)(idx=vcode.idx[sl], n=vcode.n[sl], y=vcode.y[sl])
        extra = _flip_allowance(sk, sv, q[rows], sub_k, sub_v, scale, kidx_gpu[sl], kz_gpu[sl], vidx_gpu[sl])
        err = np.max(np.abs(got[rows] - ref), axis=1)
        top = np.max(np.abs(ref), axis=1)
        _log(f"  segment {s}: worst rel {np.max(err / top):.2e}; flip allowance up to "
             f"{np.max(extra / top):.2e} of the head's maximum")
        assert np.all(err <= REL_TOL * top + extra)


def smoke_attend():
    """Used by the smoke check: one small attend call against the oracle."""
    segs, T_ = 1, 300
    sk, sv = _setups(3, 3, seed=9)
    xk = kv_tensor(1, 1, 320, 128, seed=9)[0, 0]
    xv = kv_tensor(1, 1, 320, 128, seed=9, value=True)[0, 0]
    kc, kf = oracle_key_cache(sk, xk, seg_stride=320)
    vc, vidx, vn = oracle_value_cache(sv, xv, 320)
    q = gaussian_queries(8, 128, seed=9)
    got = gpu_attend(sk, sv, q, 1, 8, kc, vc, T_, 1 / np.sqrt(128))
    ref = oracle_attend(sk, sv, q, kf, vidx, vn, slice(0, T_), 1 / np.sqrt(128))
    print(f"smoke attend ok, worst rel {check_heads(got, ref):.2e}", flush=True)
