"""Full-size parity of the Llama-3.1-8B-shaped cache (32 layers x 8 KV heads x
32768 tokens x 128, fp16; GQA 4) and of batched streaming decode (64 sequences x
8 KV heads x 8192 tokens, 64 new tokens x 8 heads appended per step), each in
the launch configuration a real call uses: every segment in one launch.

The oracle never reads a GPU output: the checked segments of a cache are
filled with oracle-encoded, oracle-packed records before the GPU scores or
attends over the whole cache (the other segments hold GPU-encoded records,
which only feed unchecked outputs), and the encoder is checked on a seeded
sample of rows against the oracle's own encoding."""
import numpy as np
import pytest

import kv_cache_vector_02_amd as tq
from oracle import estimator as est
from oracle import packing as pk
from tests.gpu_util import Setup, compare_encode, torch
from tests.test_gpu_attend import check_heads
from tests.test_gpu_scores import check_rows
from tq_inputs import gaussian_queries, kv_tensor

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _setups(bits, rot, seed):
    sk = Setup(bits=bits, prod=True, seed=seed, rot=rot)
    sv = Setup(bits=bits, prod=False, seed=seed, rot=rot, purpose_pi=4, purpose_eps=6)
    return sk, sv


def _oracle_segment(sk, sv, xk, xv):
    """Oracle code of one segment's keys and values, stored (float16) norms."""
    kc = sk.encode_oracle(xk)
    kc.n = kc.n.astype(np.float16).astype(np.float64)
    kc.gamma = kc.gamma.astype(np.float16).astype(np.float64)
    vc = sv.encode_oracle(xv)
    vc.n = vc.n.astype(np.float16).astype(np.float64)
    return kc, vc


def _plant(sk, sv, kcache, vcache, seg, stride, kc, vc):
    """Write an oracle-packed segment into the device caches (records seg*stride..)."""
    T = torch()
    planes, scal = pk.pack_key(kc, sk.bq)                       # [n, W, P], [n, 2]
    r0 = seg * stride
    kcache.planes[r0:r0 + len(planes)] = T.from_numpy(planes.view(np.int32)).cuda()
    kcache.scalars[r0:r0 + len(planes)] = T.from_numpy(scal).cuda()
    words = pk.pack_value_blocks(vc.idx, sv.bq)                 # [nb, d, bits]
    vcache.planes[r0 // 32:r0 // 32 + words.shape[0]] = T.from_numpy(words.view(np.int32)).cuda()
    vcache.scalars[r0:r0 + len(vc.n)] = T.from_numpy(vc.n.astype(np.float16)[:, None]).cuda()


def _value_rows(vcache, rows):
    """Indices of the given value records from the device block words."""
    rows = np.asarray(rows, np.int64)
    words = vcache.planes[torch().from_numpy(rows // 32).cuda()].cpu().numpy().view(np.uint32)  # [n, d, P]
    bit = (rows % 32).astype(np.uint32)[:, None, None]
    bits = (words >> bit) & 1
    return (bits.astype(np.int64) << np.arange(words.shape[2])[None, None, :]).sum(axis=2)


def _oracle_attend(sk, sv, q, kc, vc, scale):
    return est.attend(q, (kc.idx, kc.z, kc.n, kc.gamma), (vc.idx, vc.n), sk.rot, sk.s, sk.c32, sv.rot,
                      sv.c32, scale)


@pytest.fixture(scope="module")
def llama_kv():
    L, H, T_ = 32, 8, 32768
    _log("generating the llama-shaped cache inputs (2 x 2.1 GB fp16)")
    k = kv_tensor(L, H, T_, 128, seed=2).reshape(-1, 128)
    v = kv_tensor(L, H, T_, 128, seed=2, value=True).reshape(-1, 128)
    return k, v


def _llama_full_launch(llama_kv, bits, rot):
    """GPU encode of the whole Llama-shaped cache at `bits`, then tq_scores and
    tq_attend over all 256 segments in one launch each (the launch shape a
    real call takes, with the span split of the full grid).  Six segments,
    at both ends of the grid and inside it, hold oracle-packed records; every
    token of those is checked against the oracle."""
    Tt = torch()
    k, v = llama_kv
    L, H, T_, G = 32, 8, 32768, 4
    segs = L * H
    sk, sv = _setups(bits, rot, seed=2)
    _log(f"llama-shaped b{bits} {rot}: encode {k.shape[0]} keys and values")
    kx = Tt.from_numpy(k).cuda()
    vx = Tt.from_numpy(v).cuda()
    kcache = sk.alloc(segs * T_, seg_stride=T_)
    vcache = sv.alloc(segs * T_, seg_stride=T_)
    tq.encode_prod(sk.params, kx, kcache)
    tq.encode_mse(sv.params, vx, vcache)
    Tt.cuda.synchronize()
    del kx, vx
    # encoder: a seeded sample of rows against the oracle
    rg = np.random.default_rng(7 + bits)
    sample = np.sort(rg.choice(k.shape[0], 2000, replace=False))
    sample[-1] = k.shape[0] - 1
    si = Tt.from_numpy(sample).cuda()
    _log(f"  keys {compare_encode(sk, kcache.planes[si].cpu().numpy().view(np.uint32), kcache.scalars[si].cpu().numpy(), sk.encode_oracle(k[sample]))}")
    _log(f"  values {compare_encode(sv, _value_rows(vcache, sample), vcache.scalars[si].cpu().numpy(), sv.encode_oracle(v[sample]))}")
    checked = sorted({0, 1, int(rg.integers(2, segs - 2)), segs // 2, segs - 2, segs - 1})
    codes = {}
    for s in checked:
        sl = slice(s * T_, (s + 1) * T_)
        codes[s] = _oracle_segment(sk, sv, k[sl], v[sl])
        _plant(sk, sv, kcache, vcache, s, T_, *codes[s])
    q = gaussian_queries(segs * G, 128, seed=2)
    qd = Tt.from_numpy(q).cuda()
    out = Tt.full((segs * G, T_), float("nan"), dtype=Tt.float32, device="cuda")
    ws = tq.alloc_workspace(tq.scores_workspace(sk.params, segs, G))
    tq.scores(sk.params, qd, segs, G, kcache, T_, out, ws)
    o = Tt.full((segs * G, 128), float("nan"), dtype=Tt.float32, device="cuda")
    wa = tq.alloc_workspace(tq.attend_workspace(sk.params, sv.params, segs, G, T_))
    scale = 1 / np.sqrt(128)
    tq.attend(sk.params, sv.params, qd, segs, G, kcache, vcache, T_, scale, o, wa)
    Tt.cuda.synchronize()
    for s in checked:
        kc, vc = codes[s]
        rows = slice(s * G, (s + 1) * G)
        ref = est.prod_scores(q[rows], kc.idx, kc.z, kc.n, kc.gamma, sk.rot, sk.s, sk.c32)
        ws_ = check_rows(out[rows].cpu().numpy(), ref)
        wa_ = check_heads(o[rows].cpu().numpy(), _oracle_attend(sk, sv, q[rows], kc, vc, scale))
        _log(f"  segment {s}: scores worst rel {ws_:.2e}, attend worst rel {wa_:.2e}")
    assert np.isfinite(out.cpu().numpy()).all() and np.isfinite(o.cpu().numpy()).all()


@pytest.mark.parametrize("rot", ["dense", "hadamard"])
def test_llama_shaped_full_size(llama_kv, rot):
    # b = 3: keys prod (2 MSE bits + QJL), values mse 3 bits
    _llama_full_launch(llama_kv, 3, rot)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("rot", ["dense", "hadamard"])
def test_llama_shaped_bits_sweep_full_size(llama_kv, bits, rot):
    # the b sweep of the Llama-shaped workload at the full 256-segment launch
    _llama_full_launch(llama_kv, bits, rot)


def test_batched_decode_streaming_step():
    # 64 sequences x 8 KV heads (512 segments), 8192 tokens pre-encoded (keys
    # prod b=3, values mse b=3), 32 query heads per sequence (GQA 4).  One step:
    # encode the 64 x 8 new tokens into record 8192 of each segment, then
    # attend over 8193 tokens.
    Tt = torch()
    B, H, T0, G = 64, 8, 8192, 4
    segs, stride = B * H, 8224            # value blocks need a stride multiple of 32
    sk, sv = _setups(3, "dense", seed=3)
    _log("batched decode: pre-encode 64 x 8 x 8192 keys and values")
    k = kv_tensor(B, H, T0 + 1, 128, seed=3).reshape(segs, T0 + 1, 128)
    v = kv_tensor(B, H, T0 + 1, 128, seed=3, value=True).reshape(segs, T0 + 1, 128)
    kcache = sk.alloc(segs * stride, seg_stride=stride)
    vcache = sv.alloc(segs * stride, seg_stride=stride)
    slots = (np.arange(segs)[:, None] * stride + np.arange(T0)[None, :]).reshape(-1)
    sl = Tt.from_numpy(slots).cuda()
    tq.encode_prod(sk.params, Tt.from_numpy(np.ascontiguousarray(k[:, :T0]).reshape(-1, 128)).cuda(), kcache, slot=sl)
    tq.encode_mse(sv.params, Tt.from_numpy(np.ascontiguousarray(v[:, :T0]).reshape(-1, 128)).cuda(), vcache, slot=sl)
    Tt.cuda.synchronize()
    rg = np.random.default_rng(8)
    checked = [0, int(rg.integers(1, segs - 1)), segs - 1]
    codes = {}
    for s in checked:
        kc, vc = _oracle_segment(sk, sv, k[s, :T0], v[s, :T0])
        _plant(sk, sv, kcache, vcache, s, stride, kc, vc)
        codes[s] = (kc, vc)
    # the step: streaming encode of one new token per segment, then attend over T0 + 1
    new_slots = Tt.from_numpy(np.arange(segs, dtype=np.int64) * stride + T0).cuda()
    xk_new, xv_new = np.ascontiguousarray(k[:, T0]), np.ascontiguousarray(v[:, T0])
    tq.encode_prod(sk.params, Tt.from_numpy(xk_new).cuda(), kcache, slot=new_slots)
    tq.encode_mse(sv.params, Tt.from_numpy(xv_new).cuda(), vcache, slot=new_slots)
    q = gaussian_queries(segs * G, 128, seed=3)
    o = Tt.full((segs * G, 128), float("nan"), dtype=Tt.float32, device="cuda")
    ln = Tt.full((segs,), T0 + 1, dtype=Tt.int32, device="cuda")
    scale = 1 / np.sqrt(128)
    tq.attend(sk.params, sv.params, Tt.from_numpy(q).cuda(), segs, G, kcache, vcache, T0 + 1, scale, o,
              tq.alloc_workspace(tq.attend_workspace(sk.params, sv.params, segs, G, T0 + 1)), length=ln)
    Tt.cuda.synchronize()
    # the appended records against the oracle's encoding of the new tokens
    new_rec = np.arange(segs) * stride + T0
    ni = Tt.from_numpy(new_rec).cuda()
    _log(f"  appended keys {compare_encode(sk, kcache.planes[ni].cpu().numpy().view(np.uint32), kcache.scalars[ni].cpu().numpy(), sk.encode_oracle(xk_new))}")
    _log(f"  appended values {compare_encode(sv, _value_rows(vcache, new_rec), vcache.scalars[ni].cpu().numpy(), sv.encode_oracle(xv_new))}")
    got = o.cpu().numpy()
    assert np.isfinite(got).all()
    for s in checked:
        kc, vc = codes[s]
        nk, nv = _oracle_segment(sk, sv, k[s, T0:T0 + 1], v[s, T0:T0 + 1])
        for f in ("idx", "z", "n", "gamma"):
            setattr(kc, f, np.concatenate([getattr(kc, f), getattr(nk, f)]))
        for f in ("idx", "n"):
            setattr(vc, f, np.concatenate([getattr(vc, f), getattr(nv, f)]))
        rows = slice(s * G, (s + 1) * G)
        w = check_heads(got[rows], _oracle_attend(sk, sv, q[rows], kc, vc, scale))
        _log(f"  segment {s}: attend over {T0 + 1} tokens, worst rel {w:.2e}")
