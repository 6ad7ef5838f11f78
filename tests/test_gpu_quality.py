"""GPU parity of the quality harness (kv_cache_vector_02_amd.quality): its
statistics from libtq's outputs against the oracle's statistics of the
oracle's own scores and attention, on the same seeded inputs.

Workloads follow the "turboquant-pytorch" page's usage patterns: attention
fidelity with 2048 random unit keys and 100 random unit queries at d = 128
(temperature 1); needle trials with 8192-key haystacks; and attention outputs
over decoder-shaped keys and values at temperature 1/sqrt(d).

Tolerances.  The scores agree with the oracle's to 1e-3 of each row's largest
magnitude.  For softmax rows, a perturbation e of the scores moves 1 - cos by
about Cov_pi(delta, e) (pi proportional to p^2, delta the estimate's own error
against the exact scores), so |cos_gpu - cos_oracle| <= 1e-4 is ample at these
score sizes (|s| < 1, std(delta) < 0.1).  An argmax may differ only where the
oracle's estimated scores of the two candidates lie within twice the score
tolerance.  For attention outputs the per-head cosine moves by at most
sin(theta) * ||delta_o||_2 / ||o||_2 <= sin(theta) * sqrt(d) * 1e-3, theta the
oracle's angle to the exact output."""
import numpy as np
import pytest

import kv_cache_vector_02_amd as tq
from kv_cache_vector_02_amd import quality
from oracle import estimator as est
from oracle import quality as oq
from oracle import quantizer as qz
from tests.gpu_util import Setup, torch
from tests.test_gpu_attend import oracle_value_cache
from tests.test_gpu_scores import oracle_key_cache
from tq_inputs import QUERIES, gaussian_queries, kv_tensor, needle_haystacks, unit_gaussian

pytestmark = pytest.mark.gpu
SCORE_TOL = 1e-3


def _log(msg):
    print(msg, flush=True)


def _dev(a):
    return torch().from_numpy(np.ascontiguousarray(a)).cuda()


def _check_argmax(got_idx, oracle_idx, oracle_est):
    """Where the argmax differs, the oracle's two candidates are a near tie."""
    rows = np.nonzero(got_idx != oracle_idx)[0]
    for r in rows:
        gap = oracle_est[r, oracle_idx[r]] - oracle_est[r, got_idx[r]]
        assert gap <= 2 * SCORE_TOL * np.abs(oracle_est[r]).max(), (r, gap)
    return len(rows)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_attention_fidelity_unit_vectors(bits):
    _log(f"quality fidelity b{bits}: 2048 unit keys, 100 unit queries")
    keys = unit_gaussian(2048, 128, seed=11)
    qs = unit_gaussian(100, 128, seed=11, purpose=QUERIES)
    st = Setup(bits=bits, prod=True, seed=11)
    cache, (idx, z, n, g) = oracle_key_cache(st, keys)
    est_gpu = quality.estimated_scores(st.params, cache, 2048, _dev(qs))
    true_gpu = quality.exact_scores(_dev(keys), _dev(qs))
    cos, top1 = quality.fidelity(true_gpu, est_gpu)
    cos, top1 = cos.cpu().numpy(), top1.cpu().numpy()

    est_o = est.prod_scores(qs, idx, z, n, g, st.rot, st.s, st.c32)
    true_o = qs.astype(np.float64) @ keys.astype(np.float64).T
    cos_o, top1_o = oq.attention_fidelity(true_o, est_o)
    assert np.max(np.abs(cos - cos_o)) <= 1e-4, np.max(np.abs(cos - cos_o))
    eg = est_gpu.cpu().numpy()
    flips = _check_argmax(np.argmax(eg, 1), oq.argmax_rows(est_o), est_o)
    flips += _check_argmax(np.argmax(true_gpu.cpu().numpy(), 1), oq.argmax_rows(true_o), true_o)
    if flips == 0:
        assert np.array_equal(top1, top1_o)
    _log(f"  mean cos {cos.mean():.6f} (oracle {cos_o.mean():.6f}), top-1 {top1.mean():.2f} "
         f"(oracle {top1_o.mean():.2f}), near-tie argmax flips {flips}")


@pytest.mark.parametrize("m", [128, 64])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_end_to_end_fidelity_with_gpu_encode(bits, m):
    # the harness's own path: GPU encode + scores.  Index and sign bits may
    # differ from the oracle's only within 1e-5 of a decision boundary, on at
    # most 1e-4 of the coordinates; each such key moves its score by about the
    # cell width times one query coordinate, far below the softmax's scale here.
    _log(f"quality end-to-end b{bits} m{m}")
    keys = unit_gaussian(2048, 128, seed=12)
    qs = unit_gaussian(100, 128, seed=12, purpose=QUERIES)
    st = Setup(bits=bits, prod=True, seed=12, m=m)
    r = quality.attention_fidelity(st.params, _dev(keys), _dev(qs))
    code = st.encode_oracle(keys)
    n16 = code.n.astype(np.float16).astype(np.float64)
    g16 = code.gamma.astype(np.float16).astype(np.float64)
    est_o = est.prod_scores(qs, code.idx, code.z, n16, g16, st.rot, st.s, st.c32)
    cos_o, top1_o = oq.attention_fidelity(qs.astype(np.float64) @ keys.astype(np.float64).T, est_o)
    cos = r["cosine"].cpu().numpy()
    assert np.max(np.abs(cos - cos_o)) <= 1e-4
    assert abs(r["top1_rate"] - top1_o.mean()) <= 0.02
    _log(f"  mean cos {r['mean_cosine']:.6f} (oracle {cos_o.mean():.6f}), top-1 {r['top1_rate']:.2f} "
         f"(oracle {top1_o.mean():.2f})")


@pytest.mark.parametrize("eden", [False, True])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_end_to_end_fidelity_mse_keys(bits, eden):
    # MSE-only keys at b index bits (no QJL matrix), scaled by the norm or by
    # EDEN's unbiased scale: GPU encode + scores, against the oracle's encoder
    # and inner product
    _log(f"quality end-to-end, MSE-only keys b{bits} eden {eden}")
    keys = unit_gaussian(2048, 128, seed=12)
    qs = unit_gaussian(100, 128, seed=12, purpose=QUERIES)
    st = Setup(bits=bits, prod=False, seed=12)
    r = quality.attention_fidelity(st.params, _dev(keys), _dev(qs), eden=eden)
    code = (qz.encode_eden(keys, st.rot, st.c32, st.b32, storage=False) if eden else st.encode_oracle(keys))
    est_o = est.mse_scores(qs, code.idx, code.n.astype(np.float16).astype(np.float64), st.rot, st.c32)
    cos_o, top1_o = oq.attention_fidelity(qs.astype(np.float64) @ keys.astype(np.float64).T, est_o)
    cos = r["cosine"].cpu().numpy()
    assert np.max(np.abs(cos - cos_o)) <= 1e-4
    assert abs(r["top1_rate"] - top1_o.mean()) <= 0.02
    _log(f"  mean cos {r['mean_cosine']:.6f} (oracle {cos_o.mean():.6f}), top-1 {r['top1_rate']:.2f} "
         f"(oracle {top1_o.mean():.2f})")


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_needle_trials(bits):
    _log(f"quality needle b{bits}: 20 trials x 8192 keys")
    trials, L = 20, 8192
    hay, qs, pos = needle_haystacks(trials, L, 128, seed=13)
    st = Setup(bits=bits, prod=True, seed=13)
    cache, (idx, z, n, g) = oracle_key_cache(st, hay.reshape(-1, 128), seg_stride=L)
    est_gpu = quality.needle_scores(st.params, cache, _dev(qs), L).cpu().numpy()
    est_o = np.stack([est.prod_scores(qs[t:t + 1], idx[t * L:(t + 1) * L], z[t * L:(t + 1) * L],
                                      n[t * L:(t + 1) * L], g[t * L:(t + 1) * L], st.rot, st.s, st.c32)[0]
                      for t in range(trials)])
    true_o = np.einsum("tld,td->tl", hay.astype(np.float64), qs.astype(np.float64))
    assert np.array_equal(oq.argmax_rows(true_o), pos), "the needle is the exact nearest key"
    found_o = oq.needle_found(true_o, est_o)
    flips = _check_argmax(np.argmax(est_gpu, 1), oq.argmax_rows(est_o), est_o)
    found = np.argmax(est_gpu, 1) == pos
    if flips == 0:
        assert np.array_equal(found, found_o)
    # the harness's end-to-end needle run (GPU encode) on the same trials
    f_all, tb, eb = quality.needle(st.params, _dev(hay), _dev(qs))
    assert np.array_equal(tb.cpu().numpy(), pos)
    _log(f"  found {found.sum()}/{trials} (oracle {found_o.sum()}/{trials}; end to end "
         f"{int(f_all.sum())}/{trials})")


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_output_fidelity_decoder_shaped(bits):
    _log(f"quality output b{bits}: 4 segments x 2048 tokens, G=8")
    segs, L, G = 4, 2048, 8
    scale = 1 / np.sqrt(128)
    xk = kv_tensor(1, segs, L, 128, seed=14)[0]
    xv = kv_tensor(1, segs, L, 128, seed=14, value=True)[0]
    qs = gaussian_queries(segs * G, 128, seed=14)
    sk = Setup(bits=bits, prod=True, seed=14)
    sv = Setup(bits=bits, prod=False, seed=14, purpose_pi=4, purpose_eps=6)
    kc, (kidx, kz, kn, kg) = oracle_key_cache(sk, xk.reshape(-1, 128), seg_stride=L)
    vc, vidx, vn = oracle_value_cache(sv, xv.reshape(-1, 128), L)
    out = quality.compressed_attention(sk.params, sv.params, kc, vc, L, _dev(qs), G, scale).cpu().numpy()
    ref = quality.exact_attention(_dev(xk), _dev(xv), _dev(qs), G, scale).cpu().numpy()
    exact = np.concatenate([
        oq_exact(xk[s], xv[s], qs[s * G:(s + 1) * G], scale) for s in range(segs)])
    np.testing.assert_allclose(ref, exact, rtol=0, atol=1e-4 * np.abs(exact).max())
    o_o = np.concatenate([
        est.attend(qs[s * G:(s + 1) * G], (kidx[s * L:(s + 1) * L], kz[s * L:(s + 1) * L],
                                           kn[s * L:(s + 1) * L], kg[s * L:(s + 1) * L]),
                   (vidx[s * L:(s + 1) * L], vn[s * L:(s + 1) * L]), sk.rot, sk.s, sk.c32, sv.rot, sv.c32,
                   scale) for s in range(segs)])
    cos = oq.row_cosine(exact, out)
    cos_o = oq.row_cosine(exact, o_o)
    sin_o = np.sqrt(np.maximum(0.0, 1 - cos_o ** 2))
    assert np.all(np.abs(cos - cos_o) <= sin_o * np.sqrt(128) * SCORE_TOL + 1e-6)
    # the harness's end-to-end run (GPU encode of keys and values)
    c_all, _, _ = quality.output_fidelity(sk.params, sv.params, _dev(xk), _dev(xv), _dev(qs), G, scale)
    _log(f"  mean cos {cos.mean():.6f} (oracle {cos_o.mean():.6f}; end to end {float(c_all.mean()):.6f})")


def oq_exact(k, v, q, scale):
    """Exact softmax attention of q over (k, v), float64 (the oracle's weighted sum on the raw inputs)."""
    return est.softmax_weighted_sum(q.astype(np.float64) @ k.astype(np.float64).T, v, scale)


@pytest.mark.parametrize("qjl", [False, True])
def test_polar_attention_fidelity_and_needle(qjl):
    # PolarQuant keys through the harness (tq_polar_scores) against the oracle's
    # statistics of its own polar scores, on oracle-packed records
    from oracle import polar as pq
    from tests.test_gpu_polar import PolarSetup
    _log(f"quality polar{' + QJL' if qjl else ''}: fidelity and needle")
    w = 2 if qjl else 3
    st = PolarSetup(w, w, 128 if qjl else 0, "dense", seed=11)
    keys = unit_gaussian(2048, 128, seed=11)
    qs = unit_gaussian(100, 128, seed=11, purpose=QUERIES)
    code = st.oracle(keys)
    est_gpu = quality.estimated_scores(st.params, st.packed_cache(code), 2048, _dev(qs))
    cos, top1 = quality.fidelity(quality.exact_scores(_dev(keys), _dev(qs)), est_gpu)
    est_o = pq.polar_scores(qs, code, st.rot, st.s)
    true_o = qs.astype(np.float64) @ keys.astype(np.float64).T
    cos_o, top1_o = oq.attention_fidelity(true_o, est_o)
    assert np.max(np.abs(cos.cpu().numpy() - cos_o)) <= 1e-4
    flips = _check_argmax(np.argmax(est_gpu.cpu().numpy(), 1), oq.argmax_rows(est_o), est_o)
    if flips == 0:
        assert np.array_equal(top1.cpu().numpy(), top1_o)
    # needle: 20 haystacks of 8192 keys, one segment each
    hay, hq, _ = needle_haystacks(20, 8192, 128, seed=13)
    hcode = st.oracle(hay.reshape(-1, 128))
    cache = st.packed_cache(hcode, 8192)
    est_n = quality.needle_scores(st.params, cache, _dev(hq), 8192).cpu().numpy()
    for t in range(20):
        sub = pq.PolarCode(codes=None, n=hcode.n[t * 8192:(t + 1) * 8192], y=None, angles=None,
                           y_hat=hcode.y_hat[t * 8192:(t + 1) * 8192],
                           z=None if hcode.z is None else hcode.z[t * 8192:(t + 1) * 8192],
                           gamma=None if hcode.gamma is None else hcode.gamma[t * 8192:(t + 1) * 8192])
        want = pq.polar_scores(hq[t:t + 1], sub, st.rot, st.s)[0]
        assert np.max(np.abs(est_n[t] - want)) <= 2e-5 * np.linalg.norm(hq[t]) * np.max(sub.n)
    _log(f"  mean cos {cos.mean().item():.6f} (oracle {cos_o.mean():.6f}), top-1 {top1.double().mean().item():.2f}")
