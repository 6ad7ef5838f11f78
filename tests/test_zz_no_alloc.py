"""tq_scores_noalloc: tq_scores with its workspace in the library's own
per-device scratch array, for callers that cannot allocate.  Called through
the C ABI, its scores must be the same bytes as tq_scores' on the same inputs
(the same kernels), call after call with the array keeping the previous call's
contents, and agree with the oracle to 1e-3 of each row's largest magnitude;
sizes past the array's capacity are rejected before any launch."""
import numpy as np
import pytest

import kv_cache_vector_02_amd as tq
from oracle import estimator as est
from tests.gpu_util import Setup, torch
from tests.test_gpu_scores import check_rows, gpu_scores, oracle_key_cache
from tq_inputs import gaussian_queries, kv_tensor

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _noalloc(st, q, segs, group, cache, T_):
    Tt = torch()
    qd = Tt.from_numpy(np.ascontiguousarray(q, np.float32)).cuda()
    out = Tt.full((segs * group, T_), float("nan"), dtype=Tt.float32, device="cuda")
    tq.scores_noalloc(st.params, qd, segs, group, cache, T_, out)
    Tt.cuda.synchronize()
    return out.cpu().numpy()


def test_noalloc_scores_match_tq_scores_on_two_calls():
    # a larger call, then a smaller one (fewer segments, another group): each
    # against tq_scores with a caller workspace, bit for bit, and the oracle
    st = Setup(bits=3, prod=True, seed=41)
    for segs, group, T_, seed in ((6, 8, 2500, 41), (2, 4, 700, 42)):
        _log(f"noalloc scores: segs {segs}, group {group}, T {T_}")
        x = kv_tensor(1, segs, T_, 128, seed=seed)[0].reshape(-1, 128)
        cache, (idx, z, n, g) = oracle_key_cache(st, x, seg_stride=T_)
        q = gaussian_queries(segs * group, 128, seed=seed)
        got = _noalloc(st, q, segs, group, cache, T_)
        ref_ws = gpu_scores(st, q, segs, group, cache, T_)
        assert np.array_equal(got, ref_ws), "tq_scores_noalloc differs from tq_scores"
        for s in range(segs):
            rows = slice(s * group, (s + 1) * group)
            sl = slice(s * T_, (s + 1) * T_)
            check_rows(got[rows], est.prod_scores(q[rows], idx[sl], z[sl], n[sl], g[sl], st.rot, st.s, st.c32))


def test_noalloc_rejects_sizes_past_the_scratch():
    st = Setup(bits=3, prod=True, seed=43)
    cap = tq.scores_noalloc_capacity()
    segs = 1
    while tq.scores_workspace(st.params, segs, 16) <= cap:
        segs *= 2
    Tt = torch()
    q = Tt.zeros((segs * 16, 128), dtype=Tt.float32, device="cuda")
    cache = tq.alloc_cache(st.layout(), segs * 32, seg_stride=32)
    out = Tt.zeros((segs * 16, 32), dtype=Tt.float32, device="cuda")
    with pytest.raises(tq.TQError, match="scratch"):
        tq.scores_noalloc(st.params, q, segs, 16, cache, 32, out)
