"""Quality harness: how well the compressed cache keeps attention and nearest-neighbour order.

Synthetic analogs of the "turboquant-pytorch" page's usage patterns for
attention fidelity and needle-in-a-haystack retrieval, and of its bit-width
table (cosine of the attention distributions and top-1 agreement at 2, 3 and
4 bits):

* attention fidelity: per query, the softmax over the keys of the exact
  scores and of the estimated ones; the cosine of the two distributions and
  whether their argmax is the same key;
* needle: per trial, whether the argmax of the estimated scores over a
  haystack is the exact argmax;
* output fidelity: the cosine between exact softmax attention over the
  uncompressed keys and values and tq_attend over their compressed records.

The compressed side runs in libtq (tq_encode_prod, or tq_encode_mse_keys for
a key quantizer without a QJL matrix; tq_encode_mse for values; with eden,
tq_encode_eden for MSE keys and values; tq_scores, tq_attend; for polar key
parameters, tq_polar_encode and tq_polar_scores, with no attention output).  The exact side is float32 PyTorch on the same device (the
products, the softmax and the weighted sum), the yardstick the compressed
results are measured against; none of it is on the hot path.  Argmax ties go
to the lower key index.
"""
from __future__ import annotations

import kv_cache_vector_02_amd as tq

MAX_GROUP = 16   # query heads per tq_scores / tq_attend segment


def _torch():
    import torch
    return torch


def exact_scores(keys, queries):
    """<q, k> for queries [Q, d] and keys [N, d] (device) -> [Q, N] float32."""
    return queries.float() @ keys.float().t().contiguous()


def encode_keys(kp, keys, seg_stride: int = 0, eden: bool = False) -> tq.Cache:
    """Prod keys, or MSE-only keys when kp has no QJL matrix (with eden, scaled
    by EDEN's unbiased n / <y, c[idx]>); polar records for tq.PolarParams."""
    if isinstance(kp, tq.PolarParams):
        cache = tq.alloc_polar_cache(kp, keys.shape[0], seg_stride)
        tq.polar_encode(kp, keys.contiguous(), cache)
        return cache
    cache = tq.alloc_key_cache(kp, keys.shape[0], seg_stride)
    if kp.s is not None:
        tq.encode_prod(kp, keys.contiguous(), cache)
    elif eden:
        tq.encode_eden(kp, keys.contiguous(), cache, keys=True)
    else:
        tq.encode_mse_keys(kp, keys.contiguous(), cache)
    return cache


def estimated_scores(kp: tq.Params, cache: tq.Cache, n_keys: int, queries):
    """tq_scores of queries [Q, d] against the n_keys records of one cache -> [Q, N]."""
    T = _torch()
    Q = queries.shape[0]
    out = T.empty((Q, n_keys), dtype=T.float32, device=queries.device)
    one = tq.Cache(cache.planes, cache.scalars, 0)
    if isinstance(kp, tq.PolarParams):
        for h0 in range(0, Q, MAX_GROUP):
            g = min(MAX_GROUP, Q - h0)
            tq.polar_scores(kp, queries[h0:h0 + g].contiguous(), 1, g, one, n_keys, out[h0:h0 + g])
        return out
    ws = tq.alloc_workspace(tq.scores_workspace(kp, 1, MAX_GROUP))
    for h0 in range(0, Q, MAX_GROUP):
        g = min(MAX_GROUP, Q - h0)
        tq.scores(kp, queries[h0:h0 + g].contiguous(), 1, g, one, n_keys, out[h0:h0 + g], ws)
    return out


def fidelity(true_scores, est_scores, scale: float = 1.0):
    """(cosine [Q], top-1 agreement [Q] bool) of the softmax rows of scale * scores."""
    T = _torch()
    p = T.softmax(scale * true_scores.double(), dim=-1)
    p_hat = T.softmax(scale * est_scores.double(), dim=-1)
    cos = T.nn.functional.cosine_similarity(p, p_hat, dim=-1)
    top1 = T.argmax(true_scores, dim=-1) == T.argmax(est_scores, dim=-1)
    return cos, top1


def attention_fidelity(kp: tq.Params, keys, queries, scale: float = 1.0, eden: bool = False):
    """Attention-fidelity statistics of one key set [N, d] under queries [Q, d].

    Returns a dict with the per-query cosine and top-1 agreement and their means."""
    cache = encode_keys(kp, keys, eden=eden)
    est = estimated_scores(kp, cache, keys.shape[0], queries)
    true = exact_scores(keys, queries)
    cos, top1 = fidelity(true, est, scale)
    return {"cosine": cos, "top1": top1, "mean_cosine": float(cos.mean()),
            "top1_rate": float(top1.double().mean()), "est": est, "true": true}


def needle_scores(kp: tq.Params, cache: tq.Cache, queries, L: int):
    """tq_scores of one query per trial [trials, d] against its own L records -> [trials, L]."""
    T = _torch()
    trials = queries.shape[0]
    est = T.empty((trials, L), dtype=T.float32, device=queries.device)
    segs = tq.Cache(cache.planes, cache.scalars, L)
    if isinstance(kp, tq.PolarParams):
        tq.polar_scores(kp, queries.contiguous(), trials, 1, segs, L, est)
        return est
    ws = tq.alloc_workspace(tq.scores_workspace(kp, trials, 1))
    tq.scores(kp, queries.contiguous(), trials, 1, segs, L, est, ws)
    return est


def needle(kp: tq.Params, haystacks, queries, eden: bool = False):
    """Needle trials: haystacks [trials, L, d], one query [trials, d] each.

    Returns (found [trials] bool, exact argmax [trials], estimated argmax [trials])."""
    T = _torch()
    trials, L, d = haystacks.shape
    cache = encode_keys(kp, haystacks.reshape(trials * L, d), seg_stride=L, eden=eden)
    est = needle_scores(kp, cache, queries, L)
    true = T.bmm(haystacks.float(), queries.float()[:, :, None].contiguous())[:, :, 0]
    tb, eb = T.argmax(true, dim=-1), T.argmax(est, dim=-1)
    return tb == eb, tb, eb


def exact_attention(keys, values, queries, group: int, scale: float):
    """softmax(scale q K^T) V per segment: keys, values [segs, L, d]; queries [segs*group, d]."""
    T = _torch()
    segs, L, d = keys.shape
    q = queries.float().reshape(segs, group, d)
    s = T.bmm(q, keys.float().transpose(1, 2).contiguous())
    w = T.softmax(scale * s, dim=-1)
    return T.bmm(w, values.float()).reshape(segs * group, d)


def compressed_attention(kp: tq.Params, vp: tq.Params, kc: tq.Cache, vc: tq.Cache, L: int, queries,
                         group: int, scale: float):
    """tq_attend of queries [segs*group, d] over segments of L records -> [segs*group, d]."""
    T = _torch()
    segs = queries.shape[0] // group
    out = T.empty((segs * group, queries.shape[1]), dtype=T.float32, device=queries.device)
    ws = tq.alloc_workspace(tq.attend_workspace(kp, vp, segs, group, L))
    tq.attend(kp, vp, queries.contiguous(), segs, group, tq.Cache(kc.planes, kc.scalars, L),
              tq.Cache(vc.planes, vc.scalars, L), L, scale, out, ws)
    return out


def output_fidelity(kp: tq.Params, vp: tq.Params, keys, values, queries, group: int, scale: float,
                    eden: bool = False):
    """Cosine per query head between exact attention and tq_attend over the compressed records.

    keys, values: [segs, L, d] device; queries [segs*group, d] float32.
    Returns (cosine [segs*group], exact output, compressed output)."""
    T = _torch()
    segs, L, d = keys.shape
    kc = encode_keys(kp, keys.reshape(segs * L, d), seg_stride=L, eden=eden)
    vc = tq.alloc_value_cache(tq.value_layout(vp), segs * L, seg_stride=L)
    if eden:
        tq.encode_eden(vp, values.reshape(segs * L, d).contiguous(), vc, keys=False)
    else:
        tq.encode_mse(vp, values.reshape(segs * L, d).contiguous(), vc)
    out = compressed_attention(kp, vp, kc, vc, L, queries, group, scale)
    ref = exact_attention(keys, values, queries, group, scale)
    cos = T.nn.functional.cosine_similarity(ref.double(), out.double(), dim=-1)
    return cos, ref, out
