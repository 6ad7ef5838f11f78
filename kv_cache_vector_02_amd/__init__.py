"""Python binding of libtq (the TurboQuant hot path for MI355X / gfx950).

Argument marshalling only: every computation runs in the HIP kernels of
libtq.so, reached through its C ABI (include/tq.h), with the same names.
PyTorch provides device memory and the current stream.  There is no fallback:
if libtq.so is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

TQ_OK, TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_HIP = 0, 1, 2, 3
TQ_ROT_DENSE, TQ_ROT_HADAMARD, TQ_ROT_HADAMARD2 = 0, 1, 2
TQ_F32, TQ_F16 = 0, 1
TQ_LAYOUT_BLOCKS, TQ_LAYOUT_RECORDS = 0, 1

EXPORTED = (
    "tq_status_string", "tq_last_error", "tq_build_codebook", "tq_key_layout",
    "tq_value_layout", "tq_key_record_words", "tq_encode_prod", "tq_encode_mse", "tq_encode_mse_keys", "tq_encode_eden", "tq_encode_workspace", "tq_encode_prod_ws",
    "tq_scores_workspace",
    "tq_scores", "tq_scores_prepare", "tq_scores_prepared", "tq_attend_workspace", "tq_attend", "tq_attend_prepare", "tq_attend_prepared", "tq_scores_topk_workspace", "tq_scores_topk",
    "tq_key_record_bytes", "tq_val_record_bytes", "tq_scores_noalloc", "tq_scores_noalloc_capacity",
    "tq_hadamard_matrix", "tq_build_polar_codebook", "tq_polar_record_words", "tq_polar_encode",
    "tq_polar_decode", "tq_polar_scores",
)
# measurement and testing entry points (include/tq_testing.h)
EXPORTED_TESTING = ("tq_testing_stream", "tq_testing_scores_wait")


class TQError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_status_name(status)}: {msg}")
        self.status = status


def _status_name(s):
    return {0: "TQ_OK", 1: "TQ_ERR_INVALID_ARG", 2: "TQ_ERR_UNSUPPORTED", 3: "TQ_ERR_HIP"}.get(s, str(s))


class tq_params(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int), ("d_rot", ctypes.c_int), ("m", ctypes.c_int),
                ("bits", ctypes.c_int), ("rot", ctypes.c_int),
                ("pi", ctypes.c_void_p), ("eps", ctypes.c_void_p), ("s", ctypes.c_void_p),
                ("centroids", ctypes.c_void_p), ("boundaries", ctypes.c_void_p),
                ("n_sets", ctypes.c_int), ("set_div", ctypes.c_int)]


class tq_polar_params(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int), ("rot", ctypes.c_int), ("bits1", ctypes.c_int), ("bits", ctypes.c_int),
                ("m", ctypes.c_int), ("pi", ctypes.c_void_p), ("eps", ctypes.c_void_p), ("s", ctypes.c_void_p),
                ("centroids", ctypes.c_void_p), ("boundaries", ctypes.c_void_p)]


class tq_cache(ctypes.Structure):
    _fields_ = [("planes", ctypes.c_void_p), ("scalars", ctypes.c_void_p),
                ("seg_stride", ctypes.c_int64), ("records", ctypes.c_int64)]


_lib = None


def lib():
    """The loaded libtq.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run python -m kv_cache_vector_02_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, ci, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        P = ctypes.POINTER(tq_params)
        L.tq_status_string.restype = ctypes.c_char_p
        L.tq_status_string.argtypes = [ci]
        L.tq_last_error.restype = ctypes.c_char_p
        L.tq_last_error.argtypes = []
        L.tq_build_codebook.argtypes = [ci, ci, vp, vp]
        L.tq_key_layout.argtypes = [P, vp, vp, vp]
        L.tq_value_layout.argtypes = [P, vp, vp, vp]
        L.tq_key_record_words.restype = sz
        L.tq_key_record_words.argtypes = [P]
        for f in (L.tq_encode_prod, L.tq_encode_mse, L.tq_encode_mse_keys):
            f.argtypes = [P, vp, ci, i64, i64, tq_cache, vp, vp]
        L.tq_encode_eden.argtypes = [P, vp, ci, i64, i64, ci, tq_cache, vp, vp]
        L.tq_encode_prod_ws.argtypes = [P, vp, ci, i64, i64, tq_cache, vp, vp, sz, vp]
        L.tq_scores_workspace.restype = sz
        L.tq_scores_workspace.argtypes = [P, ci, ci]
        L.tq_encode_workspace.restype = sz
        L.tq_encode_workspace.argtypes = [P, i64]
        L.tq_scores.argtypes = [P, vp, ci, ci, tq_cache, vp, i64, vp, vp, sz, vp]
        L.tq_scores_prepare.argtypes = [P, vp, ci, ci, vp, sz, vp]
        L.tq_scores_prepared.argtypes = [P, ci, ci, tq_cache, vp, i64, vp, vp, sz, vp]
        L.tq_scores_topk_workspace.restype = sz
        L.tq_scores_topk_workspace.argtypes = [P, ci, i64, ci]
        L.tq_scores_topk.argtypes = [P, vp, ci, tq_cache, i64, ci, vp, vp, vp, sz, vp]
        L.tq_attend_workspace.restype = sz
        L.tq_attend_workspace.argtypes = [P, P, ci, ci, i64]
        L.tq_attend.argtypes = [P, P, vp, ci, ci, tq_cache, tq_cache, vp, i64, ctypes.c_float,
                                vp, vp, sz, vp]
        L.tq_attend_prepare.argtypes = [P, vp, ci, ci, vp, sz, vp]
        L.tq_attend_prepared.argtypes = [P, P, ci, ci, tq_cache, tq_cache, vp, i64, ctypes.c_float,
                                         vp, vp, sz, vp]
        L.tq_scores_noalloc.argtypes = [P, vp, ci, ci, tq_cache, vp, i64, vp, vp]
        L.tq_hadamard_matrix.argtypes = [vp, ci, ci, ci, vp, vp]
        L.tq_scores_noalloc_capacity.restype = sz
        L.tq_scores_noalloc_capacity.argtypes = []
        L.tq_key_record_bytes.restype = sz
        L.tq_key_record_bytes.argtypes = [P]
        L.tq_val_record_bytes.restype = sz
        L.tq_val_record_bytes.argtypes = [P]
        PP = ctypes.POINTER(tq_polar_params)
        L.tq_build_polar_codebook.argtypes = [ci, ci, vp, vp]
        L.tq_polar_record_words.restype = sz
        L.tq_polar_record_words.argtypes = [PP]
        L.tq_polar_encode.argtypes = [PP, vp, ci, i64, i64, tq_cache, vp, vp]
        L.tq_polar_decode.argtypes = [PP, tq_cache, i64, vp, i64, vp]
        L.tq_polar_scores.argtypes = [PP, vp, ci, ci, tq_cache, vp, i64, vp, vp]
        L.tq_testing_scores_wait.restype = ci
        L.tq_testing_scores_wait.argtypes = [P, vp, ci, ci, tq_cache, vp, i64, vp, vp, sz, ci, vp]
        L.tq_testing_stream.restype = ci
        L.tq_testing_stream.argtypes = [vp, sz, vp, sz, ci, ci, vp]
        for name in EXPORTED:
            if name not in ("tq_status_string", "tq_last_error", "tq_scores_workspace", "tq_key_record_words",
                            "tq_attend_workspace", "tq_encode_workspace", "tq_scores_topk_workspace",
                            "tq_key_record_bytes", "tq_val_record_bytes", "tq_scores_noalloc_capacity",
                            "tq_polar_record_words"):
                getattr(L, name).restype = ci
        _lib = L
    return _lib


def _check(status):
    if status != TQ_OK:
        raise TQError(status, lib().tq_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def build_codebook(d: int, bits: int):
    """(centroids [2^bits], boundaries [2^bits - 1]) float64, see tq_build_codebook."""
    c = np.zeros(2 ** bits, np.float64)
    b = np.zeros(2 ** bits - 1, np.float64)
    _check(lib().tq_build_codebook(int(d), int(bits), c.ctypes.data, b.ctypes.data))
    return c, b


def build_polar_codebook(level: int, bits: int):
    """(centroids [2^bits], boundaries [2^bits - 1]) float64 of a level's angle
    (see tq_build_polar_codebook)."""
    c = np.zeros(2 ** bits, np.float64)
    b = np.zeros(2 ** bits - 1, np.float64)
    _check(lib().tq_build_polar_codebook(int(level), int(bits), c.ctypes.data, b.ctypes.data))
    return c, b


@dataclass
class Params:
    """Owns what a tq_params points to: device matrices and the host codebook."""
    d: int
    bits: int
    rot: int
    centroids: np.ndarray                 # float32 host
    boundaries: np.ndarray                # float32 host
    pi: Optional[object] = None           # torch float32 [d_rot][d] on the GPU
    eps: Optional[object] = None          # torch float32 [d_rot]
    s: Optional[object] = None            # torch float32 [m][d_rot]
    d_rot: int = 0
    m: int = 0
    n_sets: int = 1                       # rotation sets held by pi / eps / s (leading dimension)
    set_div: int = 1                      # segment seg uses set (seg // set_div) % n_sets
    _c: tq_params = field(default=None, repr=False)

    def __post_init__(self):
        self.centroids = np.ascontiguousarray(self.centroids, np.float32)
        self.boundaries = np.ascontiguousarray(self.boundaries, np.float32)
        if not self.d_rot:
            self.d_rot = self.d
        if not self.m:
            self.m = self.d_rot
        self._c = tq_params(self.d, self.d_rot, self.m, self.bits, self.rot,
                            None if self.pi is None else self.pi.data_ptr(),
                            None if self.eps is None else self.eps.data_ptr(),
                            None if self.s is None else self.s.data_ptr(),
                            self.centroids.ctypes.data, self.boundaries.ctypes.data,
                            int(self.n_sets), int(self.set_div))

    @property
    def c(self):
        return ctypes.byref(self._c)

    def set(self, i: int) -> "Params":
        """The parameters of rotation set i alone (views of its pi / eps / s),
        for the encoders, which take one set per call."""
        pick = lambda t: None if t is None else (t[i] if self.n_sets > 1 else t)
        return Params(d=self.d, bits=self.bits, rot=self.rot, centroids=self.centroids, boundaries=self.boundaries,
                      pi=pick(self.pi), eps=pick(self.eps), s=pick(self.s), d_rot=self.d_rot, m=self.m)


def key_layout(p: Params):
    a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(lib().tq_key_layout(p.c, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


def value_layout(p: Params):
    a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(lib().tq_value_layout(p.c, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


@dataclass
class Cache:
    """A packed cache in device memory: plane words int32 [records, W, P] (word w of
    plane p at w * P + p), scalars float16 [records, S].  Its capacity (tq_cache
    records) is the scalars' row count."""
    planes: object
    scalars: object
    seg_stride: int = 0

    @property
    def records(self) -> int:
        return int(self.scalars.shape[0])

    @property
    def c(self):
        return tq_cache(self.planes.data_ptr(), self.scalars.data_ptr(), int(self.seg_stride), self.records)


def alloc_cache(layout, records: int, seg_stride: int = 0, device="cuda"):
    import torch
    P, W, S = layout
    return Cache(torch.zeros((records, W, P), dtype=torch.int32, device=device),
                 torch.zeros((records, S), dtype=torch.float16, device=device), seg_stride)


def key_record_words(p: Params) -> int:
    """32-bit words of one key record (tq_key_record_words)."""
    w = int(lib().tq_key_record_words(p.c))
    if w == 0:
        _check(lib().tq_key_layout(p.c, None, None, None))
    return w


def alloc_key_cache(p: Params, records: int, seg_stride: int = 0, device="cuda"):
    """A key cache for p's records: [records, W, P] words when every coordinate
    group carries the same planes, else (m = d / 2) [records, words]."""
    import torch
    P, W, S = key_layout(p)
    words = key_record_words(p)
    if words == P * W:
        return alloc_cache((P, W, S), records, seg_stride, device)
    return Cache(torch.zeros((records, words), dtype=torch.int32, device=device),
                 torch.zeros((records, S), dtype=torch.float16, device=device), seg_stride)


def alloc_value_cache(layout, records: int, seg_stride: int = 0, device="cuda"):
    """A value cache: block words int32 [ceil(records/32), d_rot, P] (bit i of word
    (B, j, p) = bit p of record 32 B + i at coordinate j), scalars float16 [records, 1].
    At d_rot = 2048 MSE records keep the per-record key layout [records, 64, P]."""
    import torch
    P, W, S = layout
    if W == 64:
        return alloc_cache(layout, records, seg_stride, device)
    return Cache(torch.zeros(((records + 31) // 32, 32 * W, P), dtype=torch.int32, device=device),
                 torch.zeros((records, S), dtype=torch.float16, device=device), seg_stride)


def _dtype_code(x):
    import torch
    if x.dtype == torch.float16:
        return TQ_F16
    if x.dtype == torch.float32:
        return TQ_F32
    raise TypeError("x must be float16 or float32")


def encode_workspace(p: Params, n: int) -> int:
    return int(lib().tq_encode_workspace(p.c, int(n)))


def encode_prod(p: Params, x, out: Cache, slot=None, stream=None, ws=None):
    """tq_encode_prod on the rows of x (2-D, row stride x.stride(0)); with ws,
    tq_encode_prod_ws (needed at d_rot = 2048)."""
    if ws is None:
        _check(lib().tq_encode_prod(p.c, _ptr(x), _dtype_code(x), x.shape[0], x.stride(0), out.c,
                                    _ptr(slot), _stream(stream)))
    else:
        _check(lib().tq_encode_prod_ws(p.c, _ptr(x), _dtype_code(x), x.shape[0], x.stride(0), out.c,
                                       _ptr(slot), _ptr(ws), ws.numel() * ws.element_size(),
                                       _stream(stream)))


def encode_mse(p: Params, x, out: Cache, slot=None, stream=None):
    _check(lib().tq_encode_mse(p.c, _ptr(x), _dtype_code(x), x.shape[0], x.stride(0), out.c,
                               _ptr(slot), _stream(stream)))


def encode_mse_keys(p: Params, x, out: Cache, slot=None, stream=None):
    """MSE-only keys in the per-record key layout (p.s is None; see tq_encode_mse_keys)."""
    _check(lib().tq_encode_mse_keys(p.c, _ptr(x), _dtype_code(x), x.shape[0], x.stride(0), out.c,
                                    _ptr(slot), _stream(stream)))


def encode_eden(p: Params, x, out: Cache, keys: bool, slot=None, stream=None):
    """MSE records with EDEN's unbiased scale n / <y, c[idx]> in place of n (see
    tq_encode_eden): MSE-only keys in the per-record layout when keys, else values."""
    layout = TQ_LAYOUT_RECORDS if keys else TQ_LAYOUT_BLOCKS
    _check(lib().tq_encode_eden(p.c, _ptr(x), _dtype_code(x), x.shape[0], x.stride(0), layout, out.c,
                                _ptr(slot), _stream(stream)))


def scores_workspace(kp: Params, segs: int, group: int) -> int:
    return int(lib().tq_scores_workspace(kp.c, segs, group))


def alloc_workspace(nbytes: int, device="cuda"):
    """A device workspace of nbytes (zero-filled; the library needs no initial
    contents)."""
    import torch
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def scores(kp: Params, q, segs: int, group: int, keys: Cache, T: int, out, ws, length=None,
           stream=None):
    _check(lib().tq_scores(kp.c, _ptr(q), segs, group, keys.c, _ptr(length), int(T), _ptr(out),
                           _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def scores_noalloc(kp: Params, q, segs: int, group: int, keys: Cache, T: int, out, length=None, stream=None):
    """tq_scores_noalloc: tq_scores with the library's per-device scratch array
    as its workspace (nothing allocated; overlapping calls on one GPU race)."""
    _check(lib().tq_scores_noalloc(kp.c, _ptr(q), segs, group, keys.c, _ptr(length), int(T), _ptr(out),
                                   _stream(stream)))


def scores_noalloc_capacity() -> int:
    return int(lib().tq_scores_noalloc_capacity())


def scores_prepare(kp: Params, q, segs: int, group: int, ws, stream=None):
    _check(lib().tq_scores_prepare(kp.c, _ptr(q), segs, group, _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)))


def scores_prepared(kp: Params, segs: int, group: int, keys: Cache, T: int, out, ws, length=None,
                    stream=None):
    _check(lib().tq_scores_prepared(kp.c, segs, group, keys.c, _ptr(length), int(T), _ptr(out), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream)))


def hadamard_matrix(eps, rounds: int, d: int, out, stream=None):
    """tq_hadamard_matrix: the explicit R-round sign-flipped Hadamard transform
    (eps: device float32 [rounds, d_rot]) into out (device float32 [d_rot, d])."""
    _check(lib().tq_hadamard_matrix(_ptr(eps), int(rounds), int(d), int(eps.shape[-1]), _ptr(out), _stream(stream)))


def key_record_bytes(p: Params) -> int:
    """Bytes of one key record (tq_key_record_bytes)."""
    return int(lib().tq_key_record_bytes(p.c))


def val_record_bytes(p: Params) -> int:
    """Bytes of one value record (tq_val_record_bytes)."""
    return int(lib().tq_val_record_bytes(p.c))


def attend_workspace(kp: Params, vp: Params, segs: int, group: int, T: int) -> int:
    return int(lib().tq_attend_workspace(kp.c, vp.c, segs, group, int(T)))


def attend(kp: Params, vp: Params, q, segs: int, group: int, keys: Cache, vals: Cache, T: int,
           scale: float, out, ws, length=None, stream=None):
    _check(lib().tq_attend(kp.c, vp.c, _ptr(q), segs, group, keys.c, vals.c, _ptr(length), int(T),
                           float(scale), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                           _stream(stream)))


def attend_prepare(kp: Params, q, segs: int, group: int, ws, stream=None):
    """tq_attend_prepare: the query pack of tq_attend into ws."""
    _check(lib().tq_attend_prepare(kp.c, _ptr(q), segs, group, _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)))


def attend_prepared(kp: Params, vp: Params, segs: int, group: int, keys: Cache, vals: Cache, T: int,
                    scale: float, out, ws, length=None, stream=None):
    """tq_attend_prepared: tq_attend against the pack of the last attend_prepare on ws."""
    _check(lib().tq_attend_prepared(kp.c, vp.c, segs, group, keys.c, vals.c, _ptr(length), int(T), float(scale),
                                    _ptr(out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def topk_workspace(kp: Params, nq: int, T: int, k: int) -> int:
    return int(lib().tq_scores_topk_workspace(kp.c, int(nq), int(T), int(k)))


def scores_topk(kp: Params, q, keys: Cache, T: int, k: int, idx, val, ws, stream=None):
    """tq_scores_topk: idx int64 [nq][k], val float32 [nq][k] (device tensors)."""
    _check(lib().tq_scores_topk(kp.c, _ptr(q), q.shape[0], keys.c, int(T), int(k), _ptr(idx), _ptr(val),
                                _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def testing_stream(src, read_bytes: int, dst, write_bytes: int, store_policy: int = 1, workgroups: int = 0,
                   stream=None):
    """tq_testing_stream: a plain HBM stream reading read_bytes of src and writing
    write_bytes of dst side by side (the bandwidth ceiling for that mix)."""
    _check(lib().tq_testing_stream(_ptr(src), int(read_bytes), _ptr(dst), int(write_bytes), int(store_policy),
                                   int(workgroups), _stream(stream)))


def testing_scores_wait(kp: Params, q, segs: int, group: int, keys: Cache, T: int, out, ws, wait_us: int,
                        length=None, stream=None):
    """tq_testing_scores_wait: tq_scores with an explicit bound on the wait for
    each segment's query pack (0: the build-it-yourself path)."""
    _check(lib().tq_testing_scores_wait(kp.c, _ptr(q), segs, group, keys.c, _ptr(length), int(T), _ptr(out),
                                        _ptr(ws), ws.numel() * ws.element_size(), int(wait_us), _stream(stream)))


# ---- PolarQuant as stage 1 (tq_polar_*) ----

@dataclass
class PolarParams:
    """Owns what a tq_polar_params points to.  centroids / boundaries are the
    host float32 arrays of every level concatenated (level 1, then 2 .. L)."""
    d: int
    rot: int
    bits1: int
    bits: int
    centroids: np.ndarray
    boundaries: np.ndarray
    pi: Optional[object] = None
    eps: Optional[object] = None
    s: Optional[object] = None
    m: int = 0
    _c: tq_polar_params = field(default=None, repr=False)

    def __post_init__(self):
        self.centroids = np.ascontiguousarray(self.centroids, np.float32)
        self.boundaries = np.ascontiguousarray(self.boundaries, np.float32)
        self._c = tq_polar_params(self.d, self.rot, self.bits1, self.bits, self.m,
                                  None if self.pi is None else self.pi.data_ptr(),
                                  None if self.eps is None else self.eps.data_ptr(),
                                  None if self.s is None else self.s.data_ptr(),
                                  self.centroids.ctypes.data, self.boundaries.ctypes.data)

    @property
    def c(self):
        return ctypes.byref(self._c)


def polar_codebooks(d: int, bits1: int, bits: int):
    """Concatenated float64 (centroids, boundaries) of levels 1 .. log2(d) from tq_build_polar_codebook."""
    L = int(d).bit_length() - 1
    books = [build_polar_codebook(1, bits1)] + [build_polar_codebook(l, bits) for l in range(2, L + 1)]
    return np.concatenate([b[0] for b in books]), np.concatenate([b[1] for b in books])


def polar_record_words(p: PolarParams) -> int:
    w = int(lib().tq_polar_record_words(p.c))
    if w == 0:
        raise TQError(TQ_ERR_INVALID_ARG, "invalid polar parameters")
    return w


def alloc_polar_cache(p: PolarParams, records: int, seg_stride: int = 0, device="cuda"):
    """Polar records: words int32 [records, tq_polar_record_words], scalars float16 [records, 1 or 2]."""
    import torch
    return Cache(torch.zeros((records, polar_record_words(p)), dtype=torch.int32, device=device),
                 torch.zeros((records, 2 if p.m else 1), dtype=torch.float16, device=device), seg_stride)


def polar_encode(p: PolarParams, x, out: Cache, slot=None, stream=None):
    _check(lib().tq_polar_encode(p.c, _ptr(x), _dtype_code(x), x.shape[0], x.stride(0), out.c, _ptr(slot),
                                 _stream(stream)))


def polar_decode(p: PolarParams, cache: Cache, n: int, out, stream=None):
    """x~ of records 0 .. n-1 into out (float32 [n, >= d], row stride out.stride(0))."""
    _check(lib().tq_polar_decode(p.c, cache.c, int(n), _ptr(out), out.stride(0), _stream(stream)))


def polar_scores(p: PolarParams, q, segs: int, group: int, keys: Cache, T: int, out, length=None, stream=None):
    _check(lib().tq_polar_scores(p.c, _ptr(q), segs, group, keys.c, _ptr(length), int(T), _ptr(out),
                                 _stream(stream)))
