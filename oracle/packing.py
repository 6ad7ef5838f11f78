"""The packed record layout, written from its specification.

A record holds bit-planes of 32-bit little-endian words followed (in a
separate array) by float16 scalars:

  plane p, coordinate j  ->  bit (j mod 32) of word (j div 32) of plane p,
  and word w of plane p is 32-bit word w * P + p of the record (P planes):
  the planes are interleaved word by word, so the P words that cover the same
  32 coordinates are adjacent.

Key record (TurboQuant-prod, b bits):  planes 0..b-2 carry bit p of the
(b-1)-bit index, plane b-1 carries the QJL bits z (bit 1 <=> (S r)_i >= 0);
scalars = (float16 n, float16 gamma).
Value record (TurboQuant-MSE, b bits): planes 0..b-1 carry bit p of the
index; scalars = (float16 n).

Value caches use the same bits transposed within blocks of 32 records: for
block B (records 32 B .. 32 B + 31), coordinate j and plane p there is one
32-bit word, word number (j * P + p) of the block, whose bit i is bit p of the
index of record 32 B + i at coordinate j.  The float16 norms stay one per
record.  (Keys are read along coordinates, values along tokens; each layout
puts the bits a reader needs in one word.)

With fewer QJL rows than coordinates (m < d, the first page's proj_dim =
head_dim / 2) the sign plane has m/32 words.  The general key record is: for
each group of 32 coordinates w = 0 .. d/32 - 1, the b-1 index words of the
group, then sign word w if w < m/32.  With m = d that is the interleaved
record above.

This matches the storage accounting the first page uses (indices packed at b
bits per coordinate, one sign bit per projection row, float16 norms).
"""
from __future__ import annotations

import numpy as np


def pack_bits(bits) -> np.ndarray:
    """[N, L] booleans (L a multiple of 32) -> [N, L/32] uint32 words."""
    bits = np.asarray(bits, dtype=bool)
    n, length = bits.shape
    if length % 32:
        raise ValueError("length must be a multiple of 32")
    b = bits.reshape(n, length // 32, 32).astype(np.uint64)
    weights = (np.uint64(1) << np.arange(32, dtype=np.uint64))
    return (b * weights).sum(axis=2).astype(np.uint32)


def unpack_bits(words) -> np.ndarray:
    words = np.asarray(words, dtype=np.uint32)
    n, w = words.shape
    shifts = np.arange(32, dtype=np.uint32)
    return ((words[:, :, None] >> shifts[None, None, :]) & 1).astype(bool).reshape(n, w * 32)


def index_planes(idx, nbits: int) -> np.ndarray:
    """[N, d] indices -> [N, nbits, d/32] words, plane p = bit p (plane-major view)."""
    idx = np.asarray(idx, dtype=np.int64)
    return np.stack([pack_bits((idx >> p) & 1) for p in range(nbits)], axis=1) if nbits else \
        np.zeros((idx.shape[0], 0, idx.shape[1] // 32), np.uint32)


def planes_to_index(planes) -> np.ndarray:
    """Plane-major [N, nbits, d/32] words -> [N, d] indices."""
    planes = np.asarray(planes, dtype=np.uint32)
    n, nb, w = planes.shape
    idx = np.zeros((n, w * 32), dtype=np.int64)
    for p in range(nb):
        idx |= unpack_bits(planes[:, p, :]).astype(np.int64) << p
    return idx


def interleave(plane_major) -> np.ndarray:
    """[N, P, W] plane-major words -> [N, W, P] record order (word w of plane p at w*P + p)."""
    return np.ascontiguousarray(np.asarray(plane_major, np.uint32).transpose(0, 2, 1))


def deinterleave(record) -> np.ndarray:
    """[N, W, P] record order -> [N, P, W] plane-major words."""
    return np.ascontiguousarray(np.asarray(record, np.uint32).transpose(0, 2, 1))


def pack_key(code, nbits_idx: int):
    """ProdCode -> (record words, scalars [N, 2] float16).

    With m = d (as many QJL rows as coordinates) the words come as
    [N, d/32, nbits_idx + 1] in record order; with m < d as [N, words per
    record], group by group (index words, then sign word w while w < m/32)."""
    idx_pm = index_planes(code.idx, nbits_idx)              # [N, B, W]
    sign = pack_bits(code.z)                                # [N, m/32]
    scalars = np.stack([code.n, code.gamma], axis=1).astype(np.float16)
    n, _, w = idx_pm.shape
    if sign.shape[1] == w:
        return interleave(np.concatenate([idx_pm, sign[:, None, :]], axis=1)), scalars
    groups = []
    for g in range(w):
        groups.append(idx_pm[:, :, g])
        if g < sign.shape[1]:
            groups.append(sign[:, g:g + 1])
    return np.ascontiguousarray(np.concatenate(groups, axis=1)), scalars


def pack_value(code, nbits: int):
    """MseCode -> (planes [N, d/32, nbits] uint32 in record order, scalars [N, 1] float16)."""
    return interleave(index_planes(code.idx, nbits)), code.n.astype(np.float16)[:, None]


def unpack_key(planes, scalars, nbits_idx: int, d: int = 0):
    """Record words -> (idx [N, d], z [N, m] bool, n [N], gamma [N]), scalars as float64.

    [N, W, P] words are the m = d record; [N, words] words the m < d record
    of coordinate count d (which must be given)."""
    s = np.asarray(scalars, np.float16).astype(np.float64)
    planes = np.asarray(planes, np.uint32)
    if planes.ndim == 3:
        pm = deinterleave(planes)
        return planes_to_index(pm[:, :nbits_idx, :]), unpack_bits(pm[:, nbits_idx, :]), s[:, 0], s[:, 1]
    w = d // 32
    mw = planes.shape[1] - w * nbits_idx
    idx_pm = np.zeros((planes.shape[0], nbits_idx, w), np.uint32)
    sign = np.zeros((planes.shape[0], mw), np.uint32)
    pos = 0
    for g in range(w):
        idx_pm[:, :, g] = planes[:, pos:pos + nbits_idx]
        pos += nbits_idx
        if g < mw:
            sign[:, g] = planes[:, pos]
            pos += 1
    return planes_to_index(idx_pm), unpack_bits(sign), s[:, 0], s[:, 1]


def unpack_value(planes, scalars, nbits: int):
    idx = planes_to_index(deinterleave(planes)[:, :nbits, :])
    return idx, np.asarray(scalars, np.float16).astype(np.float64)[:, 0]


def key_record_bytes(d_rot: int, m: int, bits: int) -> int:
    """(b-1) index planes + m sign bits + two float16 scalars."""
    return (bits - 1) * d_rot // 8 + m // 8 + 4


def value_record_bytes(d_rot: int, bits: int) -> int:
    return bits * d_rot // 8 + 2


def pack_value_blocks(idx, nbits: int) -> np.ndarray:
    """[N, d] value indices -> [ceil(N/32), d, nbits] uint32 blocked words.

    Word (B, j, p) bit i = bit p of idx[32 B + i, j]; records past N are zero.
    """
    idx = np.asarray(idx, dtype=np.int64)
    n, d = idx.shape
    nb = (n + 31) // 32
    pad = np.zeros((nb * 32, d), np.int64)
    pad[:n] = idx
    out = np.zeros((nb, d, nbits), np.uint32)
    for p in range(nbits):
        bits = ((pad >> p) & 1).reshape(nb, 32, d)          # [B, i, j]
        out[:, :, p] = pack_bits(bits.transpose(0, 2, 1).reshape(nb * d, 32)).reshape(nb, d)
    return out


def unpack_value_blocks(words, n: int) -> np.ndarray:
    """[NB, d, nbits] blocked words -> [n, d] indices."""
    words = np.asarray(words, np.uint32)
    nb, d, nbits = words.shape
    idx = np.zeros((nb * 32, d), np.int64)
    for p in range(nbits):
        bits = unpack_bits(words[:, :, p].reshape(nb * d, 1)).reshape(nb, d, 32)   # [B, j, i]
        idx |= bits.transpose(0, 2, 1).reshape(nb * 32, d).astype(np.int64) << p
    return idx[:n]


# ---- PolarQuant records ----------------------------------------------------
#
# A polar key record (d = 2^L) is a run of 32-bit words:
#   level-1 stream  the d/2 level-1 cells, cell j at bits j*b1 .. j*b1+b1-1 of a
#                   little-endian bit stream (bit k of the stream is bit k mod 32
#                   of word k div 32), ceil(d b1 / 64) words;
#   upper stream    the d/2 - 1 cells of levels 2 .. L, level by level and in
#                   ascending position within a level, b bits each, packed the
#                   same way, ceil((d/2 - 1) b / 32) words;
#   sign words      m/32 words of QJL bits (stage 2 only), bit i of the
#                   projection in bit i mod 32 of word i div 32.
# Scalars: float16 n = ||x||, and float16 gamma = ||r|| with stage 2.

def pack_stream(codes, width: int) -> np.ndarray:
    """[N, K] cells of `width` bits -> [N, ceil(K width / 32)] words (little-endian stream)."""
    codes = np.asarray(codes, np.int64)
    n, k = codes.shape
    bits = ((codes[:, :, None] >> np.arange(width)[None, None, :]) & 1).reshape(n, k * width)
    words = -(-(k * width) // 32)
    pad = np.zeros((n, words * 32), bool)
    pad[:, :k * width] = bits
    return pack_bits(pad)


def unpack_stream(words, count: int, width: int) -> np.ndarray:
    bits = unpack_bits(words)[:, :count * width].reshape(-1, count, width).astype(np.int64)
    return (bits << np.arange(width)[None, None, :]).sum(axis=2)


def polar_record_words(d: int, bits1: int, bits: int, m: int) -> int:
    return -(-(d // 2) * bits1 // 32) + -(-(d // 2 - 1) * bits // 32) + m // 32


def pack_polar(code, bits1: int, bits: int):
    """PolarCode -> (words [N, polar_record_words], scalars [N, 1 or 2] float16)."""
    l1 = pack_stream(code.codes[0], bits1)
    upper = np.concatenate([np.asarray(c, np.int64) for c in code.codes[1:]], axis=1)
    parts = [l1, pack_stream(upper, bits)]
    scal = [code.n]
    if code.z is not None:
        parts.append(pack_bits(code.z))
        scal.append(code.gamma)
    return np.ascontiguousarray(np.concatenate(parts, axis=1)), np.stack(scal, axis=1).astype(np.float16)


def unpack_polar(words, scalars, d: int, bits1: int, bits: int, m: int):
    """Record words -> (codes per level, z [N, m] or None, n [N], gamma [N] or None)."""
    words = np.asarray(words, np.uint32)
    s = np.asarray(scalars, np.float16).astype(np.float64)
    w1 = -(-(d // 2) * bits1 // 32)
    wu = -(-(d // 2 - 1) * bits // 32)
    codes = [unpack_stream(words[:, :w1], d // 2, bits1)]
    upper = unpack_stream(words[:, w1:w1 + wu], d // 2 - 1, bits)
    pos, size = 0, d // 4
    while size >= 1:
        codes.append(upper[:, pos:pos + size])
        pos += size
        size //= 2
    z = unpack_bits(words[:, w1 + wu:w1 + wu + m // 32]) if m else None
    return codes, z, s[:, 0], (s[:, 1] if m else None)
