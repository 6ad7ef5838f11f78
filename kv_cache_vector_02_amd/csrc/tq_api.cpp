// Host side of the C ABI: argument validation, codebook marshalling, dispatch.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "tq_internal.h"
#include "../../include/tq_testing.h"

namespace {

thread_local std::string g_last_error;

tq_status fail(tq_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
tq_status fail(tq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

tq_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return TQ_OK;
  return fail(TQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int index_bits(const tq_params* p, bool prod) { return prod ? p->bits - 1 : p->bits; }

// Common checks of a parameter block; fills the kernel codebook.
tq_status check_params(const tq_params* p, bool prod, tq::Codebook* cb, bool need_symmetric) {
  if (!p) return fail(TQ_ERR_INVALID_ARG, "params is NULL");
  if (p->d < 1) return fail(TQ_ERR_INVALID_ARG, "d must be >= 1 (got %d)", p->d);
  if (p->rot != TQ_ROT_DENSE && p->rot != TQ_ROT_HADAMARD && p->rot != TQ_ROT_HADAMARD2)
    return fail(TQ_ERR_INVALID_ARG, "rot must be TQ_ROT_DENSE, TQ_ROT_HADAMARD or TQ_ROT_HADAMARD2");
  if (p->rot == TQ_ROT_DENSE) {
    if (p->d_rot != p->d) return fail(TQ_ERR_INVALID_ARG, "dense rotation needs d_rot == d");
    if (!p->pi) return fail(TQ_ERR_INVALID_ARG, "dense rotation needs pi");
    if (!aligned(p->pi, 16)) return fail(TQ_ERR_INVALID_ARG, "pi must be 16-byte aligned");
  } else {
    if (p->d_rot < p->d || (p->d_rot & (p->d_rot - 1)))
      return fail(TQ_ERR_INVALID_ARG, "hadamard d_rot must be a power of two >= d");
    if (!p->eps) return fail(TQ_ERR_INVALID_ARG, "hadamard rotation needs eps");
    if (!aligned(p->eps, 16)) return fail(TQ_ERR_INVALID_ARG, "eps must be 16-byte aligned");
  }
  if (prod) {
    if (p->bits < 2 || p->bits > 4)
      return fail(TQ_ERR_INVALID_ARG, "prod bits must be in [2, 4] (got %d)", p->bits);
    if (p->m != p->d_rot && !(2 * p->m == p->d_rot && (p->d_rot == 128 || p->d_rot == 2048)))
      return fail(TQ_ERR_INVALID_ARG, "m must equal d_rot, or be d_rot / 2 at d_rot = 128 or 2048 (got m = %d)", p->m);
    if (!p->s) return fail(TQ_ERR_INVALID_ARG, "prod needs the QJL matrix s");
    if (!aligned(p->s, 16)) return fail(TQ_ERR_INVALID_ARG, "s must be 16-byte aligned");
  } else if (p->bits < 1 || p->bits > 4) {
    return fail(TQ_ERR_INVALID_ARG, "mse bits must be in [1, 4] (got %d)", p->bits);
  }
  if (!p->centroids || !p->boundaries)
    return fail(TQ_ERR_INVALID_ARG, "codebook centroids/boundaries are NULL");
  if (p->n_sets < 0 || p->set_div < 0)
    return fail(TQ_ERR_INVALID_ARG, "n_sets and set_div must be >= 0 (0 and 1 mean one set)");
  const int bq = index_bits(p, prod);
  const int K = 1 << bq;
  std::memset(cb, 0, sizeof(*cb));
  for (int i = 0; i < K; ++i) {
    float c = p->centroids[i];
    if (!std::isfinite(c)) return fail(TQ_ERR_INVALID_ARG, "centroid %d is not finite", i);
    cb->c[i] = c;
  }
  for (int i = 0; i + 1 < K; ++i) {
    float b = p->boundaries[i];
    if (!(p->centroids[i] < b && b < p->centroids[i + 1]))
      return fail(TQ_ERR_INVALID_ARG, "boundary %d must lie strictly between centroids %d and %d",
                  i, i, i + 1);
    cb->b[i] = b;
  }
  if (need_symmetric) {
    for (int i = 0; i < K; ++i)
      if (p->centroids[K - 1 - i] != -p->centroids[i])
        return fail(TQ_ERR_UNSUPPORTED, "scores/attend need an odd-symmetric codebook");
    for (int i = 0; i + 1 < K; ++i)
      if (p->boundaries[K - 2 - i] != -p->boundaries[i])
        return fail(TQ_ERR_UNSUPPORTED, "scores/attend need odd-symmetric boundaries");
  }
  return TQ_OK;
}

// prod: TurboQuant-prod keys; otherwise MSE-only, as values (token-blocked
// layout at d_rot = 128) or, with mse_keys, as per-record key records.
tq_status encode(const tq_params* p, bool prod, const void* x, int dtype, int64_t n,
                 int64_t ld_x, tq_cache out, const int64_t* slot, void* ws, size_t ws_bytes, void* stream,
                 bool mse_keys = false, bool eden = false) {
  tq::EncodeArgs a;
  std::memset(&a, 0, sizeof(a));
  tq_status st = check_params(p, prod, &a.cb, false);
  if (st != TQ_OK) return st;
  if (n < 0) return fail(TQ_ERR_INVALID_ARG, "n must be >= 0");
  if (dtype != TQ_F32 && dtype != TQ_F16) return fail(TQ_ERR_INVALID_ARG, "dtype must be TQ_F32 or TQ_F16");
  if (ld_x < p->d) return fail(TQ_ERR_INVALID_ARG, "ld_x must be >= d");
  const size_t esz = dtype == TQ_F16 ? 2 : 4;
  if (n == 0) return TQ_OK;
  if (!x || !out.planes || !out.scalars) return fail(TQ_ERR_INVALID_ARG, "x and the cache arrays must be non-NULL");
  if (out.records < 1) return fail(TQ_ERR_INVALID_ARG, "out.records (the cache's capacity) must be >= 1");
  if (!aligned(x, 16) || (ld_x * esz) % 16)
    return fail(TQ_ERR_INVALID_ARG, "x must be 16-byte aligned with rows a multiple of 16 bytes");
  if (!aligned(out.planes, 16) || !aligned(out.scalars, 4))
    return fail(TQ_ERR_INVALID_ARG, "cache planes must be 16-byte and scalars 4-byte aligned");
  if (slot && !aligned(slot, 8)) return fail(TQ_ERR_INVALID_ARG, "slot must be 8-byte aligned");
  a.x = x;
  a.f16_in = dtype == TQ_F16;
  a.n = n;
  a.ld_x = ld_x;
  a.d = p->d;
  a.pi = p->pi;
  a.eps = p->eps;
  a.s = prod ? p->s : nullptr;
  a.bq = index_bits(p, prod);
  a.prod = prod || mse_keys;
  a.qjl = prod;
  a.m = prod ? p->m : 0;
  a.eden = eden;
  const bool fwht2k = p->rot != TQ_ROT_DENSE && p->d_rot == 2048;     // one or two rounds in registers
  if (p->rot == TQ_ROT_HADAMARD2 && !fwht2k)
    return fail(TQ_ERR_UNSUPPORTED, "two Hadamard rounds run natively at d_rot = 2048; at d_rot = 128 pass "
                                    "tq_hadamard_matrix's matrix as a dense rotation");
  if (eden && !(p->d == 128 && p->d_rot == 128) && !fwht2k)
    return fail(TQ_ERR_UNSUPPORTED, "tq_encode_eden supports d = d_rot = 128 and the Hadamard rotation at d_rot = 2048");
  a.planes = (uint32_t*)out.planes;
  a.scalars = (uint16_t*)out.scalars;
  a.slot = slot;
  a.records = out.records;
  a.had = p->rot != TQ_ROT_DENSE;
  a.rounds = p->rot == TQ_ROT_HADAMARD2 ? 2 : 1;
  hipStream_t s = (hipStream_t)stream;
  if (p->d == 128 && p->d_rot == 128)
    return hip_status(tq::launch_encode_dense128(a, s), "encode launch");
  if (prod && fwht2k) {
    if (p->d % 8) return fail(TQ_ERR_UNSUPPORTED, "d_rot = 2048 encode needs d a multiple of 8 (got %d)", p->d);
    const size_t need = tq::encode2k_workspace(n);
    if (!ws) return fail(TQ_ERR_INVALID_ARG, "d_rot = 2048 encode needs a workspace (tq_encode_prod_ws)");
    if (!aligned(ws, 256)) return fail(TQ_ERR_INVALID_ARG, "ws must be 256-byte aligned");
    if (ws_bytes < need) return fail(TQ_ERR_INVALID_ARG, "workspace too small: %zu < %zu", ws_bytes, need);
    return hip_status(tq::launch_encode2k(a, ws, s), "encode launch");
  }
  if (!prod && fwht2k) {
    if (p->d % 8) return fail(TQ_ERR_UNSUPPORTED, "d_rot = 2048 encode needs d a multiple of 8 (got %d)", p->d);
    return hip_status(tq::launch_encode2k_mse(a, s), "encode launch");
  }
  return fail(TQ_ERR_UNSUPPORTED,
              "encode supports d = d_rot = 128, and the Hadamard rotation at d_rot = 2048 "
              "(got %s, rot %d, d %d, d_rot %d)", prod ? "prod" : "mse", p->rot, p->d, p->d_rot);
}

// PolarQuant parameter block: checks, then the codebook tables in float64
// rounded once to float32.
tq_status polar_params(const tq_polar_params* p, tq::PolarArgs* a) {
  std::memset(a, 0, sizeof(*a));
  if (!p) return fail(TQ_ERR_INVALID_ARG, "params is NULL");
  if (p->d != 128) return fail(TQ_ERR_UNSUPPORTED, "polar records support d = 128 (got %d)", p->d);
  if (p->rot == TQ_ROT_DENSE) {
    if (!p->pi || !aligned(p->pi, 16)) return fail(TQ_ERR_INVALID_ARG, "dense rotation needs a 16-byte aligned pi");
  } else if (p->rot == TQ_ROT_HADAMARD) {
    if (!p->eps || !aligned(p->eps, 16)) return fail(TQ_ERR_INVALID_ARG, "hadamard rotation needs a 16-byte aligned eps");
  } else if (p->rot == TQ_ROT_HADAMARD2) {
    return fail(TQ_ERR_UNSUPPORTED, "two Hadamard rounds: pass tq_hadamard_matrix's matrix as a dense rotation");
  } else {
    return fail(TQ_ERR_INVALID_ARG, "rot must be TQ_ROT_DENSE or TQ_ROT_HADAMARD");
  }
  if (p->bits1 < 1 || p->bits1 > 4 || p->bits < 1 || p->bits > 4)
    return fail(TQ_ERR_INVALID_ARG, "bits1 and bits must be in [1, 4] (got %d, %d)", p->bits1, p->bits);
  if (p->m != 0 && p->m != p->d) return fail(TQ_ERR_INVALID_ARG, "m must be 0 or d (got %d)", p->m);
  if (p->m && (!p->s || !aligned(p->s, 16))) return fail(TQ_ERR_INVALID_ARG, "m > 0 needs a 16-byte aligned s");
  if (!p->centroids || !p->boundaries) return fail(TQ_ERR_INVALID_ARG, "codebook centroids/boundaries are NULL");
  const int L = 7;
  int co = 0, bo = 0;   // offsets of the current level in the host arrays
  for (int l = 1; l <= L; ++l) {
    const int K = 1 << (l == 1 ? p->bits1 : p->bits);
    const double lo = l == 1 ? -M_PI : 0.0, hi = l == 1 ? M_PI : M_PI / 2;
    for (int i = 0; i < K; ++i)
      if (!std::isfinite(p->centroids[co + i]))
        return fail(TQ_ERR_INVALID_ARG, "level %d centroid %d is not finite", l, i);
    for (int i = 0; i + 1 < K; ++i) {
      const float b = p->boundaries[bo + i];
      if (!(p->centroids[co + i] < b && b < p->centroids[co + i + 1]) || !((double)b > lo && (double)b < hi))
        return fail(TQ_ERR_INVALID_ARG, "level %d boundary %d must lie between its centroids and inside (%g, %g)",
                    l, i, lo, hi);
    }
    for (int i = 0; i < K; ++i) {
      const double c = p->centroids[co + i];
      float* dst = l == 1 ? a->book.c1[i] : a->book.cu[l - 2][i];
      dst[0] = (float)std::cos(c);
      dst[1] = (float)std::sin(c);
    }
    for (int i = 0; i + 1 < K; ++i) {
      const double b = p->boundaries[bo + i];
      if (l == 1) {
        a->book.b1[i] = (float)b;
      } else {
        const double cb = std::cos(b), sb = std::sin(b);
        a->book.bc[l - 2][i] = (float)(cb * cb);
        a->book.bs[l - 2][i] = (float)(sb * sb);
      }
    }
    co += K;
    bo += K - 1;
  }
  a->pi = p->pi;
  a->eps = p->eps;
  a->s = p->m ? p->s : nullptr;
  a->had = p->rot == TQ_ROT_HADAMARD;
  a->b1 = p->bits1;
  a->b = p->bits;
  a->qjl = p->m ? 1 : 0;
  return TQ_OK;
}

int polar_words(const tq_polar_params* p) { return 2 * p->bits1 + 2 * p->bits + p->m / 32; }

}  // namespace

extern "C" {

const char* tq_status_string(int s) {
  switch (s) {
    case TQ_OK: return "TQ_OK";
    case TQ_ERR_INVALID_ARG: return "TQ_ERR_INVALID_ARG";
    case TQ_ERR_UNSUPPORTED: return "TQ_ERR_UNSUPPORTED";
    case TQ_ERR_HIP: return "TQ_ERR_HIP";
  }
  return "unknown tq_status";
}

const char* tq_last_error(void) { return g_last_error.c_str(); }

tq_status tq_build_codebook(int d, int bits, double* centroids, double* boundaries) {
  if (!(d == 0 || (d >= 2 && d <= 65536))) return fail(TQ_ERR_INVALID_ARG, "d must be 0 or in [2, 65536]");
  if (bits < 1 || bits > 4) return fail(TQ_ERR_INVALID_ARG, "bits must be in [1, 4]");
  if (!centroids || !boundaries) return fail(TQ_ERR_INVALID_ARG, "output arrays are NULL");
  return tq::build_codebook(d, bits, centroids, boundaries);
}

tq_status tq_key_layout(const tq_params* p, int* planes, int* words, int* scalars) {
  tq::Codebook cb;
  const bool qjl = p && p->s;     // no QJL matrix: MSE-only key records
  tq_status st = check_params(p, qjl, &cb, false);
  if (st != TQ_OK) return st;
  if (planes) *planes = p->bits;
  if (words) *words = p->d_rot / 32;
  if (scalars) *scalars = qjl ? 2 : 1;
  return TQ_OK;
}

size_t tq_key_record_words(const tq_params* p) {
  tq::Codebook cb;
  const bool qjl = p && p->s;
  if (check_params(p, qjl, &cb, false) != TQ_OK) return 0;
  const int w = p->d_rot / 32;
  return qjl ? (size_t)w * (p->bits - 1) + p->m / 32 : (size_t)w * p->bits;
}

size_t tq_key_record_bytes(const tq_params* p) {
  const size_t w = tq_key_record_words(p);
  return w ? 4 * w + 2 * (p->s ? 2 : 1) : 0;
}

size_t tq_val_record_bytes(const tq_params* p) {
  tq::Codebook cb;
  if (check_params(p, false, &cb, false) != TQ_OK) return 0;
  return (size_t)p->d_rot * p->bits / 8 + 2;
}

tq_status tq_value_layout(const tq_params* p, int* planes, int* words, int* scalars) {
  tq::Codebook cb;
  tq_status st = check_params(p, false, &cb, false);
  if (st != TQ_OK) return st;
  if (planes) *planes = p->bits;
  if (words) *words = p->d_rot / 32;
  if (scalars) *scalars = 1;
  return TQ_OK;
}

tq_status tq_encode_prod(const tq_params* p, const void* x, int dtype, int64_t n, int64_t ld_x,
                         tq_cache out, const int64_t* slot, void* stream) {
  return encode(p, true, x, dtype, n, ld_x, out, slot, nullptr, 0, stream);
}

tq_status tq_hadamard_matrix(const float* eps, int rounds, int d, int d_rot, float* out, void* stream) {
  if (d_rot < 2 || d_rot > 2048 || (d_rot & (d_rot - 1)))
    return fail(TQ_ERR_INVALID_ARG, "d_rot must be a power of two in [2, 2048] (got %d)", d_rot);
  if (d < 1 || d > d_rot) return fail(TQ_ERR_INVALID_ARG, "need 1 <= d <= d_rot (got d = %d)", d);
  if (rounds < 1 || rounds > 2) return fail(TQ_ERR_INVALID_ARG, "rounds must be 1 or 2 (got %d)", rounds);
  if (!eps || !out) return fail(TQ_ERR_INVALID_ARG, "eps and out must be non-NULL");
  if (!aligned(eps, 4) || !aligned(out, 4)) return fail(TQ_ERR_INVALID_ARG, "eps and out must be 4-byte aligned");
  return hip_status(tq::launch_hadamard_matrix(eps, rounds, d, d_rot, out, (hipStream_t)stream),
                    "hadamard matrix launch");
}

size_t tq_encode_workspace(const tq_params* p, int64_t n) {
  if (!p || n <= 0) return 0;
  if (p->d_rot == 2048 && p->rot != TQ_ROT_DENSE && p->s) return tq::encode2k_workspace(n);
  return 0;
}

tq_status tq_encode_prod_ws(const tq_params* p, const void* x, int dtype, int64_t n, int64_t ld_x,
                            tq_cache out, const int64_t* slot, void* ws, size_t ws_bytes, void* stream) {
  return encode(p, true, x, dtype, n, ld_x, out, slot, ws, ws_bytes, stream);
}

tq_status tq_encode_mse(const tq_params* p, const void* x, int dtype, int64_t n, int64_t ld_x,
                        tq_cache out, const int64_t* slot, void* stream) {
  return encode(p, false, x, dtype, n, ld_x, out, slot, nullptr, 0, stream);
}

tq_status tq_encode_mse_keys(const tq_params* p, const void* x, int dtype, int64_t n, int64_t ld_x,
                             tq_cache out, const int64_t* slot, void* stream) {
  return encode(p, false, x, dtype, n, ld_x, out, slot, nullptr, 0, stream, true);
}

tq_status tq_encode_eden(const tq_params* p, const void* x, int dtype, int64_t n, int64_t ld_x,
                         int layout, tq_cache out, const int64_t* slot, void* stream) {
  if (layout != TQ_LAYOUT_BLOCKS && layout != TQ_LAYOUT_RECORDS)
    return fail(TQ_ERR_INVALID_ARG, "layout must be TQ_LAYOUT_BLOCKS or TQ_LAYOUT_RECORDS");
  return encode(p, false, x, dtype, n, ld_x, out, slot, nullptr, 0, stream, layout == TQ_LAYOUT_RECORDS, true);
}

size_t tq_scores_workspace(const tq_params* kp, int segs, int group) {
  (void)kp;
  if (segs <= 0 || group <= 0) return 0;
  return tq::scores128_workspace(segs, group);
}

// Validation and argument set-up shared by the score entry points; q may be
// NULL when need_q is false (score pass over an already prepared pack).
static tq_status score_args(const tq_params* kp, const float* q, bool need_q, int segs, int group,
                            tq_cache keys, bool need_keys, const int32_t* len, int64_t T, float* scores,
                            bool need_scores, void* ws, size_t ws_bytes, tq::ScoreArgs* a, bool* nothing) {
  std::memset(a, 0, sizeof(*a));
  *nothing = false;
  const bool qjl = kp && kp->s;     // no QJL matrix: MSE-only keys
  tq_status st = check_params(kp, qjl, &a->cb, true);
  if (st != TQ_OK) return st;
  if (segs < 0 || group < 1 || T < 0) return fail(TQ_ERR_INVALID_ARG, "need segs >= 0, group >= 1, T >= 0");
  if (segs == 0 || (need_keys && T == 0)) {
    *nothing = true;
    return TQ_OK;
  }
  if (kp->d != 128 || kp->d_rot != 128)
    return fail(TQ_ERR_UNSUPPORTED, "tq_scores supports d = d_rot = 128 (got %d, %d)", kp->d, kp->d_rot);
  if (kp->rot == TQ_ROT_HADAMARD2)
    return fail(TQ_ERR_UNSUPPORTED, "at d_rot = 128 pass tq_hadamard_matrix's two-round matrix as a dense rotation");
  if (group > 16) return fail(TQ_ERR_UNSUPPORTED, "tq_scores supports up to 16 query heads per segment");
  if ((need_q && !q) || (need_keys && (!keys.planes || !keys.scalars)) || (need_scores && !scores) || !ws)
    return fail(TQ_ERR_INVALID_ARG, "q, keys, scores and ws must be non-NULL");
  if (need_keys && keys.seg_stride < T && segs > 1) return fail(TQ_ERR_INVALID_ARG, "keys.seg_stride must be >= T");
  if ((need_keys && (!aligned(keys.planes, 16) || !aligned(keys.scalars, 4))) || !aligned(ws, 256) ||
      (need_q && !aligned(q, 16)) || (need_scores && !aligned(scores, 4)))
    return fail(TQ_ERR_INVALID_ARG, "misaligned pointer (q and planes 16 B, scalars 4 B, ws 256 B)");
  const size_t need = tq::scores128_workspace(segs, group);
  if (ws_bytes < need) return fail(TQ_ERR_INVALID_ARG, "workspace too small: %zu < %zu", ws_bytes, need);
  const int64_t stride = segs == 1 && keys.seg_stride < T ? T : keys.seg_stride;
  if (need_keys && (int64_t)(segs - 1) * stride + T > keys.records)
    return fail(TQ_ERR_INVALID_ARG, "the keys read (%lld records) exceed keys.records (%lld)",
                (long long)((int64_t)(segs - 1) * stride + T), (long long)keys.records);
  if (need_keys && (stride * 16 * kp->bits >= (1ll << 31) || (int64_t)group * T * 4 >= (1ll << 31)))
    return fail(TQ_ERR_UNSUPPORTED, "tq_scores addresses at most 2 GiB of keys and of scores per segment");
  a->q = q;
  a->segs = segs;
  a->group = group;
  a->d = kp->d;
  a->pi = kp->pi;
  a->eps = kp->eps;
  a->rot = kp->rot;
  a->s = kp->s;
  a->m = qjl ? kp->m : 0;
  a->bq = qjl ? kp->bits - 1 : kp->bits;
  a->qjl = qjl;
  a->planes = (const uint32_t*)keys.planes;
  a->scalars = (const uint16_t*)keys.scalars;
  a->seg_stride = stride;
  a->len = len;
  a->T = T;
  a->scores = scores;
  a->ws = ws;
  a->wait_us = tq::PACK_WAIT_US;
  a->n_sets = kp->n_sets;
  a->set_div = kp->set_div;
  return TQ_OK;
}

tq_status tq_scores(const tq_params* kp, const float* q, int segs, int group, tq_cache keys,
                    const int32_t* len, int64_t T, float* scores, void* ws, size_t ws_bytes,
                    void* stream) {
  tq::ScoreArgs a;
  bool nothing;
  tq_status st = score_args(kp, q, true, segs, group, keys, true, len, T, scores, true, ws, ws_bytes, &a, &nothing);
  if (st != TQ_OK || nothing) return st;
  return hip_status(tq::launch_scores128(a, (hipStream_t)stream), "scores launch");
}

tq_status tq_testing_scores_wait(const tq_params* kp, const float* q, int segs, int group, tq_cache keys,
                                 const int32_t* len, int64_t T, float* scores, void* ws, size_t ws_bytes,
                                 int wait_us, void* stream) {
  tq::ScoreArgs a;
  bool nothing;
  if (wait_us < 0) return fail(TQ_ERR_INVALID_ARG, "wait_us must be >= 0");
  tq_status st = score_args(kp, q, true, segs, group, keys, true, len, T, scores, true, ws, ws_bytes, &a, &nothing);
  if (st != TQ_OK || nothing) return st;
  a.wait_us = wait_us;
  a.one_launch = 1;
  return hip_status(tq::launch_scores128(a, (hipStream_t)stream), "scores launch");
}

tq_status tq_scores_noalloc(const tq_params* kp, const float* q, int segs, int group, tq_cache keys,
                            const int32_t* len, int64_t T, float* scores, void* stream) {
  void* ws = nullptr;
  size_t ws_bytes = 0;
  tq_status st = hip_status(tq::scores_scratch(&ws, &ws_bytes), "resolving the scratch array");
  if (st != TQ_OK) return st;
  if (segs > 0 && group > 0 && tq::scores128_workspace(segs, group) > ws_bytes)
    return fail(TQ_ERR_UNSUPPORTED, "tq_scores_noalloc: %d segments x %d heads need %zu bytes of workspace, more "
                "than its %zu-byte scratch array (use tq_scores with a workspace)", segs, group,
                tq::scores128_workspace(segs, group), ws_bytes);
  tq::ScoreArgs a;
  bool nothing;
  st = score_args(kp, q, true, segs, group, keys, true, len, T, scores, true, ws, ws_bytes, &a, &nothing);
  if (st != TQ_OK || nothing) return st;
  return hip_status(tq::launch_scores128(a, (hipStream_t)stream), "scores launch");
}

size_t tq_scores_noalloc_capacity(void) { return tq::SCORES_SCRATCH_BYTES; }

tq_status tq_scores_prepare(const tq_params* kp, const float* q, int segs, int group, void* ws,
                            size_t ws_bytes, void* stream) {
  tq::ScoreArgs a;
  bool nothing;
  tq_cache none = {nullptr, nullptr, 0, 0};
  tq_status st = score_args(kp, q, true, segs, group, none, false, nullptr, 1, nullptr, false, ws, ws_bytes, &a,
                            &nothing);
  if (st != TQ_OK || nothing) return st;
  return hip_status(tq::launch_scores128_prepare(a, (hipStream_t)stream), "scores prepare launch");
}

tq_status tq_scores_prepared(const tq_params* kp, int segs, int group, tq_cache keys, const int32_t* len,
                             int64_t T, float* scores, void* ws, size_t ws_bytes, void* stream) {
  tq::ScoreArgs a;
  bool nothing;
  tq_status st = score_args(kp, nullptr, false, segs, group, keys, true, len, T, scores, true, ws, ws_bytes, &a,
                            &nothing);
  if (st != TQ_OK || nothing) return st;
  return hip_status(tq::launch_scores128_prepared(a, (hipStream_t)stream), "scores launch");
}

// 4-bit MSE-only keys carry 16 key fragments per 16-row tile, so at most two
// tiles (8 query heads) fit one attention workgroup's registers; a segment
// with an even group of 10..16 heads runs as two query segments of group / 2
// heads that read the same keys and values (the query and output rows of the
// halves are the segment's rows in order).  Returns the divisor (1 or 2).
static int attend_head_split(const tq_params* kp, int group) {
  return kp && !kp->s && kp->bits == 4 && group > 8 ? 2 : 1;
}

size_t tq_attend_workspace(const tq_params* kp, const tq_params* vp, int segs, int group, int64_t T) {
  (void)vp;
  if (segs <= 0 || group <= 0 || T <= 0) return 0;
  const int div = attend_head_split(kp, group);
  return tq::attend128_workspace(segs * div, (group + div - 1) / div, T);
}

// tq_attend and its two halves.  ATT_PREPARE checks and fills the query side
// only (vp, keys, vals, len, T, scale and out unused); ATT_PREPARED takes the
// pack from ws (q unused).
enum { ATT_FULL = 0, ATT_PREPARE = 1, ATT_PREPARED = 2 };

static tq_status attend_args(int mode, const tq_params* kp, const tq_params* vp, const float* q, int segs,
                             int group, tq_cache keys, tq_cache vals, const int32_t* len, int64_t T, float scale,
                             float* out, void* ws, size_t ws_bytes, tq::AttendArgs* ap, bool* nothing) {
  tq::AttendArgs& a = *ap;
  std::memset(&a, 0, sizeof(a));
  *nothing = false;
  const bool with_kv = mode != ATT_PREPARE;
  const bool qjl = kp && kp->s;     // no QJL matrix: MSE-only keys
  tq_status st = check_params(kp, qjl, &a.k.cb, true);
  if (st != TQ_OK) return st;
  if (with_kv) {
    st = check_params(vp, false, &a.cb_v, true);
    if (st != TQ_OK) return st;
  }
  if (segs < 0 || group < 1 || (with_kv && T < 0)) return fail(TQ_ERR_INVALID_ARG, "need segs >= 0, group >= 1, T >= 0");
  if (with_kv && !std::isfinite(scale)) return fail(TQ_ERR_INVALID_ARG, "scale must be finite");
  if (segs == 0) {
    *nothing = true;
    return TQ_OK;
  }
  if (kp->d != 128 || kp->d_rot != 128 || (with_kv && (vp->d != 128 || vp->d_rot != 128)))
    return fail(TQ_ERR_UNSUPPORTED, "tq_attend supports d = d_rot = 128 for keys and values");
  if (kp->rot == TQ_ROT_HADAMARD2 || (with_kv && vp->rot == TQ_ROT_HADAMARD2))
    return fail(TQ_ERR_UNSUPPORTED, "at d_rot = 128 pass tq_hadamard_matrix's two-round matrix as a dense rotation");
  if (group > 16) return fail(TQ_ERR_UNSUPPORTED, "tq_attend supports up to 16 query heads per segment");
  if (with_kv && qjl && kp->m != kp->d_rot && vp->bits < 2)
    return fail(TQ_ERR_UNSUPPORTED, "tq_attend with m = d / 2 keys supports value bits 2..4");
  if (!qjl && (kp->bits < 2 || (with_kv && vp->bits < 2)))
    return fail(TQ_ERR_UNSUPPORTED, "tq_attend with MSE-only keys supports key and value bits 2..4");
  const int div = attend_head_split(kp, group);
  if (div == 2 && group % 2)
    return fail(TQ_ERR_UNSUPPORTED, "tq_attend with 4-bit MSE-only keys supports up to 8, or an even number up "
                                    "to 16, query heads per segment");
  if (mode != ATT_PREPARED && (!q || !aligned(q, 16))) return fail(TQ_ERR_INVALID_ARG, "q must be non-NULL and 16-byte aligned");
  if (!ws || !aligned(ws, 256)) return fail(TQ_ERR_INVALID_ARG, "ws must be non-NULL and 256-byte aligned");
  a.k.q = q;
  a.k.segs = segs * div;
  a.k.group = group / div;
  a.kv_div = div;
  a.k.n_sets = kp->n_sets;
  a.k.set_div = (kp->set_div > 1 ? kp->set_div : 1) * div;   // sets follow the cache segment
  a.k.d = kp->d;
  a.k.pi = kp->pi;
  a.k.eps = kp->eps;
  a.k.rot = kp->rot;
  a.k.s = kp->s;
  a.k.m = qjl ? kp->m : 0;
  a.k.bq = qjl ? kp->bits - 1 : kp->bits;
  a.k.qjl = qjl;
  a.k.ws = ws;
  a.ws = ws;
  a.prepared = mode == ATT_PREPARED;
  if (!with_kv) {
    const size_t need = tq::scores128_workspace(segs * div, group / div);
    if (ws_bytes < need) return fail(TQ_ERR_INVALID_ARG, "workspace too small: %zu < %zu", ws_bytes, need);
    return TQ_OK;
  }
  if (!keys.planes || !keys.scalars || !vals.planes || !vals.scalars || !out)
    return fail(TQ_ERR_INVALID_ARG, "keys, vals and out must be non-NULL");
  if (vals.seg_stride % 32) return fail(TQ_ERR_INVALID_ARG, "vals.seg_stride must be a multiple of 32");
  if (segs > 1 && (keys.seg_stride < T || vals.seg_stride < T))
    return fail(TQ_ERR_INVALID_ARG, "seg_stride must be >= T for keys and values");
  if (!aligned(keys.planes, 16) || !aligned(keys.scalars, 4) || !aligned(vals.planes, 16) ||
      !aligned(vals.scalars, 4) || !aligned(out, 4))
    return fail(TQ_ERR_INVALID_ARG, "misaligned pointer (q and planes 16 B, scalars 4 B, ws 256 B)");
  if (T == 0) return fail(TQ_ERR_INVALID_ARG, "T must be >= 1");
  const size_t need = tq::attend128_workspace(segs * div, group / div, T);
  if (ws_bytes < need) return fail(TQ_ERR_INVALID_ARG, "workspace too small: %zu < %zu", ws_bytes, need);
  const int64_t kstride = segs == 1 && keys.seg_stride < T ? T : keys.seg_stride;
  const int64_t vstride = segs == 1 && vals.seg_stride < T ? (T + 31) / 32 * 32 : vals.seg_stride;
  if ((int64_t)(segs - 1) * kstride + T > keys.records || (int64_t)(segs - 1) * vstride + T > vals.records)
    return fail(TQ_ERR_INVALID_ARG, "the keys or values read exceed keys.records / vals.records");
  if (kstride * 16 * kp->bits >= (1ll << 31) || vstride * 16 * vp->bits >= (1ll << 31))
    return fail(TQ_ERR_UNSUPPORTED, "tq_attend addresses at most 2 GiB of keys and of values per segment");
  a.n_sets_v = vp->n_sets;
  a.set_div_v = vp->set_div;
  a.k.planes = (const uint32_t*)keys.planes;
  a.k.scalars = (const uint16_t*)keys.scalars;
  a.k.seg_stride = kstride;
  a.k.len = len;
  a.k.T = T;
  a.pi_v = vp->pi;
  a.eps_v = vp->eps;
  a.rot_v = vp->rot;
  a.bq_v = vp->bits;
  a.planes_v = (const uint32_t*)vals.planes;
  a.scalars_v = (const uint16_t*)vals.scalars;
  a.seg_stride_v = vstride;
  a.scale = scale;
  a.out = out;
  return TQ_OK;
}

tq_status tq_attend(const tq_params* kp, const tq_params* vp, const float* q, int segs, int group,
                    tq_cache keys, tq_cache vals, const int32_t* len, int64_t T, float scale,
                    float* out, void* ws, size_t ws_bytes, void* stream) {
  tq::AttendArgs a;
  bool nothing;
  tq_status st = attend_args(ATT_FULL, kp, vp, q, segs, group, keys, vals, len, T, scale, out, ws, ws_bytes, &a,
                             &nothing);
  if (st != TQ_OK || nothing) return st;
  return hip_status(tq::launch_attend128(a, (hipStream_t)stream), "attend launch");
}

tq_status tq_attend_prepare(const tq_params* kp, const float* q, int segs, int group, void* ws, size_t ws_bytes,
                            void* stream) {
  tq::AttendArgs a;
  bool nothing;
  tq_cache none = {nullptr, nullptr, 0, 0};
  tq_status st = attend_args(ATT_PREPARE, kp, nullptr, q, segs, group, none, none, nullptr, 0, 0.f, nullptr, ws,
                             ws_bytes, &a, &nothing);
  if (st != TQ_OK || nothing) return st;
  return hip_status(tq::launch_attend128_prepare(a, (hipStream_t)stream), "attend prepare launch");
}

tq_status tq_attend_prepared(const tq_params* kp, const tq_params* vp, int segs, int group, tq_cache keys,
                             tq_cache vals, const int32_t* len, int64_t T, float scale, float* out, void* ws,
                             size_t ws_bytes, void* stream) {
  tq::AttendArgs a;
  bool nothing;
  tq_status st = attend_args(ATT_PREPARED, kp, vp, nullptr, segs, group, keys, vals, len, T, scale, out, ws,
                             ws_bytes, &a, &nothing);
  if (st != TQ_OK || nothing) return st;
  return hip_status(tq::launch_attend128(a, (hipStream_t)stream), "attend launch");
}

size_t tq_scores_topk_workspace(const tq_params* kp, int nq, int64_t T, int k) {
  if (!kp || nq <= 0 || T <= 0 || k <= 0) return 0;
  const bool qjl = kp->s != nullptr;
  return tq::topk2k_workspace(nq, T, k, qjl ? kp->bits - 1 : kp->bits, qjl);
}

tq_status tq_scores_topk(const tq_params* kp, const float* q, int nq, tq_cache keys, int64_t T, int k,
                         int64_t* idx, float* val, void* ws, size_t ws_bytes, void* stream) {
  // with the QJL matrix s: prod keys; without it: MSE-only records
  tq::Codebook cb;
  const bool qjl = kp && kp->s;
  tq_status st = check_params(kp, qjl, &cb, true);
  if (st != TQ_OK) return st;
  if (nq < 0 || T < 0 || k < 1) return fail(TQ_ERR_INVALID_ARG, "need nq >= 0, T >= 0, k >= 1");
  if (nq == 0) return TQ_OK;
  if (kp->rot == TQ_ROT_DENSE || kp->d_rot != 2048)
    return fail(TQ_ERR_UNSUPPORTED, "tq_scores_topk supports the Hadamard rotation (one or two rounds) at d_rot = 2048");
  if (kp->n_sets > 1) return fail(TQ_ERR_UNSUPPORTED, "tq_scores_topk takes one rotation set");
  if (kp->d % 4) return fail(TQ_ERR_UNSUPPORTED, "tq_scores_topk needs d a multiple of 4 (got %d)", kp->d);
  if (k > 16) return fail(TQ_ERR_UNSUPPORTED, "tq_scores_topk supports k <= 16");
  if (T < k) return fail(TQ_ERR_INVALID_ARG, "need T >= k");
  if (T > keys.records) return fail(TQ_ERR_INVALID_ARG, "T exceeds keys.records");
  if (!q || !keys.planes || !keys.scalars || !idx || !val || !ws)
    return fail(TQ_ERR_INVALID_ARG, "q, keys, idx, val and ws must be non-NULL");
  if (!aligned(q, 16) || !aligned(keys.planes, 16) || !aligned(keys.scalars, 4) || !aligned(ws, 256) ||
      !aligned(idx, 8) || !aligned(val, 4))
    return fail(TQ_ERR_INVALID_ARG, "misaligned pointer (q and planes 16 B, scalars 4 B, ws 256 B)");
  const int bq = index_bits(kp, qjl);
  const size_t need = tq::topk2k_workspace(nq, T, k, bq, qjl);
  if (ws_bytes < need) return fail(TQ_ERR_INVALID_ARG, "workspace too small: %zu < %zu", ws_bytes, need);
  tq::TopkLaunch L;
  L.q = q;
  L.nq = nq;
  L.d = kp->d;
  L.bq = bq;
  L.qjl = qjl;
  L.k = k;
  L.eps = kp->eps;
  L.rounds = kp->rot == TQ_ROT_HADAMARD2 ? 2 : 1;
  L.s = kp->s;
  L.m = qjl ? kp->m : 0;
  tq::walsh_coefficients(cb, L.bq, L.u, &L.usum);
  L.planes = (const uint32_t*)keys.planes;
  L.scalars = (const uint16_t*)keys.scalars;
  L.T = T;
  L.idx = idx;
  L.val = val;
  L.ws = ws;
  return hip_status(tq::launch_topk2k(L, (hipStream_t)stream), "top-k launch");
}

tq_status tq_build_polar_codebook(int level, int bits, double* centroids, double* boundaries) {
  if (level < 1 || level > 16) return fail(TQ_ERR_INVALID_ARG, "level must be in [1, 16]");
  if (bits < 1 || bits > 4) return fail(TQ_ERR_INVALID_ARG, "bits must be in [1, 4]");
  if (!centroids || !boundaries) return fail(TQ_ERR_INVALID_ARG, "output arrays are NULL");
  return tq::build_polar_codebook(level, bits, centroids, boundaries);
}

size_t tq_polar_record_words(const tq_polar_params* p) {
  tq::PolarArgs a;
  if (polar_params(p, &a) != TQ_OK) return 0;
  return (size_t)polar_words(p);
}

tq_status tq_polar_encode(const tq_polar_params* p, const void* x, int dtype, int64_t n, int64_t ld_x,
                          tq_cache out, const int64_t* slot, void* stream) {
  tq::PolarArgs a;
  tq_status st = polar_params(p, &a);
  if (st != TQ_OK) return st;
  if (n < 0) return fail(TQ_ERR_INVALID_ARG, "n must be >= 0");
  if (dtype != TQ_F32 && dtype != TQ_F16) return fail(TQ_ERR_INVALID_ARG, "dtype must be TQ_F32 or TQ_F16");
  if (ld_x < p->d) return fail(TQ_ERR_INVALID_ARG, "ld_x must be >= d");
  const size_t esz = dtype == TQ_F16 ? 2 : 4;
  if (n == 0) return TQ_OK;
  if (!x || !out.planes || !out.scalars) return fail(TQ_ERR_INVALID_ARG, "x and the cache arrays must be non-NULL");
  if (out.records < 1) return fail(TQ_ERR_INVALID_ARG, "out.records (the cache's capacity) must be >= 1");
  if (!aligned(x, 16) || (ld_x * esz) % 16)
    return fail(TQ_ERR_INVALID_ARG, "x must be 16-byte aligned with rows a multiple of 16 bytes");
  if (!aligned(out.planes, 8) || !aligned(out.scalars, 4))
    return fail(TQ_ERR_INVALID_ARG, "cache planes must be 8-byte and scalars 4-byte aligned");
  if (slot && !aligned(slot, 8)) return fail(TQ_ERR_INVALID_ARG, "slot must be 8-byte aligned");
  a.x = x;
  a.f16_in = dtype == TQ_F16;
  a.n = n;
  a.ld_x = ld_x;
  a.slot = slot;
  a.planes = (uint32_t*)out.planes;
  a.scalars = (uint16_t*)out.scalars;
  a.records = out.records;
  return hip_status(tq::launch_polar_encode128(a, (hipStream_t)stream), "polar encode launch");
}

tq_status tq_polar_decode(const tq_polar_params* p, tq_cache in, int64_t n, float* out, int64_t ld_out,
                          void* stream) {
  tq::PolarArgs a;
  tq_status st = polar_params(p, &a);
  if (st != TQ_OK) return st;
  if (n < 0) return fail(TQ_ERR_INVALID_ARG, "n must be >= 0");
  if (ld_out < p->d) return fail(TQ_ERR_INVALID_ARG, "ld_out must be >= d");
  if (n == 0) return TQ_OK;
  if (!in.planes || !in.scalars || !out) return fail(TQ_ERR_INVALID_ARG, "the cache arrays and out must be non-NULL");
  if (n > in.records) return fail(TQ_ERR_INVALID_ARG, "n (%lld) exceeds in.records (%lld)", (long long)n,
                                  (long long)in.records);
  if (!aligned(in.planes, 4) || !aligned(in.scalars, 2) || !aligned(out, 4))
    return fail(TQ_ERR_INVALID_ARG, "misaligned pointer (planes and out 4 B, scalars 2 B)");
  a.planes = (uint32_t*)in.planes;
  a.scalars = (uint16_t*)in.scalars;
  a.records = in.records;
  a.n = n;
  a.out = out;
  a.ld_out = ld_out;
  return hip_status(tq::launch_polar_decode128(a, (hipStream_t)stream), "polar decode launch");
}

tq_status tq_polar_scores(const tq_polar_params* p, const float* q, int segs, int group, tq_cache keys,
                          const int32_t* len, int64_t T, float* scores, void* stream) {
  tq::PolarArgs a;
  tq_status st = polar_params(p, &a);
  if (st != TQ_OK) return st;
  if (segs < 0 || group < 1 || T < 0) return fail(TQ_ERR_INVALID_ARG, "need segs >= 0, group >= 1, T >= 0");
  if (group > 16) return fail(TQ_ERR_UNSUPPORTED, "polar scores support up to 16 query heads per segment");
  if (segs == 0 || T == 0) return TQ_OK;
  if (!q || !keys.planes || !keys.scalars || !scores)
    return fail(TQ_ERR_INVALID_ARG, "q, keys and scores must be non-NULL");
  if (!aligned(q, 16) || !aligned(keys.planes, 8) || !aligned(keys.scalars, 4) || !aligned(scores, 4) ||
      (len && !aligned(len, 4)))
    return fail(TQ_ERR_INVALID_ARG, "misaligned pointer (q 16 B, planes 8 B, scalars, scores and len 4 B)");
  if (keys.seg_stride < T && segs > 1) return fail(TQ_ERR_INVALID_ARG, "keys.seg_stride must be >= T");
  const int64_t stride = segs == 1 && keys.seg_stride < T ? T : keys.seg_stride;
  if ((int64_t)(segs - 1) * stride + T > keys.records)
    return fail(TQ_ERR_INVALID_ARG, "the keys read (%lld records) exceed keys.records (%lld)",
                (long long)((int64_t)(segs - 1) * stride + T), (long long)keys.records);
  if (T >= (1ll << 31) || (int64_t)segs * group * T >= (1ll << 40))
    return fail(TQ_ERR_UNSUPPORTED, "T or the score array is too large");
  a.q = q;
  a.segs = segs;
  a.group = group;
  a.planes = (uint32_t*)keys.planes;
  a.scalars = (uint16_t*)keys.scalars;
  a.records = keys.records;
  a.seg_stride = stride;
  a.len = len;
  a.T = T;
  a.scores = scores;
  return hip_status(tq::launch_polar_scores128(a, (hipStream_t)stream), "polar scores launch");
}

}  // extern "C"
