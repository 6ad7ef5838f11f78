// Decode-side kernels, gfx950, d_rot = 128: asymmetric scores of queries
// against packed TurboQuant-prod keys, and softmax attention over a packed
// key / value cache.
//
// Estimator (explainer page, section 8; blog notes, the prod estimator read
// with the stored ||r||_2):
//   s[h][t] = n_t ( <Pi q_h, c[idx_t]> + gamma_t sqrt(pi/2)/m <S Pi q_h, 2 z_t - 1> ).
//
// Bit-plane form.  The Lloyd-Max codebook of an even density is odd-symmetric,
// so in the +-1 variables s_p = 2 bit_p - 1 of the index bits its Walsh
// expansion has odd subsets only:
//   c[idx] = sum_{S odd} u_S prod_{p in S} s_p = sum_S u_S (2 x_S - 1),
// with x_S the parity (xor) of the bits in S: one plane for 1 index bit,
// {b0, b1} for 2, {b0, b1, b2, b0^b1^b2} for 3.  Then
//   <q~, c[idx_t]> = sum_S sum_j (2 u_S q~_j) x_S,tj  -  (sum_S u_S) sum_j q~_j
//   <p~, 2 z_t - 1> = sum_i (2 p~_i) z_ti - sum_i p~_i
// are sums of query weights selected by key bits: an integer contraction.
//
// Matrix-core form.  Each weight vector is quantised per head to an integer
// of 21 bits, q = 2^14 hi + 2^7 mid + lo (hi in [-127, 127], mid and lo in
// [-64, 63]), and the three int8 slices become rows 4 h' + {0, 1, 2} of the A
// operand of v_mfma_i32_16x16x64_i8 (4 heads per 16-row tile; row 4 h' + 3 is
// zero).  Key bits become the B operand: bytes in {0, 1}, tokens on the N
// axis.  The int32 accumulators are exact, and so is 2^14 hi + 2^7 mid + lo in
// int32; the epilogue rescales, adds the constants and applies n_t and
// gamma_t.  Lane group kg of the 16x16 accumulator holds rows 4 kg .. 4 kg + 3,
// i.e. the three slices of head kg of the tile, for token lane % 16: the
// epilogue needs no cross-lane work.  (21 bits keep the scores within ~1e-6
// of float arithmetic, which the softmax of the attention kernel needs: an
// error in a score becomes an error in an exponent.)
//
// K-slot map (any permutation is valid as long as A and B share it): lane
// group kg (= lane / 16) of every MFMA reads plane word kg (coordinates
// 32 kg .. 32 kg + 31); MFMA m in {0, 1} of a plane takes expansion dwords
// k = 4m .. 4m+3, dword k byte i being bit 8 i + k of the word.
#include <cmath>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int D = 128;
constexpr float QMAX = 16256.f;     // 127 * 2^7: two int8 slices (value side of attend)
constexpr float QMAX3 = 2080768.f;  // 127 * 2^14: three int8 slices (query weights)

__host__ __device__ constexpr int mse_planes(int bq) { return bq == 3 ? 4 : bq; }

// Bytes of one segment's query pack: fragments then per-head constants.
__host__ __device__ constexpr size_t pack_frag_bytes(int mt, int f) { return (size_t)mt * f * 64 * 16; }
__host__ __device__ constexpr size_t pack_bytes(int mt, int f) {
  return (pack_frag_bytes(mt, f) + (size_t)mt * 4 * 4 * sizeof(float) + 255) / 256 * 256;
}

struct PrepArgs {
  const float* q;
  int segs, group, d, d_rot;
  int rot;
  const float* pi;
  const float* eps;
  const float* s;
  float u[4];      // Walsh coefficients of the odd-subset planes
  float usum;
  int bq;
  int mt;          // 16-row tiles per segment (4 heads each)
  uint8_t* ws;
};

// One workgroup (4 waves) per segment.  Both 128x128 products run on the
// matrix cores (v_mfma_f32_16x16x32_bf16) with bf16 hi/lo splits of both
// operands (three products, ~2^-16 relative, far below the 2^-14 integer
// quantisation that follows; bf16 keeps fp32's range, so no rescaling):
//   q_rot^T = Pi . Q^T         (dense; the Hadamard form uses +-eps entries)
//   q_proj^T = S . q_rot^T
// wave w owns output rows 32 w .. 32 w + 31, heads on the N axis.  Every
// global operand is loaded up front (one memory round trip); the per-head
// statistics reduce in registers, then the int8 A-operand fragments are
// assembled in LDS and copied out with 16-byte stores.
constexpr int MAXG = 16;
constexpr int QLD = MAXG + 1;
constexpr int MAXFRAG = 4 * 10 * 1024;   // MT <= 4, F <= 10

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void split8_bf16(const float* v, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 h = (__bf16)v[e];
    hi[e] = h;
    lo[e] = (__bf16)(v[e] - (float)h);
  }
}

__device__ __forceinline__ f32x4 mfma3_bf16(const float* av, const float* bv, f32x4 acc) {
  bf16x8 ah, al, bh, bl;
  split8_bf16(av, ah, al);
  split8_bf16(bv, bh, bl);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ void unpack8(float4 a, float4 b, float* v) {
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <bool HAD>
__global__ __launch_bounds__(256) void prep_queries128(PrepArgs a) {
  __shared__ float qr[D * QLD], qp[D * QLD];
  __shared__ __align__(16) uint8_t frag[MAXFRAG];
  __shared__ float part[4][MAXG][4];
  __shared__ float stat[MAXG][4];
  const int seg = blockIdx.x;
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int G = a.group;
  const int np = mse_planes(a.bq);
  const int F = 2 * (np + 1);
  const int fbytes = (int)pack_frag_bytes(a.mt, F);
  const bool live = col < G;

  // ---- every global operand of this lane, in flight together ----
  float4 qv[8], mv[16], sv[16];
  const float4* qh = reinterpret_cast<const float4*>(a.q + ((size_t)seg * G + (live ? col : 0)) * D);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    qv[2 * ks] = qh[(32 * ks + 8 * kq) / 4];
    qv[2 * ks + 1] = qh[(32 * ks + 8 * kq) / 4 + 1];
  }
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    const int row = 16 * (2 * wave + mi) + col;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int k0 = 32 * ks + 8 * kq;
      if (HAD) {
        mv[(mi * 4 + ks) * 2] = reinterpret_cast<const float4*>(a.eps)[k0 / 4];
        mv[(mi * 4 + ks) * 2 + 1] = reinterpret_cast<const float4*>(a.eps)[k0 / 4 + 1];
      } else {
        const float4* prow = reinterpret_cast<const float4*>(a.pi + (size_t)row * D + k0);
        mv[(mi * 4 + ks) * 2] = prow[0];
        mv[(mi * 4 + ks) * 2 + 1] = prow[1];
      }
      const float4* srow = reinterpret_cast<const float4*>(a.s + (size_t)row * D + k0);
      sv[(mi * 4 + ks) * 2] = srow[0];
      sv[(mi * 4 + ks) * 2 + 1] = srow[1];
    }
  }
  for (int i = t; i < fbytes / 16; i += blockDim.x) reinterpret_cast<uint4*>(frag)[i] = make_uint4(0, 0, 0, 0);

  // ---- q_rot^T = Pi . Q^T ----
  float rmax = 0.f, rsum = 0.f;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    const int mt = 2 * wave + mi;
    const int j = 16 * mt + col;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int k0 = 32 * ks + 8 * kq;
      float av[8], bv[8];
      unpack8(mv[(mi * 4 + ks) * 2], mv[(mi * 4 + ks) * 2 + 1], av);
      if (HAD) {
#pragma unroll
        for (int e = 0; e < 8; ++e) av[e] = (__popc(j & (k0 + e)) & 1) ? -av[e] : av[e];
      }
      unpack8(qv[2 * ks], qv[2 * ks + 1], bv);
#pragma unroll
      for (int e = 0; e < 8; ++e) bv[e] = live ? bv[e] : 0.f;
      acc = mfma3_bf16(av, bv, acc);
    }
    const float sc = HAD ? rsqrtf((float)D) : 1.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = acc[r] * sc;
      qr[(16 * mt + 4 * kq + r) * QLD + col] = v;
      rmax = fmaxf(rmax, fabsf(v));
      rsum += v;
    }
  }
  __syncthreads();
  // ---- q_proj^T = S . q_rot^T ----
  float pmax = 0.f, psum = 0.f;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    const int mt = 2 * wave + mi;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int k0 = 32 * ks + 8 * kq;
      float av[8], bv[8];
      unpack8(sv[(mi * 4 + ks) * 2], sv[(mi * 4 + ks) * 2 + 1], av);
#pragma unroll
      for (int e = 0; e < 8; ++e) bv[e] = qr[(k0 + e) * QLD + col];
      acc = mfma3_bf16(av, bv, acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      qp[(16 * mt + 4 * kq + r) * QLD + col] = acc[r];
      pmax = fmaxf(pmax, fabsf(acc[r]));
      psum += acc[r];
    }
  }
  // ---- per-head statistics: lanes col, col+16, col+32, col+48 of every wave ----
#pragma unroll
  for (int o = 16; o < 64; o <<= 1) {
    rmax = fmaxf(rmax, __shfl_xor(rmax, o, 64));
    pmax = fmaxf(pmax, __shfl_xor(pmax, o, 64));
    rsum += __shfl_xor(rsum, o, 64);
    psum += __shfl_xor(psum, o, 64);
  }
  if (kq == 0) {
    part[wave][col][0] = rmax;
    part[wave][col][1] = rsum;
    part[wave][col][2] = pmax;
    part[wave][col][3] = psum;
  }
  __syncthreads();
  if (t < MAXG) {
    float mx = 0.f, sr = 0.f, px = 0.f, sp = 0.f;
    for (int w = 0; w < 4; ++w) {
      mx = fmaxf(mx, part[w][t][0]);
      sr += part[w][t][1];
      px = fmaxf(px, part[w][t][2]);
      sp += part[w][t][3];
    }
    float umax = 0.f;
    for (int p = 0; p < np; ++p) umax = fmaxf(umax, fabsf(2.f * a.u[p]));
    const float mm = mx * umax, pm = 2.f * px;
    stat[t][0] = mm > 0.f ? mm / QMAX3 : 1.f;
    stat[t][1] = -a.usum * sr;
    stat[t][2] = pm > 0.f ? pm / QMAX3 : 1.f;
    stat[t][3] = -sp;
  }
  __syncthreads();
  // ---- quantise and scatter into the LDS fragments ----
  {
    const int j = t & (D - 1);
    const int hs = t >> 7;
    const int kg = j >> 5, b = j & 31;
    const int bi = b >> 3, m = (b & 7) >> 2, k = b & 3;
    for (int h = hs; h < G; h += 2) {
      const int mt = h >> 2, hl = h & 3;
      const float inv_m = 1.f / stat[h][0], inv_q = 1.f / stat[h][2];
      for (int p = 0; p <= np; ++p) {
        const float w = p < np ? 2.f * a.u[p] * qr[j * QLD + h] * inv_m : 2.f * qp[j * QLD + h] * inv_q;
        const int qi = (int)rintf(fminf(fmaxf(w, -QMAX3), QMAX3));
        const int hi = (qi + 8192) >> 14;
        const int rem = qi - 16384 * hi;
        const int mid = (rem + 64) >> 7;
        const int lo = rem - 128 * mid;
        const int off = ((mt * F + 2 * p + m) * 64 + 4 * hl + 16 * kg) * 16 + 4 * k + bi;
        frag[off] = (uint8_t)(int8_t)hi;        // rows 4 hl, 4 hl + 1, 4 hl + 2 are
        frag[off + 16] = (uint8_t)(int8_t)mid;  // consecutive lanes
        frag[off + 32] = (uint8_t)(int8_t)lo;
      }
    }
  }
  __syncthreads();
  uint8_t* base = a.ws + (size_t)seg * pack_bytes(a.mt, F);
  for (int i = t; i < fbytes / 16; i += blockDim.x)
    reinterpret_cast<uint4*>(base)[i] = reinterpret_cast<const uint4*>(frag)[i];
  float* consts = reinterpret_cast<float*>(base + fbytes);
  if (t < a.mt * 4 * 4) consts[t] = t < G * 4 ? stat[t >> 2][t & 3] : 0.f;
}

struct Score128Args {
  const uint8_t* ws;
  const uint32_t* planes;
  const uint16_t* scalars;
  int64_t seg_stride;
  const int32_t* len;
  int64_t T;
  int group;
  float kappa;
  float* scores;
  int chunk_tiles;   // 16-token tiles per workgroup
};

__device__ __forceinline__ void expand8(uint32_t w, uint32_t e[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) e[k] = (w >> k) & 0x01010101u;
}

template <int P>
struct Words;
template <>
struct Words<1> {
  typedef uint32_t v __attribute__((ext_vector_type(1), aligned(4)));
};
template <>
struct Words<2> {
  typedef uint32_t v __attribute__((ext_vector_type(2), aligned(4)));
};
template <>
struct Words<3> {
  typedef uint32_t v __attribute__((ext_vector_type(3), aligned(4)));
};
template <>
struct Words<4> {
  typedef uint32_t v __attribute__((ext_vector_type(4), aligned(4)));
};

constexpr int SROW = 40;   // LDS row stride (floats) of the output transpose tile

// One workgroup = 4 waves = chunk_tiles 16-token tiles of one segment.  A wave
// takes pairs of adjacent tiles (32 tokens); the 32 x 8 outputs of a 16-row
// tile pass through a per-wave LDS tile so that each lane stores 4 consecutive
// tokens of one head (16 bytes) and a store covers whole 128-byte lines.
template <int BQ, int MT>
__global__ __launch_bounds__(256) void scores128(Score128Args a) {
  constexpr int NP = mse_planes(BQ);      // MSE planes after the parity plane
  constexpr int F = 2 * (NP + 1);         // MFMAs per tile per 16-row tile
  constexpr int P = BQ + 1;               // stored planes per key record
  typedef typename Words<P>::v wvec;
  __shared__ __align__(16) float sbuf[4][MT * 4 * SROW];
  const int seg = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t16 = lane & 15;
  const int kg = lane >> 4;
  const int64_t len = a.len ? (int64_t)a.len[seg] : a.T;
  const int64_t tok0 = (int64_t)blockIdx.x * a.chunk_tiles * 16;
  if (tok0 >= len) return;

  // query fragments and per-head constants for this segment
  const uint8_t* pack = a.ws + (size_t)seg * pack_bytes(MT, F);
  i32x4 afr[MT][F];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int f = 0; f < F; ++f)
      afr[mt][f] = reinterpret_cast<const i32x4*>(pack)[(mt * F + f) * 64 + lane];
  const float* consts = reinterpret_cast<const float*>(pack + pack_frag_bytes(MT, F));
  float cst[MT][4];     // head 4 mt + kg: sigma_mse, const_mse, sigma_qjl, const_qjl
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int c = 0; c < 4; ++c) cst[mt][c] = consts[(mt * 4 + kg) * 4 + c];

  // segment bases (uniform) and 32-bit per-lane offsets
  const uint32_t* seg_planes = a.planes + (seg * a.seg_stride + tok0) * (P * 4) + kg * P;
  const uint32_t* seg_scal = reinterpret_cast<const uint32_t*>(a.scalars) + seg * a.seg_stride + tok0;
  float* out = a.scores + (size_t)seg * a.group * a.T + tok0;

  int ntok = (int)(len - tok0 < (int64_t)a.chunk_tiles * 16 ? len - tok0 : (int64_t)a.chunk_tiles * 16);
  const int npairs = (ntok + 31) / 32;
  const int lastt = ntok - 1;
  // loads are unconditional, clamped to the last valid token, so no
  // exec-masked branches surround them
  auto load = [&](int tt, wvec& w, uint32_t& sc) {
    const int t = tt < lastt ? tt : lastt;
    w = *reinterpret_cast<const wvec*>(seg_planes + t * (P * 4));
    sc = seg_scal[t];
  };
  // one 16-token tile -> LDS rows (heads 2 kg, 2 kg + 1), columns col0 + t16
  auto compute = [&](int tt, wvec wl, uint32_t scl, int col0) {
    const bool valid = tt < ntok;
    uint32_t w[P];
#pragma unroll
    for (int p = 0; p < P; ++p) w[p] = valid ? wl[p] : 0u;
    i32x4 am[MT], aq[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) am[mt] = aq[mt] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p <= NP; ++p) {
      uint32_t word;
      if (p == NP) {
        word = w[BQ];                                  // QJL signs
      } else if (p < BQ) {
        word = w[p];                                   // single index bits
      } else {
        if constexpr (BQ == 3) word = w[0] ^ w[1] ^ w[2];   // parity of 3 bits
      }
      uint32_t e[8];
      expand8(word, e);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const i32x4 bv = {(int)e[4 * m], (int)e[4 * m + 1], (int)e[4 * m + 2], (int)e[4 * m + 3]};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if (p == NP) aq[mt] = mfma16x16x64i8(afr[mt][2 * p + m], bv, aq[mt]);
          else am[mt] = mfma16x16x64i8(afr[mt][2 * p + m], bv, am[mt]);
        }
      }
    }
    const float n = (float)__builtin_bit_cast(_Float16, (uint16_t)(scl & 0xffff));
    const float gk = (float)__builtin_bit_cast(_Float16, (uint16_t)(scl >> 16)) * a.kappa;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int im = am[mt][0] * 16384 + am[mt][1] * 128 + am[mt][2];
      const int iq = aq[mt][0] * 16384 + aq[mt][1] * 128 + aq[mt][2];
      const float mse = (float)im * cst[mt][0] + cst[mt][1];
      const float qjl = (float)iq * cst[mt][2] + cst[mt][3];
      sbuf[wave][(4 * mt + kg) * SROW + col0 + t16] = n * fmaf(gk, qjl, mse);
    }
  };
  // lanes 8 h' + c store tokens 4c .. 4c+3 of head 8 r + h' of the pair
  auto flush = [&](int pbase) {
    const int hr = lane >> 3, c4 = 4 * (lane & 7);
#pragma unroll
    for (int rr = 0; rr < (MT + 1) / 2; ++rr) {
      const int head = rr * 8 + hr;
      if (head >= a.group) continue;
      const float4 v = *reinterpret_cast<const float4*>(&sbuf[wave][head * SROW + c4]);
      float* dst = out + (size_t)head * a.T + pbase + c4;
      if (pbase + c4 + 3 < ntok) {
        *reinterpret_cast<float4*>(dst) = v;
      } else {
        if (pbase + c4 < ntok) dst[0] = v.x;
        if (pbase + c4 + 1 < ntok) dst[1] = v.y;
        if (pbase + c4 + 2 < ntok) dst[2] = v.z;
      }
    }
  };

  wvec w0, w1, w2, w3;
  uint32_t s0, s1, s2, s3;
  int pr = wave;
  load(32 * pr + t16, w0, s0);
  load(32 * pr + 16 + t16, w1, s1);
  load(32 * (pr + 4) + t16, w2, s2);
  load(32 * (pr + 4) + 16 + t16, w3, s3);
  for (; pr < npairs; pr += 8) {
    compute(32 * pr + t16, w0, s0, 0);
    compute(32 * pr + 16 + t16, w1, s1, 16);
    load(32 * (pr + 8) + t16, w0, s0);
    load(32 * (pr + 8) + 16 + t16, w1, s1);
    flush(32 * pr);
    if (pr + 4 < npairs) {
      compute(32 * (pr + 4) + t16, w2, s2, 0);
      compute(32 * (pr + 4) + 16 + t16, w3, s3, 16);
      flush(32 * (pr + 4));
    }
    load(32 * (pr + 12) + t16, w2, s2);
    load(32 * (pr + 12) + 16 + t16, w3, s3);
  }
}

template <int BQ, int MT>
hipError_t launch_scores(const Score128Args& s, int segs, hipStream_t stream) {
  const int64_t tiles = (s.T + 15) / 16;
  const int64_t chunks = (tiles + s.chunk_tiles - 1) / s.chunk_tiles;
  hipLaunchKernelGGL((scores128<BQ, MT>), dim3((unsigned)chunks, (unsigned)segs), dim3(256), 0, stream, s);
  return hipGetLastError();
}

void walsh_coefficients(const Codebook& cb, int bq, float u[4], float* usum) {
  // u_S = 2^-bq sum_idx c[idx] prod_{p in S} (2 bit_p(idx) - 1), odd S in the plane order
  const int K = 1 << bq;
  int subsets[4];
  int ns = 0;
  for (int p = 0; p < bq; ++p) subsets[ns++] = 1 << p;
  if (bq == 3) subsets[ns++] = 7;
  double tot = 0;
  for (int s = 0; s < 4; ++s) u[s] = 0.f;
  for (int s = 0; s < ns; ++s) {
    double acc = 0;
    for (int idx = 0; idx < K; ++idx) {
      double chi = 1;
      for (int p = 0; p < bq; ++p)
        if (subsets[s] >> p & 1) chi *= ((idx >> p) & 1) ? 1.0 : -1.0;
      acc += cb.c[idx] * chi;
    }
    u[s] = (float)(acc / K);
    tot += acc / K;
  }
  *usum = (float)tot;
}

}  // namespace

size_t scores128_workspace(int segs, int group) {
  const int mt = (group + 3) / 4;
  return (size_t)segs * pack_bytes(mt, 2 * (mse_planes(3) + 1));   // sized for the widest key
}

hipError_t launch_scores128_prep(const ScoreArgs& a, hipStream_t stream) {
  PrepArgs p;
  p.q = a.q;
  p.segs = a.segs;
  p.group = a.group;
  p.d = a.d;
  p.d_rot = D;
  p.rot = a.rot;
  p.pi = a.pi;
  p.eps = a.eps;
  p.s = a.s;
  walsh_coefficients(a.cb, a.bq, p.u, &p.usum);
  p.bq = a.bq;
  p.mt = (a.group + 3) / 4;
  p.ws = static_cast<uint8_t*>(a.ws);
  if (a.rot == TQ_ROT_HADAMARD)
    hipLaunchKernelGGL(prep_queries128<true>, dim3(a.segs), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(prep_queries128<false>, dim3(a.segs), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_scores128(const ScoreArgs& a, hipStream_t stream) {
  hipError_t e = launch_scores128_prep(a, stream);
  if (e != hipSuccess) return e;
  const int mt = (a.group + 3) / 4;
  Score128Args s;
  s.ws = static_cast<const uint8_t*>(a.ws);
  s.planes = a.planes;
  s.scalars = a.scalars;
  s.seg_stride = a.seg_stride;
  s.len = a.len;
  s.T = a.T;
  s.group = a.group;
  s.kappa = (float)(std::sqrt(M_PI / 2.0) / D);
  s.scores = a.scores;
  s.chunk_tiles = 32;
  switch (a.bq * 10 + mt) {
    case 11: return launch_scores<1, 1>(s, a.segs, stream);
    case 12: return launch_scores<1, 2>(s, a.segs, stream);
    case 13: return launch_scores<1, 3>(s, a.segs, stream);
    case 14: return launch_scores<1, 4>(s, a.segs, stream);
    case 21: return launch_scores<2, 1>(s, a.segs, stream);
    case 22: return launch_scores<2, 2>(s, a.segs, stream);
    case 23: return launch_scores<2, 3>(s, a.segs, stream);
    case 24: return launch_scores<2, 4>(s, a.segs, stream);
    case 31: return launch_scores<3, 1>(s, a.segs, stream);
    case 32: return launch_scores<3, 2>(s, a.segs, stream);
    case 33: return launch_scores<3, 3>(s, a.segs, stream);
    case 34: return launch_scores<3, 4>(s, a.segs, stream);
  }
  return hipErrorInvalidValue;
}

namespace {

// ---------------------------------------------------------------------------
// Attention over a compressed cache (first page, usage pattern 1: scores from
// the compressed keys, softmax, weighted sum of the MSE-dequantised values).
//
//   p_t = exp(scale s_t - m),  o = sum_t p_t n_v,t Pi_v^T c_v[idx_t] / sum_t p_t
//
// The value sum stays in the rotated domain (Pi_v^T is linear and is applied
// once per head at the end) and uses the same Walsh form as the keys:
//   sum_t P'_t c_v[idx_t,j] = sum_S u_S (2 sum_t P'_t x_S,tj - sum_t P'_t),
// P'_t = p_t n_v,t, a contraction over tokens: A = P' (three int8 slices per
// head, 21 bits relative to the group maximum, rows 4 h' + slice as for the
// keys), B = value bits, whose block layout gives each lane one coordinate
// across 32 tokens in one word.  The constant term uses the same quantised
// P' as the bit sums, so quantisation errors enter only through the
// zero-mean centroids.
//
// Work split: a workgroup (4 waves) covers 512 tokens of one segment; a wave
// owns one group of 128 tokens (8 key tiles; 4 value blocks).  The waves'
// partials (m, l, o~) merge in LDS, one partial per (segment, chunk, head)
// goes to the workspace, and attend_combine128 merges the chunks (log-sum-exp)
// and applies Pi_v^T.
// ---------------------------------------------------------------------------
constexpr int PST = 132;        // partial: m, l, 2 pad, o~[128]
constexpr int ACHUNK = 512;     // tokens per attend workgroup

struct Attend128Args {
  const uint8_t* pack;          // key-side query fragments (prep_queries128)
  const uint32_t* kplanes;
  const uint16_t* kscal;
  int64_t kstride;
  const uint32_t* vplanes;      // value blocks
  const uint16_t* vscal;
  int64_t vstride;              // multiple of 32
  const int32_t* len;
  int64_t T;
  int group;
  float kappa;
  float scale2;                 // softmax scale * log2(e)
  float vu[4];                  // value Walsh coefficients, odd subsets
  float vusum;
  float* part;                  // [segs][nchunks][group][PST]
  int nchunks;
};

// position of group token tt in the A-operand byte rows (matches the value
// expansion: block tt / 32, bit b -> MFMA (b % 8) / 4, dword b % 4, byte b / 8)
__device__ __forceinline__ int vperm(int tt) {
  const int b = tt & 31;
  return (tt & ~31) + 16 * ((b & 7) >> 2) + 4 * (b & 3) + (b >> 3);
}

template <int BQK, int BQV, int KMT>
__global__ __launch_bounds__(256) void attend128(Attend128Args a) {
  constexpr int NPK = mse_planes(BQK);
  constexpr int FK = 2 * (NPK + 1);
  constexpr int PK = BQK + 1;
  constexpr int NPV = mse_planes(BQV);
  constexpr int PV = BQV;
  constexpr int NH = KMT * 4;               // heads of the 16-row tiles (4 each)
  typedef typename Words<PK>::v kvec;
  typedef typename Words<PV>::v vvec;
  __shared__ float sred[4][NH][PST];
  __shared__ __align__(16) uint8_t pq[4][KMT][16][128];
  __shared__ float vnorm[4][128];
  const int seg = blockIdx.y;
  const int chunk = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t16 = lane & 15;
  const int kg = lane >> 4;
  const int64_t len = a.len ? (int64_t)a.len[seg] : a.T;
  const int64_t g0 = (int64_t)chunk * ACHUNK + 128 * wave;
  const int ntok = (int)(len - g0 <= 0 ? 0 : (len - g0 < 128 ? len - g0 : 128));

  // lane group kg holds head 4 mt + kg on both sides
  float o_st[KMT][8], m_st[KMT], l_st[KMT];
#pragma unroll
  for (int mt = 0; mt < KMT; ++mt) {
    m_st[mt] = -INFINITY;
    l_st[mt] = 0.f;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) o_st[mt][nt] = 0.f;
  }

  if (ntok > 0) {
    // ---- every global load of the group, in flight together ----
    const int last = ntok - 1;
    const uint32_t* kbase = a.kplanes + (seg * a.kstride + g0) * (PK * 4) + kg * PK;
    const uint32_t* ksbase = reinterpret_cast<const uint32_t*>(a.kscal) + seg * a.kstride + g0;
    kvec kw[8];
    uint32_t ks[8];
#pragma unroll
    for (int tile = 0; tile < 8; ++tile) {
      int tt = tile * 16 + t16;
      tt = tt < last ? tt : last;
      kw[tile] = *reinterpret_cast<const kvec*>(kbase + tt * (PK * 4));
      ks[tile] = ksbase[tt];
    }
    // value block kg of the group (clamped to the last block holding tokens)
    const int vb = kg < (last >> 5) ? kg : (last >> 5);
    const uint32_t* vbase = a.vplanes + ((seg * a.vstride + g0) / 32 + vb) * (D * PV) + t16 * PV;
    vvec vw[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) vw[nt] = *reinterpret_cast<const vvec*>(vbase + 16 * nt * PV);
    {
      int tt = 2 * lane;
      tt = tt < last ? tt : (last & ~1);
      const uint32_t nn = *reinterpret_cast<const uint32_t*>(a.vscal + seg * a.vstride + g0 + tt);
      vnorm[wave][2 * lane] = 2 * lane < ntok ? (float)__builtin_bit_cast(_Float16, (uint16_t)(nn & 0xffff)) : 0.f;
      vnorm[wave][2 * lane + 1] =
          2 * lane + 1 < ntok ? (float)__builtin_bit_cast(_Float16, (uint16_t)(nn >> 16)) : 0.f;
    }
    // key-side fragments and constants (head 4 mt + kg)
    const uint8_t* pack = a.pack + (size_t)seg * pack_bytes(KMT, FK);
    i32x4 afr[KMT][FK];
#pragma unroll
    for (int mt = 0; mt < KMT; ++mt)
#pragma unroll
      for (int f = 0; f < FK; ++f)
        afr[mt][f] = reinterpret_cast<const i32x4*>(pack)[(mt * FK + f) * 64 + lane];
    const float* consts = reinterpret_cast<const float*>(pack + pack_frag_bytes(KMT, FK));
    float cst[KMT][4];
#pragma unroll
    for (int mt = 0; mt < KMT; ++mt)
#pragma unroll
      for (int c = 0; c < 4; ++c) cst[mt][c] = consts[(mt * 4 + kg) * 4 + c];

    // ---- phase 1: scores of the 8 key tiles (token t16 + 16 tile, head 4 mt + kg) ----
    float sc[8][KMT];
#pragma unroll
    for (int tile = 0; tile < 8; ++tile) {
      const bool valid = tile * 16 + t16 < ntok;
      uint32_t w[PK];
#pragma unroll
      for (int p = 0; p < PK; ++p) w[p] = valid ? kw[tile][p] : 0u;
      i32x4 am[KMT], aq[KMT];
#pragma unroll
      for (int mt = 0; mt < KMT; ++mt) am[mt] = aq[mt] = i32x4{0, 0, 0, 0};
#pragma unroll
      for (int p = 0; p <= NPK; ++p) {
        uint32_t word;
        if (p == NPK) {
          word = w[BQK];
        } else if (p < BQK) {
          word = w[p];
        } else {
          if constexpr (BQK == 3) word = w[0] ^ w[1] ^ w[2];
        }
        uint32_t e8[8];
        expand8(word, e8);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const i32x4 bv = {(int)e8[4 * m], (int)e8[4 * m + 1], (int)e8[4 * m + 2], (int)e8[4 * m + 3]};
#pragma unroll
          for (int mt = 0; mt < KMT; ++mt) {
            if (p == NPK) aq[mt] = mfma16x16x64i8(afr[mt][2 * p + m], bv, aq[mt]);
            else am[mt] = mfma16x16x64i8(afr[mt][2 * p + m], bv, am[mt]);
          }
        }
      }
      const float n = (float)__builtin_bit_cast(_Float16, (uint16_t)(ks[tile] & 0xffff));
      const float gk = (float)__builtin_bit_cast(_Float16, (uint16_t)(ks[tile] >> 16)) * a.kappa;
#pragma unroll
      for (int mt = 0; mt < KMT; ++mt) {
        const int im = am[mt][0] * 16384 + am[mt][1] * 128 + am[mt][2];
        const int iq = aq[mt][0] * 16384 + aq[mt][1] * 128 + aq[mt][2];
        const float mse = (float)im * cst[mt][0] + cst[mt][1];
        const float qjl = (float)iq * cst[mt][2] + cst[mt][3];
        sc[tile][mt] = valid ? n * fmaf(gk, qjl, mse) * a.scale2 : -INFINITY;
      }
    }

    // ---- phase 2: softmax statistics and the int8 P' rows ----
    float vn[8];
#pragma unroll
    for (int tile = 0; tile < 8; ++tile) vn[tile] = vnorm[wave][tile * 16 + t16];
    float fsig[KMT];
#pragma unroll
    for (int mt = 0; mt < KMT; ++mt) {
      float mx = -INFINITY;
#pragma unroll
      for (int tile = 0; tile < 8; ++tile) mx = fmaxf(mx, sc[tile][mt]);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      float pv[8], ls = 0.f, pmax = 0.f;
#pragma unroll
      for (int tile = 0; tile < 8; ++tile) {
        const float pp = exp2f(sc[tile][mt] - mx);
        ls += pp;
        pv[tile] = pp * vn[tile];
        pmax = fmaxf(pmax, pv[tile]);
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        ls += __shfl_xor(ls, o, 64);
        pmax = fmaxf(pmax, __shfl_xor(pmax, o, 64));
      }
      const float sig = pmax > 0.f ? pmax / QMAX3 : 1.f;
      const float inv = 1.f / sig;
      int qsum = 0;
#pragma unroll
      for (int tile = 0; tile < 8; ++tile) {
        const int qi = (int)rintf(fminf(pv[tile] * inv, QMAX3));
        qsum += qi;
        const int hi = (qi + 8192) >> 14;
        const int rem = qi - 16384 * hi;
        const int mid = (rem + 64) >> 7;
        const int lo = rem - 128 * mid;
        const int pos = vperm(tile * 16 + t16);
        pq[wave][mt][4 * kg][pos] = (uint8_t)(int8_t)hi;
        pq[wave][mt][4 * kg + 1][pos] = (uint8_t)(int8_t)mid;
        pq[wave][mt][4 * kg + 2][pos] = (uint8_t)(int8_t)lo;
        pq[wave][mt][4 * kg + 3][pos] = 0;
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) qsum += __shfl_xor(qsum, o, 64);
      m_st[mt] = mx;
      l_st[mt] = ls;
      fsig[mt] = sig;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) o_st[mt][nt] = -a.vusum * sig * (float)qsum;
    }

    // ---- phase 3: A operands (row = lane % 16, token bytes of block kg) ----
    i32x4 pa[KMT][2];
#pragma unroll
    for (int mt = 0; mt < KMT; ++mt)
#pragma unroll
      for (int m = 0; m < 2; ++m) pa[mt][m] = *reinterpret_cast<const i32x4*>(&pq[wave][mt][t16][32 * kg + 16 * m]);

    // ---- phase 4: value planes, each folded with its Walsh weight ----
#pragma unroll
    for (int sp = 0; sp < NPV; ++sp) {
      i32x4 acc[KMT][8];
#pragma unroll
      for (int mt = 0; mt < KMT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = i32x4{0, 0, 0, 0};
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        uint32_t word;
        if (sp < BQV) {
          word = vw[nt][sp];
        } else {
          if constexpr (BQV == 3) word = vw[nt][0] ^ vw[nt][1] ^ vw[nt][2];
        }
        uint32_t e8[8];
        expand8(word, e8);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const i32x4 bv = {(int)e8[4 * m], (int)e8[4 * m + 1], (int)e8[4 * m + 2], (int)e8[4 * m + 3]};
#pragma unroll
          for (int mt = 0; mt < KMT; ++mt) acc[mt][nt] = mfma16x16x64i8(pa[mt][m], bv, acc[mt][nt]);
        }
      }
      const float w2 = 2.f * a.vu[sp];
#pragma unroll
      for (int mt = 0; mt < KMT; ++mt) {
        const float f = w2 * fsig[mt];
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
          o_st[mt][nt] = fmaf((float)(acc[mt][nt][0] * 16384 + acc[mt][nt][1] * 128 + acc[mt][nt][2]), f,
                              o_st[mt][nt]);
      }
    }
  }

  // ---- phase 5: merge the four waves' partials in LDS ----
#pragma unroll
  for (int mt = 0; mt < KMT; ++mt) {
    float* r = sred[wave][4 * mt + kg];
    if (t16 == 0) {
      r[0] = m_st[mt];
      r[1] = l_st[mt];
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) r[4 + 16 * nt + t16] = o_st[mt][nt];
  }
  __syncthreads();
  const int nh = a.group < NH ? a.group : NH;
  float* outp = a.part + ((size_t)seg * a.nchunks + chunk) * a.group * PST;
  for (int i = threadIdx.x; i < nh * 130; i += blockDim.x) {
    const int h = i / 130, c = i % 130;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sred[w][h][0]);
    float v = 0.f;
    if (M != -INFINITY) {
      if (c == 0) {
        v = M;
      } else {
        const int src = c == 1 ? 1 : c + 2;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float wt = exp2f(sred[w][h][0] - M);     // 0 for empty waves
          v += wt * sred[w][h][src];
        }
      }
    } else {
      v = c == 0 ? -INFINITY : 0.f;
    }
    outp[h * PST + (c < 2 ? c : c + 2)] = v;
  }
}

struct Combine128Args {
  const float* part;
  int nchunks, group, d;
  const int32_t* len;
  int64_t T;
  int rot;
  const float* pi_v;
  const float* eps_v;
  float* out;
};

// One workgroup (128 threads) per query head: log-sum-exp merge of the chunk
// partials, normalisation, then the inverse rotation o = Pi_v^T o~.
__global__ __launch_bounds__(128) void attend_combine128(Combine128Args a) {
  __shared__ float ot[D];
  const int hg = blockIdx.x;               // seg * group + head
  const int seg = hg / a.group, h = hg % a.group;
  const int j = threadIdx.x;
  const int64_t len = a.len ? (int64_t)a.len[seg] : a.T;
  const int nch = (int)((len + ACHUNK - 1) / ACHUNK);
  const float* base = a.part + (size_t)seg * a.nchunks * a.group * PST + (size_t)h * PST;
  float M = -INFINITY;
  for (int c = 0; c < nch; ++c) M = fmaxf(M, base[(size_t)c * a.group * PST]);
  float L = 0.f, acc = 0.f;
  if (M != -INFINITY) {
    for (int c = 0; c < nch; ++c) {
      const float* pc = base + (size_t)c * a.group * PST;
      const float wt = exp2f(pc[0] - M);
      L += wt * pc[1];
      acc += wt * pc[4 + j];
    }
  }
  ot[j] = L > 0.f ? acc / L : 0.f;
  __syncthreads();
  if (j >= a.d) return;
  float o = 0.f;
  if (a.rot == TQ_ROT_DENSE) {
    for (int k = 0; k < D; ++k) o = fmaf(a.pi_v[(size_t)k * a.d + j], ot[k], o);
  } else {
    for (int k = 0; k < D; ++k) o += ((__popc(j & k) & 1) ? -ot[k] : ot[k]);
    o *= a.eps_v[j] * rsqrtf((float)D);
  }
  a.out[(size_t)hg * a.d + j] = o;
}

template <int BQK, int BQV, int MT>
hipError_t launch_attend(const Attend128Args& s, int segs, hipStream_t stream) {
  hipLaunchKernelGGL((attend128<BQK, BQV, MT>), dim3((unsigned)s.nchunks, (unsigned)segs), dim3(256), 0,
                     stream, s);
  return hipGetLastError();
}

size_t attend_pack_bytes(int segs, int group) { return scores128_workspace(segs, group); }

}  // namespace

size_t attend128_workspace(int segs, int group, int64_t T) {
  const int64_t nch = (T + ACHUNK - 1) / ACHUNK;
  return attend_pack_bytes(segs, group) + (size_t)segs * nch * group * PST * sizeof(float);
}

hipError_t launch_attend128(const AttendArgs& a, hipStream_t stream) {
  hipError_t e = launch_scores128_prep(a.k, stream);
  if (e != hipSuccess) return e;
  Attend128Args s;
  s.pack = static_cast<const uint8_t*>(a.ws);
  s.kplanes = a.k.planes;
  s.kscal = a.k.scalars;
  s.kstride = a.k.seg_stride;
  s.vplanes = a.planes_v;
  s.vscal = a.scalars_v;
  s.vstride = a.seg_stride_v;
  s.len = a.k.len;
  s.T = a.k.T;
  s.group = a.k.group;
  s.kappa = (float)(std::sqrt(M_PI / 2.0) / D);
  s.scale2 = a.scale * 1.4426950408889634f;
  walsh_coefficients(a.cb_v, a.bq_v, s.vu, &s.vusum);
  s.nchunks = (int)((a.k.T + ACHUNK - 1) / ACHUNK);
  s.part = reinterpret_cast<float*>(static_cast<uint8_t*>(a.ws) + attend_pack_bytes(a.k.segs, a.k.group));
  const int mt = (a.k.group + 3) / 4;
  switch ((a.k.bq * 10 + a.bq_v) * 10 + mt) {
    case 111: e = launch_attend<1, 1, 1>(s, a.k.segs, stream); break;
    case 112: e = launch_attend<1, 1, 2>(s, a.k.segs, stream); break;
    case 113: e = launch_attend<1, 1, 3>(s, a.k.segs, stream); break;
    case 114: e = launch_attend<1, 1, 4>(s, a.k.segs, stream); break;
    case 121: e = launch_attend<1, 2, 1>(s, a.k.segs, stream); break;
    case 122: e = launch_attend<1, 2, 2>(s, a.k.segs, stream); break;
    case 123: e = launch_attend<1, 2, 3>(s, a.k.segs, stream); break;
    case 124: e = launch_attend<1, 2, 4>(s, a.k.segs, stream); break;
    case 131: e = launch_attend<1, 3, 1>(s, a.k.segs, stream); break;
    case 132: e = launch_attend<1, 3, 2>(s, a.k.segs, stream); break;
    case 133: e = launch_attend<1, 3, 3>(s, a.k.segs, stream); break;
    case 134: e = launch_attend<1, 3, 4>(s, a.k.segs, stream); break;
    case 211: e = launch_attend<2, 1, 1>(s, a.k.segs, stream); break;
    case 212: e = launch_attend<2, 1, 2>(s, a.k.segs, stream); break;
    case 213: e = launch_attend<2, 1, 3>(s, a.k.segs, stream); break;
    case 214: e = launch_attend<2, 1, 4>(s, a.k.segs, stream); break;
    case 221: e = launch_attend<2, 2, 1>(s, a.k.segs, stream); break;
    case 222: e = launch_attend<2, 2, 2>(s, a.k.segs, stream); break;
    case 223: e = launch_attend<2, 2, 3>(s, a.k.segs, stream); break;
    case 224: e = launch_attend<2, 2, 4>(s, a.k.segs, stream); break;
    case 231: e = launch_attend<2, 3, 1>(s, a.k.segs, stream); break;
    case 232: e = launch_attend<2, 3, 2>(s, a.k.segs, stream); break;
    case 233: e = launch_attend<2, 3, 3>(s, a.k.segs, stream); break;
    case 234: e = launch_attend<2, 3, 4>(s, a.k.segs, stream); break;
    case 311: e = launch_attend<3, 1, 1>(s, a.k.segs, stream); break;
    case 312: e = launch_attend<3, 1, 2>(s, a.k.segs, stream); break;
    case 313: e = launch_attend<3, 1, 3>(s, a.k.segs, stream); break;
    case 314: e = launch_attend<3, 1, 4>(s, a.k.segs, stream); break;
    case 321: e = launch_attend<3, 2, 1>(s, a.k.segs, stream); break;
    case 322: e = launch_attend<3, 2, 2>(s, a.k.segs, stream); break;
    case 323: e = launch_attend<3, 2, 3>(s, a.k.segs, stream); break;
    case 324: e = launch_attend<3, 2, 4>(s, a.k.segs, stream); break;
    case 331: e = launch_attend<3, 3, 1>(s, a.k.segs, stream); break;
    case 332: e = launch_attend<3, 3, 2>(s, a.k.segs, stream); break;
    case 333: e = launch_attend<3, 3, 3>(s, a.k.segs, stream); break;
    case 334: e = launch_attend<3, 3, 4>(s, a.k.segs, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  Combine128Args c;
  c.part = s.part;
  c.nchunks = s.nchunks;
  c.group = a.k.group;
  c.d = a.k.d;
  c.len = a.k.len;
  c.T = a.k.T;
  c.rot = a.rot_v;
  c.pi_v = a.pi_v;
  c.eps_v = a.eps_v;
  c.out = a.out;
  hipLaunchKernelGGL(attend_combine128, dim3((unsigned)(a.k.segs * a.k.group)), dim3(128), 0, stream, c);
  return hipGetLastError();
}

}  // namespace tq
