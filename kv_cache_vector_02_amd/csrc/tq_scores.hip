// Asymmetric scores of decode queries against packed TurboQuant-prod keys,
// gfx950, d_rot = 128.
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
// of 15 bits, q = 128 hi + lo, hi in [-127, 127], lo in [-64, 63], and the two
// int8 slices become rows of the A operand of v_mfma_i32_16x16x64_i8
// (row 2 h' + slice, 8 heads per 16-row tile).  Key bits become the B
// operand: bytes in {0, 1}, tokens on the N axis.  The int32 accumulators
// are exact; the epilogue forms 128 hi + lo, rescales, adds the constants and
// applies n_t and gamma_t.  Each lane of the 16x16 accumulator holds one token
// and the two slices of two heads, so the epilogue needs no cross-lane work.
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
constexpr float QMAX = 16256.f;  // 127 * 128

__host__ __device__ constexpr int mse_planes(int bq) { return bq == 3 ? 4 : bq; }

// Bytes of one segment's query pack: fragments then per-head constants.
__host__ __device__ constexpr size_t pack_frag_bytes(int mt, int f) { return (size_t)mt * f * 64 * 16; }
__host__ __device__ constexpr size_t pack_bytes(int mt, int f) {
  return (pack_frag_bytes(mt, f) + (size_t)mt * 8 * 4 * sizeof(float) + 255) / 256 * 256;
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
  int mt;          // 16-row tiles per segment
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
constexpr int MAXFRAG = 2 * 10 * 1024;   // MT <= 2, F <= 10

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
    stat[t][0] = mm > 0.f ? mm / QMAX : 1.f;
    stat[t][1] = -a.usum * sr;
    stat[t][2] = pm > 0.f ? pm / QMAX : 1.f;
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
      const int mt = h >> 3, hl = h & 7;
      const float inv_m = 1.f / stat[h][0], inv_q = 1.f / stat[h][2];
      for (int p = 0; p <= np; ++p) {
        const float w = p < np ? 2.f * a.u[p] * qr[j * QLD + h] * inv_m : 2.f * qp[j * QLD + h] * inv_q;
        const int qi = (int)rintf(fminf(fmaxf(w, -QMAX), QMAX));
        const int hi = (qi + 64) >> 7;
        const int lo = qi - 128 * hi;
        const int off = ((mt * F + 2 * p + m) * 64 + 2 * hl + 16 * kg) * 16 + 4 * k + bi;
        frag[off] = (uint8_t)(int8_t)hi;
        frag[off + 16] = (uint8_t)(int8_t)lo;   // row 2 hl + 1 is the next lane
      }
    }
  }
  __syncthreads();
  uint8_t* base = a.ws + (size_t)seg * pack_bytes(a.mt, F);
  for (int i = t; i < fbytes / 16; i += blockDim.x)
    reinterpret_cast<uint4*>(base)[i] = reinterpret_cast<const uint4*>(frag)[i];
  float* consts = reinterpret_cast<float*>(base + fbytes);
  if (t < G * 4) consts[t] = stat[t >> 2][t & 3];
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
  __shared__ __align__(16) float sbuf[4][MT][8 * SROW];
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
  float cst[MT][2][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int c = 0; c < 4; ++c) cst[mt][e][c] = consts[(mt * 8 + 2 * kg + e) * 4 + c];

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
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float mse = (float)(am[mt][2 * e] * 128 + am[mt][2 * e + 1]) * cst[mt][e][0] + cst[mt][e][1];
        const float qjl = (float)(aq[mt][2 * e] * 128 + aq[mt][2 * e + 1]) * cst[mt][e][2] + cst[mt][e][3];
        sbuf[wave][mt][(2 * kg + e) * SROW + col0 + t16] = n * fmaf(gk, qjl, mse);
      }
    }
  };
  // lanes 8 h' + c store tokens 4c .. 4c+3 of head h' of the pair
  auto flush = [&](int pbase) {
    const int hr = lane >> 3, c4 = 4 * (lane & 7);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int head = mt * 8 + hr;
      if (head >= a.group) continue;
      const float4 v = *reinterpret_cast<const float4*>(&sbuf[wave][mt][hr * SROW + c4]);
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
  const int mt = (group + 7) / 8;
  return (size_t)segs * pack_bytes(mt, 2 * (mse_planes(3) + 1));   // sized for the widest key
}

hipError_t launch_scores128(const ScoreArgs& a, hipStream_t stream) {
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
  p.mt = (a.group + 7) / 8;
  p.ws = static_cast<uint8_t*>(a.ws);
  if (a.rot == TQ_ROT_HADAMARD)
    hipLaunchKernelGGL(prep_queries128<true>, dim3(a.segs), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(prep_queries128<false>, dim3(a.segs), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  Score128Args s;
  s.ws = p.ws;
  s.planes = a.planes;
  s.scalars = a.scalars;
  s.seg_stride = a.seg_stride;
  s.len = a.len;
  s.T = a.T;
  s.group = a.group;
  s.kappa = (float)(std::sqrt(M_PI / 2.0) / D);
  s.scores = a.scores;
  s.chunk_tiles = 32;
  switch (a.bq * 10 + p.mt) {
    case 11: return launch_scores<1, 1>(s, a.segs, stream);
    case 12: return launch_scores<1, 2>(s, a.segs, stream);
    case 21: return launch_scores<2, 1>(s, a.segs, stream);
    case 22: return launch_scores<2, 2>(s, a.segs, stream);
    case 31: return launch_scores<3, 1>(s, a.segs, stream);
    case 32: return launch_scores<3, 2>(s, a.segs, stream);
  }
  return hipErrorInvalidValue;
}

size_t attend128_workspace(int segs, int group, int64_t T) { (void)T; return (size_t)segs * group * 0 + 256; }

}  // namespace tq
