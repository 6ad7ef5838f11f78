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

__device__ float block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = fmaxf(r, red[i]);
  return r;
}

__device__ float block_sum(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) r += red[i];
  return r;
}

// One workgroup (128 threads) per segment: rotate and project each query head,
// quantise the plane weights and scatter them into the A-operand fragments.
__global__ __launch_bounds__(128) void prep_queries128(PrepArgs a) {
  __shared__ float qs[D], qrot[D], qproj[D];
  __shared__ float red[4];
  const int seg = blockIdx.x;
  const int j = threadIdx.x;
  const int np = mse_planes(a.bq);
  const int F = 2 * (np + 1);
  uint8_t* base = a.ws + (size_t)seg * pack_bytes(a.mt, F);
  // zero the fragments (rows of heads beyond the group stay zero)
  {
    uint4* z = reinterpret_cast<uint4*>(base);
    const int n16 = (int)(pack_frag_bytes(a.mt, F) / 16);
    for (int i = j; i < n16; i += blockDim.x) z[i] = make_uint4(0, 0, 0, 0);
  }
  float* consts = reinterpret_cast<float*>(base + pack_frag_bytes(a.mt, F));
  __syncthreads();
  for (int hh = 0; hh < a.group; ++hh) {
    const float* qh = a.q + ((size_t)seg * a.group + hh) * a.d;
    qs[j] = j < a.d ? qh[j] : 0.f;
    __syncthreads();
    float acc = 0.f;
    if (a.rot == TQ_ROT_DENSE) {
      const float* row = a.pi + (size_t)j * a.d;
      for (int k = 0; k < a.d; ++k) acc += row[k] * qs[k];
    } else {
      for (int k = 0; k < a.d; ++k) acc += ((__popc(j & k) & 1) ? -1.f : 1.f) * a.eps[k] * qs[k];
      acc *= rsqrtf((float)a.d_rot);
    }
    qrot[j] = acc;
    __syncthreads();
    float pacc = 0.f;
    {
      const float* row = a.s + (size_t)j * D;
      for (int k = 0; k < D; ++k) pacc += row[k] * qrot[k];
    }
    qproj[j] = pacc;
    float umax = 0.f;
    for (int p = 0; p < np; ++p) umax = fmaxf(umax, fabsf(2.f * a.u[p]));
    const float mmax = block_max(fabsf(qrot[j]) * umax, red);
    const float pmax = block_max(fabsf(2.f * pacc), red);
    const float qsum = block_sum(qrot[j], red);
    const float psum = block_sum(pacc, red);
    const float sig_m = mmax > 0.f ? mmax / QMAX : 1.f;
    const float sig_q = pmax > 0.f ? pmax / QMAX : 1.f;
    const int mt = hh >> 3;
    const int hl = hh & 7;
    if (j == 0) {
      float* c = consts + (size_t)hh * 4;
      c[0] = sig_m;
      c[1] = -a.usum * qsum;
      c[2] = sig_q;
      c[3] = -psum;
    }
    // coordinate j -> (kg, word bit) -> (m, k, i)
    const int kg = j >> 5, b = j & 31;
    const int i = b >> 3, m = (b & 7) >> 2, k = b & 3;
    for (int p = 0; p <= np; ++p) {
      const float w = p < np ? 2.f * a.u[p] * qrot[j] : 2.f * pacc;
      const float sig = p < np ? sig_m : sig_q;
      const int qi = (int)rintf(w / sig);
      const int hi = (qi + 64) >> 7;
      const int lo = qi - 128 * hi;
      for (int sl = 0; sl < 2; ++sl) {
        const int rho = 2 * hl + sl;
        const size_t off = (((size_t)mt * F + 2 * p + m) * 64 + rho + 16 * kg) * 16 + 4 * k + i;
        base[off] = (uint8_t)(int8_t)(sl == 0 ? hi : lo);
      }
    }
    __syncthreads();
  }
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

template <int BQ, int MT>
__global__ __launch_bounds__(256) void scores128(Score128Args a) {
  constexpr int NP = mse_planes(BQ);      // MSE planes after the parity plane
  constexpr int F = 2 * (NP + 1);         // MFMAs per tile per 16-row tile
  constexpr int P = BQ + 1;               // stored planes per key record
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

  const uint32_t* seg_planes = a.planes + seg * a.seg_stride * (P * 4);
  const uint32_t* seg_scal = reinterpret_cast<const uint32_t*>(a.scalars) + seg * a.seg_stride;
  float* out = a.scores + (size_t)seg * a.group * a.T;

  for (int tile = wave; tile < a.chunk_tiles; tile += 4) {
    const int64_t t = tok0 + (int64_t)tile * 16 + t16;
    if (tok0 + (int64_t)tile * 16 >= len) break;
    const bool valid = t < len;
    uint32_t w[P];
#pragma unroll
    for (int p = 0; p < P; ++p) w[p] = valid ? seg_planes[t * (P * 4) + p * 4 + kg] : 0u;
    const uint32_t sc = valid ? seg_scal[t] : 0u;

    i32x4 am[MT], aq[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) am[mt] = aq[mt] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p <= NP; ++p) {
      uint32_t word;
      if (p == NP) word = w[BQ];                       // QJL signs
      else if (p < BQ) word = w[p];                    // single index bits
      else word = w[0] ^ w[1] ^ w[2];                  // parity of 3 bits
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
    if (!valid) continue;
    const float n = (float)__builtin_bit_cast(_Float16, (uint16_t)(sc & 0xffff));
    const float gk = (float)__builtin_bit_cast(_Float16, (uint16_t)(sc >> 16)) * a.kappa;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int head = mt * 8 + 2 * kg + e;
        const float mse = (float)(am[mt][2 * e] * 128 + am[mt][2 * e + 1]) * cst[mt][e][0] + cst[mt][e][1];
        const float qjl = (float)(aq[mt][2 * e] * 128 + aq[mt][2 * e + 1]) * cst[mt][e][2] + cst[mt][e][3];
        if (head < a.group) out[(size_t)head * a.T + t] = n * fmaf(gk, qjl, mse);
      }
    }
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
  hipLaunchKernelGGL(prep_queries128, dim3(a.segs), dim3(128), 0, stream, p);
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
