// PolarQuant as stage 1 at d = 128: the score pass over polar keys and the
// dequantizer (FastVQ README, "PolarQuant Algorithm" in its recursive form and
// "TurboQuant Combination" for the QJL stage; the encoder is in tq_encode.hip).
//
// Record of a key (u32 words): level-1 stream (64 codes of B1 bits, 2 B1
// words), upper stream (the 63 codes of levels 2..7 level by level, B bits
// each, 2 B words), then 4 QJL sign words when the record has them.  Level l
// starts at position 64 - 128 / 2^(l-1) of the upper stream: 0, 32, 48, 56,
// 60, 62.  The children of angle j of level l are the blocks 2j, 2j+1 of level
// l-1; level 1's children are coordinates 2j, 2j+1.
//
// Score of query head g against token t:
//   s = n_t ( <q'_g, y~_t> + gamma_t <kappa S q'_g, 2 z_t - 1> ),  q'_g = rot(q_g).
// y~_t is linear in the level-1 lengths rho_j (products of the upper
// centroid cos/sin along the path) once the level-1 codes are fixed:
//   <q', y~> = sum_j rho_j (q'[2j] cos c1_j + q'[2j+1] sin c1_j),
// so each workgroup tabulates the bracket for every pair j and level-1 code
// (64 x 2^B1 entries per head) and the QJL term for every nibble of sign bits
// (32 x 16 entries per head) in the LDS, and a lane per token walks the tree
// down from the unit length (63 centroid lookups) and sums 64 table entries
// (+ 32 for the signs) per head.  The tables keep the heads innermost, so one
// 16-byte LDS read serves four heads.
#include <algorithm>
#include <cmath>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int D = 128;
constexpr int PS_THREADS = 256;

template <int W, int N>
__device__ __forceinline__ uint32_t code_at(const uint32_t (&w)[N], int pos) {
  uint32_t c = w[pos >> 5] >> (pos & 31);
  if ((pos & 31) + W > 32) c |= w[(pos >> 5) + 1] << (32 - (pos & 31));
  return c & ((1u << W) - 1);
}

// Split the NP lengths rin of one level into the 2 NP lengths below with the
// centroid pairs of the level's codes (upper-stream positions OFF + j).
template <int B, int NP, int LI, int OFF, int NW>
__device__ __forceinline__ void descend(const float (&rin)[NP], float (&rout)[2 * NP], const uint32_t (&us)[NW],
                                        const float2* tu) {
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const float2 t = tu[16 * LI + code_at<B>(us, (OFF + j) * B)];
    rout[2 * j] = rin[j] * t.x;
    rout[2 * j + 1] = rin[j] * t.y;
  }
}

// The 16 lengths of the level-3 blocks (8 coordinates each) of a record,
// from the unit length down through levels 7..4 of its upper stream.
template <int B, int NW>
__device__ __forceinline__ void level3_lengths(const uint32_t (&us)[NW], const float2* tu, float (&r3)[16]) {
  const float2 t7 = tu[16 * 5 + code_at<B>(us, 62 * B)];
  float r6[2] = {t7.x, t7.y};
  float r5[4], r4[8];
  descend<B, 2, 4, 60>(r6, r5, us, tu);
  descend<B, 4, 3, 56>(r5, r4, us, tu);
  descend<B, 8, 2, 48>(r4, r3, us, tu);
}

// In-place Walsh-Hadamard transform (Sylvester order) of nv vectors of 128
// floats in the LDS; the caller synchronises before and after.
__device__ void fwht128_lds(float* v, int nv) {
  for (int h = 1; h < D; h <<= 1) {
    for (int p = threadIdx.x; p < nv * (D / 2); p += blockDim.x) {
      const int g = p / (D / 2), k = p % (D / 2);
      const int lo = g * D + (k / h) * 2 * h + (k % h), hi = lo + h;
      const float x = v[lo], y = v[hi];
      v[lo] = x + y;
      v[hi] = x - y;
    }
    __syncthreads();
  }
}

// out[g][i] = scale * sum_k M[i][k] in[g][k] for G rows of 128 (M row-major
// 128 x 128): thread (i, k half) keeps its 64 matrix entries in registers and
// serves every row; part holds the two halves.
__device__ void matvec128(const float* __restrict__ M, const float* in, float* part, float* out, int G,
                          float scale) {
  const int i = threadIdx.x & 127, kh = threadIdx.x >> 7;
  float m[64];
  const float4* row = reinterpret_cast<const float4*>(M + (size_t)i * D + 64 * kh);
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const float4 w = row[c];
    m[4 * c] = w.x; m[4 * c + 1] = w.y; m[4 * c + 2] = w.z; m[4 * c + 3] = w.w;
  }
  for (int g = 0; g < G; ++g) {
    const float* x = in + g * D + 64 * kh;
    float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 64; ++k) s4[k & 3] = fmaf(m[k], x[k], s4[k & 3]);
    part[(kh * G + g) * D + i] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
  }
  __syncthreads();
  for (int p = threadIdx.x; p < G * D; p += blockDim.x) out[p] = scale * (part[p] + part[G * D + p]);
  __syncthreads();
}

// Head quads of a segment's tables: 1, 2 or 4 (up to 16 heads).
__host__ __device__ constexpr int head_quads(int G) { return G <= 4 ? 1 : G <= 8 ? 2 : 4; }

// LDS layout of the score kernel, in floats (every region a multiple of 4).
struct ScoreLds {
  int qraw, qr, qs, part, t1, tn, tu, total;
  __host__ __device__ ScoreLds(int b1, bool qjl, int G) {
    const int GP = 4 * head_quads(G);
    qraw = 0;
    qr = qraw + G * D;
    qs = qr + G * D;
    part = qs + (qjl ? G * D : 0);
    t1 = part + 2 * G * D;
    tn = t1 + 64 * (1 << b1) * GP;
    tu = tn + (qjl ? 32 * 16 * GP : 0);
    total = tu + 2 * 16 * 7;
  }
};

template <int B1, int B, bool QJL>
__global__ __launch_bounds__(PS_THREADS) void polar_scores128(PolarArgs a) {
  constexpr int K1 = 1 << B1;
  constexpr int NW1 = 2 * B1, NWU = 2 * B, P = NW1 + NWU + (QJL ? 4 : 0);
  extern __shared__ float4 sm4[];
  float* sm = reinterpret_cast<float*>(sm4);
  const int G = a.group, NQ = head_quads(G), GP = 4 * NQ;
  const ScoreLds L(B1, QJL, G);
  float* qraw = sm + L.qraw;
  float* qr = sm + L.qr;
  float* qs = sm + L.qs;
  float* part = sm + L.part;
  float* t1 = sm + L.t1;
  float* tn = sm + L.tn;
  float2* tab1 = reinterpret_cast<float2*>(sm + L.tu);
  float2* tabu = tab1 + 16;

  const int seg = blockIdx.x / a.wps;
  const int64_t T = a.T, tpw = a.tpw;
  const int64_t t0 = (int64_t)(blockIdx.x % a.wps) * tpw;
  int64_t tend = a.len ? (int64_t)a.len[seg] : T;
  tend = tend < T ? tend : T;
  tend = tend < t0 + tpw ? tend : t0 + tpw;
  if (t0 >= tend) return;   // the whole workgroup: nothing to score

  // ---- the segment's query heads: rotate, project, tabulate ----
  const float* q = a.q + (size_t)seg * G * D;
  for (int p = threadIdx.x; p < G * D; p += PS_THREADS)
    qraw[p] = a.had ? q[p] * a.eps[p % D] : q[p];
  polar_tables_to_lds(a.book, tab1);
  __syncthreads();
  if (a.had) {
    fwht128_lds(qraw, G);
    for (int p = threadIdx.x; p < G * D; p += PS_THREADS) qr[p] = qraw[p] * 0.08838834764831845f;
    __syncthreads();
  } else {
    matvec128(a.pi, qraw, part, qr, G, 1.f);
  }
  if (QJL) matvec128(a.s, qr, part, qs, G, 1.2533141373155003f / D);   // kappa = sqrt(pi/2) / m
  for (int p = threadIdx.x; p < 64 * K1 * GP; p += PS_THREADS) {
    const int g = p % GP, c = (p / GP) % K1, j = p / (GP * K1);
    t1[p] = g < G ? fmaf(qr[g * D + 2 * j], tab1[c].x, qr[g * D + 2 * j + 1] * tab1[c].y) : 0.f;
  }
  if (QJL) {
    for (int p = threadIdx.x; p < 32 * 16 * GP; p += PS_THREADS) {
      const int g = p % GP, v = (p / GP) % 16, w = p / (GP * 16);
      float s = 0.f;
      if (g < G) {
#pragma unroll
        for (int i = 0; i < 4; ++i) s += ((v >> i) & 1) ? qs[g * D + 4 * w + i] : -qs[g * D + 4 * w + i];
      }
      tn[p] = s;
    }
  }
  __syncthreads();

  // ---- tokens: lane = token, wave = (block of 64 tokens, head quad) ----
  const int64_t rec0 = (int64_t)seg * a.seg_stride;
  const int lane = threadIdx.x & 63;
  const int64_t items = (tend - t0 + 63) / 64 * NQ;     // (token block, quad) pairs
  for (int64_t wi = threadIdx.x >> 6; wi < items; wi += PS_THREADS / 64) {
    const int quad = (int)(wi % NQ);
    const int64_t t = t0 + (wi / NQ) * 64 + lane;
    if (t >= tend) continue;
    const uint2* src = reinterpret_cast<const uint2*>(a.planes + (rec0 + t) * P);
    uint32_t wd[P];
#pragma unroll
    for (int i = 0; i < P / 2; ++i) {
      const uint2 w = src[i];
      wd[2 * i] = w.x;
      wd[2 * i + 1] = w.y;
    }
    uint32_t w1[NW1], us[NWU];
#pragma unroll
    for (int i = 0; i < NW1; ++i) w1[i] = wd[i];
#pragma unroll
    for (int i = 0; i < NWU; ++i) us[i] = wd[NW1 + i];
    float n, gam = 0.f;
    if (QJL) {
      const uint32_t sc = reinterpret_cast<const uint32_t*>(a.scalars)[rec0 + t];
      n = (float)__builtin_bit_cast(_Float16, (uint16_t)(sc & 0xffffu));
      gam = (float)__builtin_bit_cast(_Float16, (uint16_t)(sc >> 16));
    } else {
      n = (float)__builtin_bit_cast(_Float16, a.scalars[rec0 + t]);
    }
    // level-1 sums of the quad's heads, block by block: each level-3 block's
    // length splits into 2 then 4 pair lengths, each weighting its pair's
    // table entry
    const float* t1q = t1 + 4 * quad;
    float r3[16];
    level3_lengths<B>(us, tabu, r3);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const float2 t3 = tabu[16 + code_at<B>(us, (32 + b) * B)];
      const float r2[2] = {r3[b] * t3.x, r3[b] * t3.y};
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float2 t2 = tabu[code_at<B>(us, (2 * b + k) * B)];
        const float r1[2] = {r2[k] * t2.x, r2[k] * t2.y};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int j = 4 * b + 2 * k + e;
          acc += r1[e] * *reinterpret_cast<const f32x4*>(t1q + (j * K1 + (int)code_at<B1>(w1, j * B1)) * GP);
        }
      }
    }
    if (QJL) {
      const float* tnq = tn + 4 * quad;
      f32x4 aq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < 32; ++w) {
        const uint32_t v = (wd[NW1 + NWU + (w >> 3)] >> (4 * (w & 7))) & 15u;
        aq += *reinterpret_cast<const f32x4*>(tnq + (w * 16 + (int)v) * GP);
      }
      acc += gam * aq;
    }
    float* out = a.scores + ((size_t)seg * G + 4 * quad) * a.T + t;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (4 * quad + e < G) out[(size_t)e * a.T] = n * acc[e];
  }
}

// Dequantize: per pass 16 records; 16 lanes per record each rebuild one
// 8-coordinate block of y~ into the LDS (four lookups down to the block, then
// its level-3, level-2 and level-1 angles), then x~ = n rot^T(y~): dense as
// 2 x 128 threads of 8 records each with the thread's rotation column read
// from memory, Hadamard as an LDS transform.
template <int B1, int B>
__global__ __launch_bounds__(256) void polar_decode128(PolarArgs a) {
  constexpr int NW1 = 2 * B1, P = NW1 + 2 * B + 0;
  const int PR = P + (a.qjl ? 4 : 0);     // record words
  __shared__ float Y[16 * D];
  __shared__ float2 tab[16 * 7];
  polar_tables_to_lds(a.book, tab);
  __syncthreads();
  const float2* tab1 = tab;
  const float2* tabu = tab + 16;
  for (int64_t base = (int64_t)blockIdx.x * 16; base < a.n; base += (int64_t)gridDim.x * 16) {
    {
      const int vl = threadIdx.x >> 4, sub = threadIdx.x & 15;
      const int64_t rec = base + vl;
      float* yv = Y + vl * D + 8 * sub;
      if (rec < a.n) {
        const uint32_t* w = a.planes + rec * PR;
        auto code = [&](const uint32_t* stream, int pos, int width) {
          const int wi = pos >> 5, sh = pos & 31;
          uint32_t c = stream[wi] >> sh;
          if (sh + width > 32) c |= stream[wi + 1] << (32 - sh);
          return (int)(c & ((1u << width) - 1));
        };
        const uint32_t* us = w + NW1;
        // lengths down to level-3 block `sub` (8 coordinates): levels 7..4
        float rho = 1.f;
        {
          const float2 t = tabu[16 * 5 + code(us, 62 * B, B)];
          rho *= (sub >> 3) ? t.y : t.x;
        }
        {
          const float2 t = tabu[16 * 4 + code(us, (60 + (sub >> 3)) * B, B)];
          rho *= ((sub >> 2) & 1) ? t.y : t.x;
        }
        {
          const float2 t = tabu[16 * 3 + code(us, (56 + (sub >> 2)) * B, B)];
          rho *= ((sub >> 1) & 1) ? t.y : t.x;
        }
        {
          const float2 t = tabu[16 * 2 + code(us, (48 + (sub >> 1)) * B, B)];
          rho *= (sub & 1) ? t.y : t.x;
        }
        const float2 t3 = tabu[16 * 1 + code(us, (32 + sub) * B, B)];
        const float r2[2] = {rho * t3.x, rho * t3.y};
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const float2 t2 = tabu[code(us, (2 * sub + k) * B, B)];
          const float r1[2] = {r2[k] * t2.x, r2[k] * t2.y};
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int j = 4 * sub + 2 * k + e;     // level-1 pair
            const float2 c1 = tab1[code(w, j * B1, B1)];
            yv[4 * k + 2 * e] = r1[e] * c1.x;
            yv[4 * k + 2 * e + 1] = r1[e] * c1.y;
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) yv[e] = 0.f;
      }
    }
    __syncthreads();
    const int i = threadIdx.x & 127, vh = threadIdx.x >> 7;
    float acc[8];
    if (a.had) {
      fwht128_lds(Y, 16);
#pragma unroll
      for (int v = 0; v < 8; ++v) acc[v] = Y[(8 * vh + v) * D + i] * a.eps[i] * 0.08838834764831845f;
    } else {
#pragma unroll
      for (int v = 0; v < 8; ++v) acc[v] = 0.f;
      for (int k = 0; k < D; ++k) {
        const float p = a.pi[(size_t)k * D + i];      // rot^T: column i of pi
#pragma unroll
        for (int v = 0; v < 8; ++v) acc[v] = fmaf(p, Y[(8 * vh + v) * D + k], acc[v]);
      }
    }
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const int64_t rec = base + 8 * vh + v;
      if (rec < a.n) {
        const uint16_t nb = a.qjl ? a.scalars[2 * rec] : a.scalars[rec];
        a.out[rec * a.ld_out + i] = (float)__builtin_bit_cast(_Float16, nb) * acc[v];
      }
    }
    __syncthreads();   // Y is rewritten by the next pass
  }
}

int cu_count() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  return cus;
}

template <int B1, int B, bool QJL>
hipError_t scores3(const PolarArgs& a, hipStream_t stream) {
  auto kern = polar_scores128<B1, B, QJL>;
  const size_t lds = polar_scores128_lds(B1, QJL, a.group);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(a.segs * a.wps)), dim3(PS_THREADS), lds, stream, a);
  return hipGetLastError();
}

template <int B1, int B>
hipError_t scores2(const PolarArgs& a, hipStream_t stream) {
  return a.qjl ? scores3<B1, B, true>(a, stream) : scores3<B1, B, false>(a, stream);
}

template <int B1>
hipError_t scores1(const PolarArgs& a, hipStream_t stream) {
  switch (a.b) {
    case 1: return scores2<B1, 1>(a, stream);
    case 2: return scores2<B1, 2>(a, stream);
    case 3: return scores2<B1, 3>(a, stream);
    case 4: return scores2<B1, 4>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <int B1>
hipError_t decode1(const PolarArgs& a, hipStream_t stream) {
  const int grid = (int)std::min<int64_t>((a.n + 15) / 16, (int64_t)cu_count() * 8);
  switch (a.b) {
    case 1: hipLaunchKernelGGL((polar_decode128<B1, 1>), dim3(grid), dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((polar_decode128<B1, 2>), dim3(grid), dim3(256), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((polar_decode128<B1, 3>), dim3(grid), dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((polar_decode128<B1, 4>), dim3(grid), dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

size_t polar_scores128_lds(int b1, int qjl, int group) { return sizeof(float) * ScoreLds(b1, qjl, group).total; }

// Workgroups per segment: enough for about four per compute unit over the
// whole call, each with a multiple of 256 tokens (one per lane and pass), so
// that the per-workgroup query preparation stays a small part of its work.
hipError_t launch_polar_scores128(const PolarArgs& args, hipStream_t stream) {
  PolarArgs a = args;
  const int64_t passes = (a.T + PS_THREADS - 1) / PS_THREADS;
  const int64_t want = std::max<int64_t>(1, (4 * (int64_t)cu_count() + a.segs - 1) / a.segs);
  a.wps = (int)std::min<int64_t>(passes, want);
  a.tpw = (int64_t)PS_THREADS * ((passes + a.wps - 1) / a.wps);
  if ((int64_t)a.segs * a.wps > 0x7fffffffll) return hipErrorInvalidValue;
  switch (a.b1) {
    case 1: return scores1<1>(a, stream);
    case 2: return scores1<2>(a, stream);
    case 3: return scores1<3>(a, stream);
    case 4: return scores1<4>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_polar_decode128(const PolarArgs& a, hipStream_t stream) {
  switch (a.b1) {
    case 1: return decode1<1>(a, stream);
    case 2: return decode1<2>(a, stream);
    case 3: return decode1<3>(a, stream);
    case 4: return decode1<4>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
