// Top-k retrieval at d_rot = 2048 (sign-flipped Hadamard rotation) over
// TurboQuant-prod keys or MSE-only records: for each query q, the k records of
// largest estimated inner product
//   prod:  s(q, t) = n_t ( <Pi q, c[idx_t]> + gamma_t sqrt(pi/2)/m <S Pi q, 2 z_t - 1> )
//   MSE:   s(q, t) = n_t <Pi q, c[idx_t]>
// (explainer page, section 8; blog notes, the prod estimator read with the
// stored ||r||_2), ties to the lower record index.
//
// Query side (three launches, two without the QJL matrix): the 2048-point
// Walsh-Hadamard transform per query in registers; q_proj = S q_rot as a
// 2048 x 2048 fp16 hi/lo MFMA GEMM over all queries; then per query the
// statistics and the quantised weights, written as int8 A-operand fragments
// of v_mfma_i32_16x16x64_i8 in balanced base 256, two digits (16 bits
// relative to the query's largest weight; the rounding errors of 2048
// coordinates average down, and the estimates stay within 1e-3 of the row
// maximum at every bit width).
//
// Record side, per chunk of records (two launches): the bit-plane contraction
// of the query weights with the records' bits (the same Walsh-plane form as
// the decode kernels: MSE planes and the QJL plane, bytes in {0, 1} on the
// B operand) writes a score block [queries][records]; then one workgroup per
// query keeps the block's top k.  A last launch merges the chunks' candidates.
//
// Score GEMM tiling: a workgroup (4 waves) holds 4 query row tiles (32
// queries) and 128 records (2 column tiles of 16 per wave); the K loop runs
// over 16 chunks of 128 coordinates, the query fragments of the next chunk
// going global -> registers -> LDS while the current chunk is computed.
// Consecutive workgroups walk records with the same queries, whose fragments
// stay in L2.
#include <cmath>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int D2 = 2048;
constexpr int NCH = D2 / 128;            // 128-coordinate chunks
constexpr float RQMAX2 = 32512.f;        // 127 * 2^8
constexpr int RTQ = 4;                   // query row tiles per score workgroup
constexpr int KMAX = 16;                 // largest k

__host__ __device__ constexpr int r_planes(int bq) { return bq == 3 ? 4 : bq == 4 ? 8 : bq; }   // MSE Walsh planes
// Odd subsets of the bq index bits in plane order: single bits, then the
// parity of 3 bits, or for 4 bits the four three-bit parities.
__host__ __device__ constexpr int r_subset(int bq, int p) {
  return p < bq ? 1 << p : bq == 3 ? 7 : (p == 4 ? 7 : p == 5 ? 11 : p == 6 ? 13 : 14);
}
// A fragments per chunk per row tile: two per MSE plane, two for the QJL plane
__host__ __device__ constexpr int r_frags(int bq, int qjl) { return 2 * (r_planes(bq) + qjl); }
constexpr int RQPT = 8;                  // queries per row tile (two A rows each)

struct RetrArgs {
  const float* q;          // [nq][ld_q]
  int nq, nqp, d, ld_q;    // nqp: queries padded to whole score workgroups
  int bq;
  int qjl;                 // 1: prod keys (QJL plane), 0: MSE-only records
  const float* eps;        // [rounds][2048]
  int rounds;
  int m;                   // QJL rows: 2048, or 1024
  const float* s;          // [2048][2048], prod only
  float u[8];
  float usum;
  float kappa;
  // workspace
  _Float16 *s_hi, *s_lo;   // [2048][2048]
  float* qrot;             // [nqp][2048]
  _Float16 *qh, *ql;       // [nqp][2048] scaled q_rot, fp16 hi / lo
  float* qscale;           // [nqp] scale undone after the projection
  float* qproj;            // [nqp][2048]
  uint8_t* pack;           // [nrt][16 chunks][F][64 lanes][16 B]
  float* consts;           // [nqp][4]: sigma_mse, const_mse, kappa sigma_qjl, kappa const_qjl
};

__global__ __launch_bounds__(256) void r_split_s(const float* __restrict__ s, _Float16* hi, _Float16* lo, int64_t cnt) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < cnt; i += (int64_t)gridDim.x * 256) {
    _Float16 h, l;
    split_f16(s[i], h, l);
    hi[i] = h;
    lo[i] = l;
  }
}

// One wave per (padded) query: q_rot = H diag(eps) pad(q) / sqrt(2048), and a
// power-of-two scaled fp16 hi/lo copy for the projection GEMM.
__global__ __launch_bounds__(256) void r_rotate(RetrArgs a) {
  const int lane = threadIdx.x & 63;
  const int q = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (q >= a.nqp) return;
  const int j0 = 32 * lane;
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = 0.f;
  if (q < a.nq) {
    const float* src = a.q + (int64_t)q * a.ld_q + j0;
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
      if (j0 + i < a.d) {
        const float4 f = *reinterpret_cast<const float4*>(src + i);
        v[i] = f.x; v[i + 1] = f.y; v[i + 2] = f.z; v[i + 3] = f.w;
      }
    }
  }
  const float4* e4 = reinterpret_cast<const float4*>(a.eps + j0);
#pragma unroll
  for (int i = 0; i < 32; i += 4) {
    const float4 e = e4[i / 4];
    v[i] *= e.x; v[i + 1] *= e.y; v[i + 2] *= e.z; v[i + 3] *= e.w;
  }
  fwht2048_wave(v, lane);
#pragma unroll 1
  for (int r = 1; r < a.rounds; ++r) {     // further Hadamard rounds
    const float4* er = reinterpret_cast<const float4*>(a.eps + (size_t)r * D2 + j0);
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
      const float4 e = er[i / 4];
      v[i] *= 0.02209708691207961f * e.x; v[i + 1] *= 0.02209708691207961f * e.y;
      v[i + 2] *= 0.02209708691207961f * e.z; v[i + 3] *= 0.02209708691207961f * e.w;
    }
    fwht2048_wave(v, lane);
  }
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] *= 0.02209708691207961f;   // 1 / sqrt(2048)
    mx = fmaxf(mx, fabsf(v[i]));
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, shfl_xor_f(mx, o));
  // scale by 2^-e with 2^e > max |q_rot| (exact), so |q_rot scaled| < 1
  const float sc = mx > 0.f ? ldexpf(1.f, -(ilogbf(mx) + 1)) : 1.f;
  float* dr = a.qrot + (int64_t)q * D2 + j0;
  half8 hh[4], hl[4];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    dr[i] = v[i];
    _Float16 h, l;
    split_f16(v[i] * sc * 1024.f, h, l);   // 2^10 keeps the lo part normal
    hh[i / 8][i % 8] = h;
    hl[i / 8][i % 8] = l;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    reinterpret_cast<half8*>(a.qh + (int64_t)q * D2 + j0)[k] = hh[k];
    reinterpret_cast<half8*>(a.ql + (int64_t)q * D2 + j0)[k] = hl[k];
  }
  if (lane == 0) a.qscale[q] = 1.f / (sc * 1024.f);
}

// q_proj[q][i] = sum_k q_rot[q][k] S[i][k]: 128 x 128 tiles, a wave owns 64 x 64
// (2 x 2 accumulators of 32 x 32), fp16 hi/lo with the lo*lo term dropped.
__global__ __launch_bounds__(256) void r_project(RetrArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int qw = blockIdx.y * 128 + 64 * (wave >> 1);
  const int iw = blockIdx.x * 128 + 64 * (wave & 1);
  const int l32 = lane & 31, kh = lane >> 5;
  const _Float16* ah = a.qh + (int64_t)(qw + l32) * D2 + 8 * kh;
  const _Float16* al = a.ql + (int64_t)(qw + l32) * D2 + 8 * kh;
  const _Float16* bh = a.s_hi + (int64_t)(iw + l32) * D2 + 8 * kh;
  const _Float16* bl = a.s_lo + (int64_t)(iw + l32) * D2 + 8 * kh;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  for (int k0 = 0; k0 < D2; k0 += 16) {
    half8 Ah[2], Al[2], Bh[2], Bl[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      Ah[t] = *reinterpret_cast<const half8*>(ah + (int64_t)32 * t * D2 + k0);
      Al[t] = *reinterpret_cast<const half8*>(al + (int64_t)32 * t * D2 + k0);
      Bh[t] = *reinterpret_cast<const half8*>(bh + (int64_t)32 * t * D2 + k0);
      Bl[t] = *reinterpret_cast<const half8*>(bl + (int64_t)32 * t * D2 + k0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        acc[i][j] = mfma32x32x16(Ah[i], Bh[j], acc[i][j]);
        acc[i][j] = mfma32x32x16(Al[i], Bh[j], acc[i][j]);
        acc[i][j] = mfma32x32x16(Ah[i], Bl[j], acc[i][j]);
      }
  }
  // accumulator register r: row (query) 8 (r / 4) + 4 kh + r % 4, column (output) l32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = qw + 32 * i + 8 * (r >> 2) + 4 * kh + (r & 3);
        a.qproj[(int64_t)q * D2 + iw + 32 * j + l32] = acc[i][j][r] * a.qscale[q];
      }
}

// integer weight -> balanced base-256 int8 digits: q = 256 d0 + d1
__device__ __forceinline__ void digits(float w, int& d0, int& d1) {
  const int qi = (int)rintf(fminf(fmaxf(w, -RQMAX2), RQMAX2));
  d0 = (qi + 128) >> 8;
  d1 = qi - 256 * d0;
}

// One wave per (padded) query: statistics, then the int8 digit fragments.
// Lane l holds coordinates 32 l .. 32 l + 31 = chunk l / 4, lane group l % 4
// of the fragments, bit b of the group's word = coordinate 32 (l % 4) + b:
// byte (b / 8) of dword (b % 4) of MFMA ((b / 4) % 2).
__global__ __launch_bounds__(256) void r_pack(RetrArgs a) {
  const int lane = threadIdx.x & 63;
  const int q = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (q >= a.nqp) return;
  const int np = r_planes(a.bq), F = r_frags(a.bq, a.qjl);
  constexpr int R = 2;                                // A rows (digits) per query
  const bool live = q < a.nq;
  float vr[32], vp[32];
  float mx = 0.f, sr = 0.f, px = 0.f, sp = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    vr[i] = live ? a.qrot[(int64_t)q * D2 + 32 * lane + i] : 0.f;
    vp[i] = live && a.qjl && 32 * lane + i < a.m ? a.qproj[(int64_t)q * D2 + 32 * lane + i] : 0.f;
    mx = fmaxf(mx, fabsf(vr[i]));
    px = fmaxf(px, fabsf(vp[i]));
    sr += vr[i];
    sp += vp[i];
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    mx = fmaxf(mx, shfl_xor_f(mx, o));
    px = fmaxf(px, shfl_xor_f(px, o));
    sr += shfl_xor_f(sr, o);
    sp += shfl_xor_f(sp, o);
  }
  float umax = 0.f;
  for (int p = 0; p < np; ++p) umax = fmaxf(umax, fabsf(2.f * a.u[p]));
  const float qm = RQMAX2;
  const float sm = mx * umax > 0.f ? mx * umax / qm : 1.f;
  const float sq = px > 0.f ? 2.f * px / qm : 1.f;
  if (lane == 0) {
    a.consts[4 * q + 0] = live ? sm : 0.f;
    a.consts[4 * q + 1] = live ? -a.usum * sr : 0.f;
    a.consts[4 * q + 2] = live ? sq * a.kappa : 0.f;
    a.consts[4 * q + 3] = live ? -sp * a.kappa : 0.f;
  }
  const int rt = q / RQPT, qq = q % RQPT;
  const int c = lane >> 2, kg = lane & 3;
  for (int p = 0; p < np + a.qjl; ++p) {
    float up = a.u[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) up = p == i ? a.u[i] : up;
    const float wsc = p < np ? 2.f * up / sm : 2.f / sq;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      uint8_t* frag = a.pack + ((((int64_t)rt * NCH + c) * F + 2 * p + m) * 64) * 16;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        int dd[R][4];
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
          const int b = 8 * ib + 4 * m + k;
          const float w = live ? (p < np ? vr[b] : vp[b]) * wsc : 0.f;
          digits(w, dd[0][ib], dd[1][ib]);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint32_t word = (uint32_t)(dd[r][0] & 0xff) | ((uint32_t)(dd[r][1] & 0xff) << 8) |
                                ((uint32_t)(dd[r][2] & 0xff) << 16) | ((uint32_t)(dd[r][3] & 0xff) << 24);
          *reinterpret_cast<uint32_t*>(frag + 16 * (16 * kg + R * qq + r) + 4 * k) = word;
        }
      }
    }
  }
}

__device__ __forceinline__ void expand8r(uint32_t w, uint32_t e[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) e[k] = (w >> k) & 0x01010101u;
}

struct ScoreBlockArgs {
  const uint8_t* pack;
  const float* consts;
  const uint32_t* planes;    // records, key layout with W = 64
  const uint16_t* scalars;
  int64_t T;                 // records
  int64_t r0, rc;            // chunk: first record, records
  int nq;
  float* scores;             // [nq][rc]
};

// HALF: prod records with m = 1024 QJL rows (for each group g its index
// words, then sign word g while g < 32); the lanes of groups 32..63 load the P
// words ending with the group's last index word and rotate them into place, so
// the sign slot holds a foreign word, whose QJL weights (rows >= 1024) are zero.
template <int BQ, int QJL, bool HALF = false>
__global__ __launch_bounds__(256) void r_score_block(ScoreBlockArgs a) {
  constexpr int NP = r_planes(BQ), F = r_frags(BQ, QJL), QPT = RQPT;
  constexpr int P = BQ + QJL;
  constexpr int MWD = HALF ? 32 : 64;                   // sign words per record
  constexpr int RW = QJL ? 64 * BQ + MWD : 64 * P;     // words per record
  constexpr int HL = 2;                         // queries per lane group per row tile
  constexpr int FR = RTQ * F * 64;              // 16-byte fragment units per chunk per workgroup
  constexpr int LPT = FR / 256;                 // of them per thread
  typedef typename Words<P>::v wvec;
  __shared__ __align__(16) uint4 afr[FR];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t16 = lane & 15, kg = lane >> 4;
  const int rt0 = blockIdx.y * RTQ;              // first query row tile
  const int64_t rec0 = a.r0 + (int64_t)blockIdx.x * 128 + 32 * wave;   // this wave's 32 records
  const rsrc_t rk = make_rsrc(a.planes + a.r0 * RW, clamp_bytes((a.T - a.r0) * (int64_t)(RW * 4)));
  const uint4* gpack = reinterpret_cast<const uint4*>(a.pack);
  auto gfrag = [&](int c, int u) {   // u-th 16-byte unit of chunk c of this workgroup's row tiles
    const int rt = u / (F * 64), rem = u % (F * 64);
    return gpack[((int64_t)(rt0 + rt) * NCH + c) * F * 64 + rem];
  };
  uint4 nxt[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) nxt[i] = gfrag(0, threadIdx.x + 256 * i);
  auto rec_words = [&](int c, int ct) {
    const int64_t rec = rec0 + 16 * ct + t16;
    const int g = 4 * c + kg;
    const bool late = HALF && g >= MWD;
    const int goff = late ? MWD * P + (g - MWD) * BQ - 1 : g * P;
    const uint32_t off = rec < a.T ? (uint32_t)(((rec - a.r0) * RW + goff) * 4) : OOB_OFFSET;
    wvec w = load_words<P>(rk, off);
    if constexpr (HALF) {
      wvec r;
#pragma unroll
      for (int i = 0; i < P; ++i) r[i] = late ? w[(i + 1) % P] : w[i];
      w = r;
    }
    return w;
  };
  wvec wn[2];
  wn[0] = rec_words(0, 0);
  wn[1] = rec_words(0, 1);
  i32x4 am[RTQ][2], aq[RTQ][2];
#pragma unroll
  for (int r = 0; r < RTQ; ++r)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) am[r][ct] = aq[r][ct] = i32x4{0, 0, 0, 0};
  for (int c = 0; c < NCH; ++c) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < LPT; ++i) afr[threadIdx.x + 256 * i] = nxt[i];
    __syncthreads();
    const wvec w0 = wn[0], w1 = wn[1];
    if (c + 1 < NCH) {
#pragma unroll
      for (int i = 0; i < LPT; ++i) nxt[i] = gfrag(c + 1, threadIdx.x + 256 * i);
      wn[0] = rec_words(c + 1, 0);
      wn[1] = rec_words(c + 1, 1);
    }
#pragma unroll
    for (int p = 0; p < NP + QJL; ++p) {
      uint32_t e0[8], e1[8];
      uint32_t x0 = 0u, x1 = 0u;
      if (p == NP) {
        if constexpr (QJL) {
          x0 = w0[BQ];
          x1 = w1[BQ];
        }
      } else {
#pragma unroll
        for (int b = 0; b < BQ; ++b)
          if (r_subset(BQ, p) >> b & 1) {
            x0 ^= w0[b];
            x1 ^= w1[b];
          }
      }
      expand8r(x0, e0);
      expand8r(x1, e1);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const i32x4 b0 = {(int)e0[4 * m], (int)e0[4 * m + 1], (int)e0[4 * m + 2], (int)e0[4 * m + 3]};
        const i32x4 b1 = {(int)e1[4 * m], (int)e1[4 * m + 1], (int)e1[4 * m + 2], (int)e1[4 * m + 3]};
#pragma unroll
        for (int r = 0; r < RTQ; ++r) {
          const i32x4 av = __builtin_bit_cast(i32x4, afr[(r * F + 2 * p + m) * 64 + lane]);
          if (p == NP) {
            aq[r][0] = mfma16x16x64i8(av, b0, aq[r][0]);
            aq[r][1] = mfma16x16x64i8(av, b1, aq[r][1]);
          } else {
            am[r][0] = mfma16x16x64i8(av, b0, am[r][0]);
            am[r][1] = mfma16x16x64i8(av, b1, am[r][1]);
          }
        }
      }
    }
  }
  // epilogue: lane group kg holds rows 4 kg .. 4 kg + 3 of each row tile
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int64_t rec = rec0 + 16 * ct + t16;
    if (rec >= a.T || rec >= a.r0 + a.rc) continue;
    const uint32_t sc = QJL ? reinterpret_cast<const uint32_t*>(a.scalars)[rec] : (uint32_t)a.scalars[rec];
    const float n = (float)__builtin_bit_cast(_Float16, (uint16_t)(sc & 0xffff));
    const float g = (float)__builtin_bit_cast(_Float16, (uint16_t)(sc >> 16));
#pragma unroll
    for (int r = 0; r < RTQ; ++r) {
#pragma unroll
      for (int hh = 0; hh < HL; ++hh) {
        const int q = (rt0 + r) * QPT + HL * kg + hh;
        if (q >= a.nq) continue;
        // int32: |hi digit sum| <= 127 x 2048 x 8 planes, times 256 stays below 2^31
        const float im = (float)(am[r][ct][2 * hh] * 256 + am[r][ct][2 * hh + 1]);
        const float iq = (float)(aq[r][ct][2 * hh] * 256 + aq[r][ct][2 * hh + 1]);
        const float* cq = a.consts + 4 * q;
        const float mse = fmaf(im, cq[0], cq[1]);
        if constexpr (QJL) {
          const float qjl = fmaf(iq, cq[2], cq[3]);
          a.scores[(int64_t)q * a.rc + (rec - a.r0)] = n * fmaf(g, qjl, mse);
        } else {
          (void)iq;
          a.scores[(int64_t)q * a.rc + (rec - a.r0)] = n * mse;
        }
      }
    }
  }
}

// ---- top k: (value desc, index asc) ----
__device__ __forceinline__ bool better(float v, int64_t i, float w, int64_t j) {
  return v > w || (v == w && i < j);
}

struct TopkArgs {
  const float* val;        // [rows][ld] values
  const int64_t* idx;      // [rows][n] indices, or null: index = base + position
  int64_t n;               // entries per row
  int64_t ld;              // row stride of val / idx
  int64_t base;
  int k;
  float* oval;             // [rows][ostride] outputs
  int64_t* oidx;
  int64_t ostride;
};

// One workgroup per row: each thread keeps its own best k of a strided scan,
// then k rounds of a workgroup-wide selection of the best remaining head.
__global__ __launch_bounds__(256) void r_topk(TopkArgs a) {
  __shared__ float sv[256];
  __shared__ int64_t si[256];
  __shared__ int st[256];
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  float bv[KMAX];
  int64_t bi[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    bv[j] = -INFINITY;
    bi[j] = INT64_MAX;
  }
  const float* vr = a.val + (int64_t)row * a.ld;
  const int64_t* ir = a.idx ? a.idx + (int64_t)row * a.ld : nullptr;
  auto consider = [&](float v, int64_t i) {
    if (!better(v, i, bv[KMAX - 1], bi[KMAX - 1])) return;
    // insert, keeping bv sorted best first
    float cv = v;
    int64_t ci = i;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (better(cv, ci, bv[j], bi[j])) {
        const float tv = bv[j];
        const int64_t ti = bi[j];
        bv[j] = cv;
        bi[j] = ci;
        cv = tv;
        ci = ti;
      }
    }
  };
  int64_t e0 = 0;
  if (!ir && (a.ld & 3) == 0) {
    // a block of scores: 16-byte loads, four per thread in flight (the
    // result does not depend on the visiting order: ties go by index)
    const float4* v4 = reinterpret_cast<const float4*>(vr);
    const int64_t n4 = a.n >> 2;
    for (int64_t q = t; q < n4; q += 4 * 256) {
      float4 x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = q + 256 * u < n4 ? v4[q + 256 * u] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (q + 256 * u >= n4) break;
        const int64_t i0 = a.base + 4 * (q + 256 * u);
        consider(x[u].x, i0);
        consider(x[u].y, i0 + 1);
        consider(x[u].z, i0 + 2);
        consider(x[u].w, i0 + 3);
      }
    }
    e0 = 4 * n4;
  }
  for (int64_t e = e0 + t; e < a.n; e += 256) consider(vr[e], ir ? ir[e] : a.base + e);
  int head = 0;
  for (int r = 0; r < a.k; ++r) {
    float hv = -INFINITY;
    int64_t hi = INT64_MAX;
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j == head) {
        hv = bv[j];
        hi = bi[j];
      }
    sv[t] = hv;
    si[t] = hi;
    st[t] = t;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if (t < s && better(sv[t + s], si[t + s], sv[t], si[t])) {
        sv[t] = sv[t + s];
        si[t] = si[t + s];
        st[t] = st[t + s];
      }
      __syncthreads();
    }
    if (t == 0) {
      a.oval[(int64_t)row * a.ostride + r] = sv[0];
      a.oidx[(int64_t)row * a.ostride + r] = si[0];
    }
    if (t == st[0]) ++head;
    __syncthreads();
  }
}

template <int BQ, int QJL>
hipError_t score_blocks(const ScoreBlockArgs& b, int nrt, hipStream_t stream, bool half = false) {
  const dim3 grid((unsigned)((b.rc + 127) / 128), (unsigned)((nrt + RTQ - 1) / RTQ));
  if constexpr (QJL == 1) {
    if (half) {
      hipLaunchKernelGGL((r_score_block<BQ, QJL, true>), grid, dim3(256), 0, stream, b);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((r_score_block<BQ, QJL>), grid, dim3(256), 0, stream, b);
  return hipGetLastError();
}

}  // namespace

// records per score block
static int64_t block_records(int64_t T) { return T < 65536 ? (T + 127) / 128 * 128 : 65536; }

static int padded_queries(int nq, int bq) {
  (void)bq;
  const int per = RQPT * RTQ;   // queries per score workgroup
  return (nq + per - 1) / per * per;
}

size_t topk2k_workspace(int nq, int64_t T, int k, int bq, int qjl) {
  const int nqp = (padded_queries(nq, bq) + 127) / 128 * 128;
  const int64_t rc = block_records(T);
  const int64_t nch = (T + rc - 1) / rc;
  const int nrt = padded_queries(nq, bq) / RQPT;
  size_t s = 0;
  auto add = [&](size_t b) { s += (b + 255) / 256 * 256; };
  add((size_t)2 * D2 * D2 * 2);              // S hi, lo
  add((size_t)nqp * D2 * 4);                 // q_rot
  add((size_t)2 * nqp * D2 * 2);             // q hi, lo
  add((size_t)nqp * 4);                      // scale
  add((size_t)nqp * D2 * 4);                 // q_proj
  add((size_t)nrt * NCH * r_frags(bq, qjl) * 1024);   // fragments
  add((size_t)nqp * 16);                     // constants
  add((size_t)nq * rc * 4);                  // score block
  add((size_t)nq * nch * k * 4);             // candidate values
  add((size_t)nq * nch * k * 8);             // candidate indices (int64)
  return s;
}

hipError_t launch_topk2k(const TopkLaunch& L, hipStream_t stream) {
  const int bq = L.bq;
  RetrArgs a;
  a.q = L.q;
  a.nq = L.nq;
  a.nqp = (padded_queries(L.nq, bq) + 127) / 128 * 128;
  a.d = L.d;
  a.ld_q = L.d;
  a.bq = bq;
  a.qjl = L.qjl;
  a.eps = L.eps;
  a.rounds = L.rounds;
  a.s = L.s;
  for (int i = 0; i < 8; ++i) a.u[i] = L.u[i];
  a.usum = L.usum;
  a.m = L.qjl ? L.m : D2;
  a.kappa = (float)(std::sqrt(M_PI / 2.0) / a.m);
  const int64_t rc = block_records(L.T);
  const int64_t nch = (L.T + rc - 1) / rc;
  const int nrt = padded_queries(L.nq, bq) / RQPT;
  uint8_t* w = static_cast<uint8_t*>(L.ws);
  auto take = [&](size_t b) {
    uint8_t* p = w;
    w += (b + 255) / 256 * 256;
    return p;
  };
  a.s_hi = reinterpret_cast<_Float16*>(take((size_t)D2 * D2 * 2 * 2));
  a.s_lo = a.s_hi + (size_t)D2 * D2;
  a.qrot = reinterpret_cast<float*>(take((size_t)a.nqp * D2 * 4));
  a.qh = reinterpret_cast<_Float16*>(take((size_t)2 * a.nqp * D2 * 2));
  a.ql = a.qh + (size_t)a.nqp * D2;
  a.qscale = reinterpret_cast<float*>(take((size_t)a.nqp * 4));
  a.qproj = reinterpret_cast<float*>(take((size_t)a.nqp * D2 * 4));
  a.pack = take((size_t)nrt * NCH * r_frags(bq, L.qjl) * 1024);
  a.consts = reinterpret_cast<float*>(take((size_t)a.nqp * 16));
  float* block = reinterpret_cast<float*>(take((size_t)L.nq * rc * 4));
  // candidate values and indices in regions of their own (the int64 indices
  // 256-byte aligned whatever nq * nch * k is)
  float* cval = reinterpret_cast<float*>(take((size_t)L.nq * nch * L.k * 4));
  int64_t* cidx = reinterpret_cast<int64_t*>(take((size_t)L.nq * nch * L.k * 8));

  if (L.qjl) hipLaunchKernelGGL(r_split_s, dim3(1024), dim3(256), 0, stream, L.s, a.s_hi, a.s_lo, (int64_t)a.m * D2);
  hipLaunchKernelGGL(r_rotate, dim3((unsigned)(a.nqp / 4)), dim3(256), 0, stream, a);
  if (L.qjl) hipLaunchKernelGGL(r_project, dim3((unsigned)(a.m / 128), (unsigned)(a.nqp / 128)), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(r_pack, dim3((unsigned)(padded_queries(L.nq, bq) / 4)), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ScoreBlockArgs b;
  b.pack = a.pack;
  b.consts = a.consts;
  b.planes = L.planes;
  b.scalars = L.scalars;
  b.T = L.T;
  b.rc = rc;
  b.nq = L.nq;
  b.scores = block;
  for (int64_t ch = 0; ch < nch; ++ch) {
    b.r0 = ch * rc;
    switch (bq * 2 + L.qjl) {
      case 3: e = score_blocks<1, 1>(b, nrt, stream, a.m < D2); break;
      case 5: e = score_blocks<2, 1>(b, nrt, stream, a.m < D2); break;
      case 7: e = score_blocks<3, 1>(b, nrt, stream, a.m < D2); break;
      case 2: e = score_blocks<1, 0>(b, nrt, stream); break;
      case 4: e = score_blocks<2, 0>(b, nrt, stream); break;
      case 6: e = score_blocks<3, 0>(b, nrt, stream); break;
      case 8: e = score_blocks<4, 0>(b, nrt, stream); break;
      default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    TopkArgs t;
    t.val = block;
    t.idx = nullptr;
    t.n = L.T - b.r0 < rc ? L.T - b.r0 : rc;
    t.ld = rc;
    t.base = b.r0;
    t.k = L.k;
    t.oval = cval + ch * L.k;
    t.oidx = cidx + ch * L.k;
    t.ostride = nch * L.k;
    hipLaunchKernelGGL(r_topk, dim3((unsigned)L.nq), dim3(256), 0, stream, t);
  }
  TopkArgs t;
  t.val = cval;
  t.idx = cidx;
  t.n = nch * L.k;
  t.ld = nch * L.k;
  t.base = 0;
  t.k = L.k;
  t.oval = L.val;
  t.oidx = L.idx;
  t.ostride = L.k;
  hipLaunchKernelGGL(r_topk, dim3((unsigned)L.nq), dim3(256), 0, stream, t);
  return hipGetLastError();
}

}  // namespace tq
