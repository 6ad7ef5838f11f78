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
// written in base 256 with int8 digits (each in [-128, 127]): two digits,
// q = 256 hi + lo, for 16 bits, or three, q = 65536 hi + 256 mid + lo, for 24
// bits.  The digits become rows of the A operand of v_mfma_i32_16x16x64_i8:
// with two, rows 2 h' + {0, 1} (8 heads per 16-row tile); with three, rows
// 4 h' + {0, 1, 2} (4 heads per tile, row 4 h' + 3 zero).  Key bits become the
// B operand: bytes in {0, 1}, tokens on the N axis.  The int32 accumulators
// are exact (at most 128 terms, |sum| < 2^14 per digit row), and so is the
// base-256 recombination; the epilogue rescales, adds the constants and
// applies n_t and gamma_t.  Lane group kg of the 16x16 accumulator holds rows
// 4 kg .. 4 kg + 3, i.e. all digits of its heads for token lane % 16: the
// epilogue needs no cross-lane work.  Scores of keys with 1 or 2 MSE bits use
// two digits (within ~1e-4 of float arithmetic relative to the row maximum,
// half the matrix work); 3 MSE bits and the attention kernel use three (an
// error in a score becomes an error in an exponent there).
//
// K-slot map (any permutation is valid as long as A and B share it): lane
// group kg (= lane / 16) of every MFMA reads plane word kg (coordinates
// 32 kg .. 32 kg + 31); MFMA m in {0, 1} of a plane takes expansion dwords
// k = 4m .. 4m+3, dword k byte i being bit 8 i + k of the word.
#include <atomic>
#include <algorithm>
#include <chrono>
#include <mutex>
#include <cmath>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int D = 128;
constexpr float QMAX2 = 32512.f;     // 127 * 2^8: two base-256 int8 digits
constexpr float QMAX3 = 8323072.f;   // 127 * 2^16: three base-256 int8 digits

// Odd subsets of the bq index bits (the Walsh planes of an odd-symmetric
// codebook), in plane order: the single bits, then for 3 bits their parity
// and for 4 bits the four three-bit parities.
__host__ __device__ constexpr int mse_planes(int bq) { return bq == 3 ? 4 : bq == 4 ? 8 : bq; }
__host__ __device__ constexpr int plane_subset(int bq, int p) {
  return p < bq ? 1 << p : bq == 3 ? 7 : (p == 4 ? 7 : p == 5 ? 11 : p == 6 ? 13 : 14);
}

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
  float u[8];      // Walsh coefficients of the odd-subset planes
  float usum;
  int bq;
  int slices;      // base-256 digits per weight: 2 (8 heads per tile) or 3 (4 heads)
  int mt;          // 16-row tiles per segment
  uint8_t* ws;
  int n_sets, set_div;   // rotation sets: segment seg uses set (seg / set_div) % n_sets
  int m_rows;            // rows of one set's QJL matrix
  int seg_per_wg;        // prep_queries128: consecutive segments per workgroup (same rotation set)
};

// One workgroup (8 waves) per segment, or per group of consecutive segments
// whose heads together fill the 16 head columns.  Both 128x128 products run on the
// matrix cores (v_mfma_f32_16x16x32_bf16) with bf16 hi/lo splits of both
// operands (three products, ~2^-16 relative, far below the 2^-21 integer
// quantisation that follows; bf16 keeps fp32's range, so no rescaling):
//   q_rot^T = Pi . Q^T         (dense; the Hadamard form uses +-eps entries)
//   q_proj^T = S . q_rot^T
// wave w owns output rows 16 w .. 16 w + 15, heads on the N axis.  Every
// global operand is loaded up front (one memory round trip); per-head
// statistics reduce through shuffles and LDS; the quantiser then builds whole
// A-operand dwords (four coordinates, one slice) and stores them to the pack.
constexpr int MAXG = 16;
constexpr int QTS = D + 4;               // LDS row stride (floats) of the head-major q tiles
constexpr int PREP_THREADS = 512;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void split8_bf16(const float* v, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 h = (__bf16)v[e];
    hi[e] = h;
    lo[e] = (__bf16)(v[e] - (float)h);
  }
}

__device__ __forceinline__ void unpack8(float4 a, float4 b, float* v) {
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// integer weight -> balanced base-256 int8 digits: q = 65536 hi + 256 mid + lo;
// the two low digits span [-32896, 32639], hence the offset of hi
__device__ __forceinline__ void slices3(float w, int& hi, int& mid, int& lo) {
  const int qi = (int)rintf(fminf(fmaxf(w, -QMAX3), QMAX3));
  hi = (qi + 32896) >> 16;
  const int rem = qi - 65536 * hi;
  mid = (rem + 128) >> 8;
  lo = rem - 256 * mid;
}
// q = 256 hi + lo
__device__ __forceinline__ void slices2(float w, int& hi, int& lo) {
  const int qi = (int)rintf(fminf(fmaxf(w, -QMAX2), QMAX2));
  hi = (qi + 128) >> 8;
  lo = qi - 256 * hi;
}

__device__ __forceinline__ uint32_t pack4(int b0, int b1, int b2, int b3) {
  return (uint32_t)(b0 & 0xff) | ((uint32_t)(b1 & 0xff) << 8) | ((uint32_t)(b2 & 0xff) << 16) |
         ((uint32_t)b3 << 24);
}

// The one-launch scores' hand-over words of one segment (their protocol is
// described with the hand-over helpers below).
struct ScoreSync {
  uint64_t flag;
  uint64_t claim;
  uint64_t done;
  uint64_t pad;
};

struct PrepLds {
  float qr[MAXG * QTS];      // q_rot[head][coordinate]
  float qp[MAXG * QTS];      // q_proj[head][coordinate]
  float part[8][MAXG][4];
  float stat[MAXG][4];
  float wsc[9][MAXG];        // weight scale per (plane, head); row 8 is the QJL plane
  int own;                   // the claim was taken (one-launch producer)
};

// Segment seg's query pack -> dst (all 512 threads of the workgroup); S is the
// number of base-256 digits per weight; CPOL the cache policy of the pack's
// stores (the one-launch scores write it device-coherent for the workgroups
// of other XCDs).
// MW: QJL sign words per key (m / 32); with MW = 2 the QJL rows past 64 are
// zero, so the pack's QJL weights for coordinate groups 2 and 3 vanish.
// With cs (the one-launch producer of segment seg, ns = 1): the claim is
// exchanged at the start, its answer needed only before the first pack store
// (false: a consumer holds it and builds; nothing is stored), and the pack's
// zero count under this launch's tag is stored with the pack.  Returns
// whether the pack was written.
template <bool HAD, int S, int CPOL = 0, bool QJL = true, int MW = 4>
__device__ __forceinline__ bool prep_pack(const PrepArgs& a, int seg, int ns, PrepLds& L, uint8_t* dst,
                                          ScoreSync* cs = nullptr, uint64_t ticket = 0) {
  float* qr = L.qr;
  float* qp = L.qp;
  auto& part = L.part;
  auto& stat = L.stat;
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int G = a.group;
  const int np = mse_planes(a.bq);
  const int F = 2 * (np + (QJL ? 1 : 0));
  const int fbytes = (int)pack_frag_bytes(a.mt, F);
  const uint32_t pbytes = (uint32_t)pack_bytes(a.mt, F);
  // this segment's rotation set
  const int set = a.n_sets > 1 ? (seg / a.set_div) % a.n_sets : 0;
  const float* set_pi = a.pi ? a.pi + (size_t)set * D * D : nullptr;
  const float* set_eps = a.eps ? a.eps + (size_t)set * D : nullptr;
  const float* set_s = a.s ? a.s + (size_t)set * a.m_rows * D : nullptr;
  const int row = 16 * wave + col;        // A-operand row of this lane
  static_assert(MAXG * 32 == PREP_THREADS, "one float4 of the query heads per thread");
  uint64_t prev = 0;
  if (cs && t == 0) prev = __hip_atomic_exchange(&cs->claim, ticket, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---- every global operand in flight together: the segment's query heads
  // once per workgroup (one float4 per thread, for the LDS), this lane's rows
  // of Pi and S ----
  float4 mv[8], sv[8];
  const int qh = t >> 5, q4 = t & 31;      // head, float4 within the head (16 x 32 = 512 threads)
  float4 qv = {0.f, 0.f, 0.f, 0.f};
  // column c of the products: head c % G of segment seg + c / G (ns G <= 16)
  if (qh < ns * G) qv = reinterpret_cast<const float4*>(a.q + ((size_t)seg * G + qh) * D)[q4];
  const float4* prow = reinterpret_cast<const float4*>(set_pi + (size_t)(HAD ? 0 : row) * D);
  // MSE-only keys have no QJL matrix: its rows read as zeros (q_proj = 0)
  // (with m = d / 2, rows from 64 on read as zeros)
  const bool srow_live = MW == 4 || row < 32 * MW;
  const float4* srow =
      reinterpret_cast<const float4*>(QJL ? set_s + (size_t)(MW == 4 ? row : srow_live ? row : 0) * D : set_pi);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int k4a = 8 * ks + 2 * kq, k4b = k4a + 1;      // coordinates 32 ks + 8 kq + 0..7
    if (HAD) {
      mv[2 * ks] = reinterpret_cast<const float4*>(set_eps)[k4a];
      mv[2 * ks + 1] = reinterpret_cast<const float4*>(set_eps)[k4b];
    } else {
      mv[2 * ks] = prow[k4a];
      mv[2 * ks + 1] = prow[k4b];
    }
    if constexpr (QJL && MW == 4) {
      sv[2 * ks] = srow[k4a];
      sv[2 * ks + 1] = srow[k4b];
    } else if constexpr (QJL) {
      sv[2 * ks] = srow_live ? srow[k4a] : float4{0.f, 0.f, 0.f, 0.f};
      sv[2 * ks + 1] = srow_live ? srow[k4b] : float4{0.f, 0.f, 0.f, 0.f};
    } else {
      sv[2 * ks] = sv[2 * ks + 1] = float4{0.f, 0.f, 0.f, 0.f};
    }
  }
  // keep all of them ahead of the first product (one memory round trip)
  __builtin_amdgcn_sched_barrier(0);
  // the query heads go to the q_proj rows of the LDS (free until the second
  // product; heads past G are zero)
  *reinterpret_cast<float4*>(&qp[qh * QTS + 4 * q4]) = qv;
  __syncthreads();

  // ---- q_rot^T = Pi . Q^T, rows 16 wave + 4 kq + r, head col ----
  {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int k0 = 32 * ks + 8 * kq;
      float av[8], bv[8];
      unpack8(mv[2 * ks], mv[2 * ks + 1], av);
      if (HAD) {
#pragma unroll
        for (int e = 0; e < 8; ++e) av[e] = (__popc(row & (k0 + e)) & 1) ? -av[e] : av[e];
      }
      const float4* qs = reinterpret_cast<const float4*>(&qp[col * QTS + k0]);
      unpack8(qs[0], qs[1], bv);
      bf16x8 ah, al, bh, bl;
      split8_bf16(av, ah, al);
      split8_bf16(bv, bh, bl);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
    }
    const float sc = HAD ? rsqrtf((float)D) : 1.f;
    float4 v = {acc[0] * sc, acc[1] * sc, acc[2] * sc, acc[3] * sc};
    *reinterpret_cast<float4*>(&qr[col * QTS + 16 * wave + 4 * kq]) = v;
    float mx = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    float sm = (v.x + v.y) + (v.z + v.w);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    sm += __shfl_xor(sm, 16, 64);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    sm += __shfl_xor(sm, 32, 64);
    if (kq == 0) {
      part[wave][col][0] = mx;
      part[wave][col][1] = sm;
    }
  }
  __syncthreads();
  // ---- q_proj^T = S . q_rot^T ----
  {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int k0 = 32 * ks + 8 * kq;
      float av[8], bv[8];
      unpack8(sv[2 * ks], sv[2 * ks + 1], av);
      const float4* src = reinterpret_cast<const float4*>(&qr[col * QTS + k0]);
      unpack8(src[0], src[1], bv);
      bf16x8 ah, al, bh, bl;
      split8_bf16(av, ah, al);
      split8_bf16(bv, bh, bl);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
    }
    float4 v = {acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<float4*>(&qp[col * QTS + 16 * wave + 4 * kq]) = v;
    float mx = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    float sm = (v.x + v.y) + (v.z + v.w);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    sm += __shfl_xor(sm, 16, 64);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    sm += __shfl_xor(sm, 32, 64);
    if (kq == 0) {
      part[wave][col][2] = mx;
      part[wave][col][3] = sm;
    }
  }
  __syncthreads();
  if (t < MAXG) {
    float mx = 0.f, sr = 0.f, px = 0.f, sp = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      mx = fmaxf(mx, part[w][t][0]);
      sr += part[w][t][1];
      px = fmaxf(px, part[w][t][2]);
      sp += part[w][t][3];
    }
    float umax = 0.f;
#pragma unroll
    for (int p = 0; p < 8; ++p) umax = p < np ? fmaxf(umax, fabsf(2.f * a.u[p])) : umax;
    const float mm = mx * umax, pm = 2.f * px;
    const float qmax = S == 2 ? QMAX2 : QMAX3;
    const float sm = mm > 0.f ? mm / qmax : 1.f, sq = pm > 0.f ? pm / qmax : 1.f;
    stat[t][0] = sm;
    stat[t][1] = -a.usum * sr;
    stat[t][2] = sq;
    stat[t][3] = -sp;
#pragma unroll
    for (int p = 0; p < 8; ++p) L.wsc[p][t] = 2.f * a.u[p] / sm;
    L.wsc[8][t] = 2.f / sq;
  }
  if (cs && t == 0) L.own = prev != ticket;
  __syncthreads();
  if (cs && !L.own) return false;
  if (cs && t == 0) __hip_atomic_store(&cs->done, ticket << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // ---- quantise: one item = (tile mt, fragment f = 2 p + m, lane group kg,
  // head hl of the tile) covers the 16 coordinates 32 kg + 8 bi + 4 m + k
  // (bi, k = 0..3), byte bi of dword k of the A operand of lanes
  // 16 kg + R hl + r, r = the digit (R rows per head; a fourth row stays zero) ----
  constexpr int R = S == 2 ? 2 : 4;             // A rows per head
  constexpr int HT = 16 / R;                    // heads per 16-row tile
  const int nitems = a.mt * F * 4 * HT;
  for (int j = 0; j < ns; ++j) {     // segment seg + j: its heads are columns j G ..
  const rsrc_t rdst = make_rsrc(dst + (size_t)j * pbytes, pbytes);
  for (int it = t; it < nitems; it += PREP_THREADS) {
    const int hl = it % HT, rest = it / HT;
    const int kg = rest & 3;
    const int f = (rest >> 2) % F, mt = (rest >> 2) / F;
    const int p = f >> 1, m = f & 1;
    const int h = HT * mt + hl;
    const bool live = h < G;
    const int hs = live ? j * G + h : 0;
    const float* src = (p < np ? qr : qp) + hs * QTS + 32 * kg + 4 * m;
    const float wsc = live ? L.wsc[p < np ? p : 8][hs] : 0.f;
    float4 v[4];
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) v[bi] = *reinterpret_cast<const float4*>(src + 8 * bi);
    uint32_t d0[4], d1[4], d2[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      int s0[4], s1[4], s2[4];
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        const float w = v[bi][k] * wsc;
        if constexpr (S == 2) {
          slices2(w, s0[bi], s1[bi]);
          s2[bi] = 0;
        } else {
          slices3(w, s0[bi], s1[bi], s2[bi]);
        }
      }
      d0[k] = pack4(s0[0], s0[1], s0[2], s0[3]);
      d1[k] = pack4(s1[0], s1[1], s1[2], s1[3]);
      d2[k] = pack4(s2[0], s2[1], s2[2], s2[3]);
    }
    const uint32_t ro = (uint32_t)(((mt * F + f) * 64 + 16 * kg + R * hl) * 16);
    __builtin_amdgcn_raw_buffer_store_b128(i32x4{(int)d0[0], (int)d0[1], (int)d0[2], (int)d0[3]}, rdst, ro, 0, CPOL);
    __builtin_amdgcn_raw_buffer_store_b128(i32x4{(int)d1[0], (int)d1[1], (int)d1[2], (int)d1[3]}, rdst, ro + 16, 0,
                                           CPOL);
    if constexpr (R == 4) {
      __builtin_amdgcn_raw_buffer_store_b128(i32x4{(int)d2[0], (int)d2[1], (int)d2[2], (int)d2[3]}, rdst, ro + 32,
                                             0, CPOL);
      __builtin_amdgcn_raw_buffer_store_b128(i32x4{0, 0, 0, 0}, rdst, ro + 48, 0, CPOL);
    }
  }
  if (t < a.mt * 16 / R * 4)
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, t < G * 4 ? stat[j * G + (t >> 2)][t & 3] : 0.f),
                                          rdst, (uint32_t)(fbytes + 4 * t), 0, CPOL);
  }
  return true;
}

// (at most two waves per SIMD: the register budget keeps every operand load
// of a lane in flight at once)
template <bool HAD, int S, bool QJL, int MW = 4>
__global__ __launch_bounds__(PREP_THREADS) __attribute__((amdgpu_waves_per_eu(1, 2)))
void prep_queries128(PrepArgs a) {
  __shared__ PrepLds L;
  const int F = 2 * (mse_planes(a.bq) + (QJL ? 1 : 0));
  const int seg0 = blockIdx.x * a.seg_per_wg;
  const int ns = a.segs - seg0 < a.seg_per_wg ? a.segs - seg0 : a.seg_per_wg;
  prep_pack<HAD, S, 0, QJL, MW>(a, seg0, ns, L, a.ws + (size_t)seg0 * pack_bytes(a.mt, F));
}

// One-launch scores: the first workgroup of each segment builds the query
// pack while the segment's other workgroups already have their first keys in
// flight.  Per segment three words in the workspace hand the pack over:
//   flag   the ticket of the launch whose pack is complete (a per-call odd
//          number from the host clock, so never the cleared value 0)
//   claim  the ticket of the launch whose pack has a builder: the one
//          workgroup whose exchange finds another value here builds the pack,
//          so exactly one workgroup writes it per launch
//   done   (ticket low 32 bits) << 32 | consumers of that launch done with
//          the pack: set to the tag with a zero count by the builder before it
//          publishes the flag, then one add per consumer at its end; the last
//          of the segment's active consumers clears all three words, so a
//          replayed launch (a captured graph keeps its ticket) finds them clear
// The producer issues its claim exchange with its operand loads and reads the
// answer only before its first pack store, so the exchange adds no round trip
// to its chain; the tagged zero count goes out with the pack stores, and one
// wait for all of them precedes the flag.  A consumer waits a bounded time for
// the flag (the producer may not be resident yet); if it has not come, it
// claims the pack itself and builds it, or, if another workgroup holds the
// claim (a running workgroup, which will publish), waits for the flag.  The
// pack and the words travel with device-coherent (sc1) accesses and relaxed
// device-scope atomics, each store waited for before the flag: no L2 writeback
// or invalidate is needed, since no other data is shared within the launch.
// The words may hold anything before a workspace's first call.  (ScoreSync,
// the four words of a segment, is defined above prep_pack, which takes the
// producer's claim.)

// Waits at most `ticks` of the 100 MHz constant clock (0: not at all; < 0:
// without bound).
__device__ __forceinline__ bool wait_ticket(uint64_t* flag, uint64_t ticket, long long ticks) {
  if (ticks == 0) return __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ticket;
  const long long t0 = wall_clock64();
  while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != ticket) {
    if (ticks > 0 && wall_clock64() - t0 > ticks) return false;
    __builtin_amdgcn_s_sleep(2);
  }
  return true;
}

// True for the one workgroup per launch and segment whose exchange takes the claim.
__device__ __forceinline__ bool take_claim(ScoreSync* s, uint64_t ticket) {
  return __hip_atomic_exchange(&s->claim, ticket, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != ticket;
}

// The builder, after its pack stores and before the flag: a zero count under
// this launch's tag, complete before anything else is stored.
__device__ __forceinline__ void publish(ScoreSync* s, uint64_t ticket) {
  __hip_atomic_store(&s->done, ticket << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);
  __hip_atomic_store(&s->flag, ticket, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);
}

// A consumer done with the pack; the last of `active` clears the words.
__device__ __forceinline__ void sync_done(ScoreSync* s, uint64_t ticket, uint32_t active) {
  const uint64_t old = __hip_atomic_fetch_add(&s->done, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if ((old >> 32) == (ticket & 0xffffffffull) && (uint32_t)old + 1u == active) {
    __hip_atomic_store(&s->flag, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&s->claim, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&s->done, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

struct Score128Args {
  const uint8_t* ws;            // query packs (prep_queries128)
  const uint32_t* planes;
  const uint16_t* scalars;
  int64_t seg_stride;
  const int32_t* len;
  int64_t T;
  int group;
  float kappa;
  float* scores;
  int chunk_tiles;   // 16-token tiles per workgroup
  // one-launch form only
  int chunks;        // consumer workgroups per segment
  PrepArgs prep;     // query side (prep.ws = the packs)
  ScoreSync* sync;   // [segs]
  uint64_t ticket;
  long long wait_ticks;   // consumers' bound on the wait for the pack
  int one_launch;         // keep the one-launch form for a long pass
};

__device__ __forceinline__ void expand8(uint32_t w, uint32_t e[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) e[k] = (w >> k) & 0x01010101u;
}

// Cache policy of the score stores: the sc1 (device-scope coherence) bit, which
// measured about 5% faster than the default write-back policy for the
// 19 MB of scores a decode step writes (less left dirty in L2 at kernel end).
constexpr int CPOL_SC1 = 16;

constexpr int SROW = 40;   // LDS row stride (floats) of the output transpose tile

__device__ __forceinline__ int combine3(i32x4 acc) {
  return (acc[0] * 256 + acc[1]) * 256 + acc[2];   // 65536 hi + 256 mid + lo
}
// The same in fp32, for accumulators of more than 256 digit terms (four MSE
// planes of 128 coordinates), whose 65536 hi would leave int32; the top digit
// is exact and the sum rounds once at 2^-24 relative.
__device__ __forceinline__ float combine3f(i32x4 acc) {
  return fmaf((float)acc[0], 65536.f, fmaf((float)acc[1], 256.f, (float)acc[2]));
}
// Recombined MSE accumulator of NP planes (three digits).
template <int NP>
__device__ __forceinline__ float mse_digits(i32x4 acc) {
  if constexpr (NP > 2) return combine3f(acc);
  else return (float)combine3(acc);
}

// m = d / 2 records: for the lanes of coordinate groups 2 and 3 (late),
// words loaded one early -> index words in slots 0 .. P-2, the early word in
// the sign slot P-1.
template <int P, typename W>
__device__ __forceinline__ W rotate_late_groups(W w, bool late) {
  W r;
#pragma unroll
  for (int i = 0; i < P; ++i) r[i] = late ? w[(i + 1) % P] : w[i];
  return r;
}

// Word of Walsh plane p (plane_subset order) of an MSE-only key record: a
// single index bit, or the parity of the subset's bits.  (The prod kernels
// spell the same selection out inline, QJL signs at p == NP.)
template <int BQ, int NP, bool QJL, typename W>
__device__ __forceinline__ uint32_t plane_word(W w, int p) {
  static_assert(!QJL, "prod records select their words inline");
  if (p < BQ) return w[p];
  if constexpr (BQ == 3) return w[0] ^ w[1] ^ w[2];
  if constexpr (BQ == 4) {
    const uint32_t all = w[0] ^ w[1] ^ w[2] ^ w[3];
    return all ^ w[p == 4 ? 3 : p == 5 ? 2 : p == 6 ? 1 : 0];   // subsets 7, 11, 13, 14
  }
  return 0u;
}

// Workgroup = 8 waves = chunk_tiles 16-token tiles of one segment.  A wave
// takes pairs of adjacent tiles (32 tokens), pairs wave, wave + 8, ...,
// with RING pairs of loads in flight; the 32 x 8 outputs of a 16-row tile
// pass through a per-wave LDS tile so that each lane stores 4 consecutive
// tokens of one head (16 bytes) and a store covers whole 128-byte lines.
constexpr int SC_WAVES = 8;     // waves per workgroup of the one-launch form (and of short passes)
constexpr int PASS_WAVES = 4;   // waves per workgroup of a long score pass

// FUSED: the one-launch form (1-D grid: segs producers, then segs x chunks
// consumers); HAD selects the producer's rotation.  QJL: prod keys (BQ index
// planes, the sign plane, n and gamma); without it MSE-only keys (BQ index
// planes and n).
// MW: QJL sign words per record (m / 32).  With MW = 2 (m = d / 2) the record
// has no sign word in coordinate groups 2 and 3: their lanes load the P words
// that end with the group's last index word (the first is the previous
// group's last word) and rotate them into place; the sign slot then holds
// that foreign word, and the pack's QJL weights for these groups are zero.
template <int BQ, int MT, int S, bool FUSED, bool HAD, bool QJL, int MW = 4, int NWV = SC_WAVES>
__global__ __launch_bounds__(NWV * 64) __attribute__((amdgpu_waves_per_eu(FUSED && MT == 1 ? 4 : 1)))
void scores128(Score128Args a) {
  static_assert(!FUSED || NWV == SC_WAVES, "the one-launch producers build the pack with 8 waves");
  constexpr int NP = mse_planes(BQ);      // Walsh planes of the index bits
  constexpr int F = 2 * (NP + QJL);       // MFMAs per tile per 16-row tile
  constexpr int P = BQ + QJL;             // planes per coordinate group (words a lane loads)
  constexpr int SB = QJL ? 4 : 2;         // scalar bytes per key record
  constexpr uint32_t RB = MW == 4 ? 16 * P : 4 * (4 * BQ + MW);   // plane bytes per key record
  constexpr int RING = 4;                 // pairs of loads in flight per wave
  constexpr int ROUND = 8;                // pairs per straight-line round
  constexpr int HL = S == 2 ? 2 : 1;      // heads per lane group per 16-row tile
  constexpr int NH = MT * 4 * HL;         // heads covered by the tiles
  typedef typename Words<P>::v wvec;
  constexpr int SBUF = NWV * NH * SROW;                    // floats of the output tiles
  constexpr int PREPF = (int)((sizeof(PrepLds) + 15) / 16 * 4);   // floats of the producer's scratch
  constexpr int PACKF = (int)(pack_bytes(MT, F) / 4);                  // floats of one query pack
  constexpr int SMEM0 = FUSED && PREPF > SBUF ? PREPF : SBUF;
  constexpr int SMEM = FUSED && PACKF > SMEM0 ? PACKF : SMEM0;
  __shared__ __align__(16) float smem[SMEM + (FUSED ? 4 : 0)];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t16 = lane & 15;
  const int kg = lane >> 4;
  int seg, chunk;
  // consumers with tokens to score (the ones that count themselves done)
  auto active_chunks = [&](int sg) -> uint32_t {
    const int64_t l = a.len ? (int64_t)a.len[sg] : a.T;
    const int64_t span = (int64_t)a.chunk_tiles * 16;
    return l > 0 ? (uint32_t)((l + span - 1) / span) : 0u;
  };
  if constexpr (FUSED) {
    const int b = blockIdx.x;
    if (b < a.prep.segs) {
      // producer of segment b (none needed when it has no tokens): unless a
      // consumer that gave up waiting holds the claim, the pack with
      // device-coherent stores, every store complete, then the flag
      if (active_chunks(b) == 0) return;
      if (prep_pack<HAD, S, CPOL_SC1, QJL, MW>(a.prep, b, 1, *reinterpret_cast<PrepLds*>(smem),
                                               a.prep.ws + (size_t)b * pack_bytes(MT, F), &a.sync[b], a.ticket)) {
        // the pack and the tagged count complete, then the flag
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0)
          __hip_atomic_store(&a.sync[b].flag, a.ticket, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      return;
    }
    seg = (b - a.prep.segs) / a.chunks;
    chunk = (b - a.prep.segs) % a.chunks;
  } else {
    seg = blockIdx.y;
    chunk = blockIdx.x;
  }
  const int64_t len = a.len ? (int64_t)a.len[seg] : a.T;
  const int64_t tok0 = (int64_t)chunk * a.chunk_tiles * 16;
  if (tok0 >= len) return;

  const int64_t rec0 = seg * a.seg_stride + tok0;
  const rsrc_t rk = make_rsrc(a.planes + rec0 * (RB / 4), clamp_bytes((a.seg_stride - tok0) * RB));
  const rsrc_t rs = make_rsrc(a.scalars + rec0 * (SB / 2), clamp_bytes((a.seg_stride - tok0) * SB));
  const rsrc_t ro = make_rsrc(a.scores + (size_t)seg * a.group * a.T + tok0,
                              clamp_bytes(((int64_t)(a.group - 1) * a.T + a.T - tok0) * 4));
  const uint32_t vk = t16 * RB + (MW == 4 ? kg * (P * 4) : (kg < 2 ? kg * P : kg * BQ + 1) * 4);
  const uint32_t vs = t16 * SB;
  const int ntok = (int)(len - tok0 < (int64_t)a.chunk_tiles * 16 ? len - tok0 : (int64_t)a.chunk_tiles * 16);
  const int npairs = (ntok + 31) / 32;

  wvec wr[RING][2];
  uint32_t sr[RING][2];
  // pairs past this workgroup's span get the out-of-range offset: zeros, and
  // no memory traffic (no over-read of the next span); the keys are read once,
  // so their loads are non-temporal (on a cache larger than the memory-side
  // cache this took the pass from 103 to 93-95 us)
  auto load_pair = [&](int slot, int pr) {
    const bool ok = pr < npairs;
    const uint32_t tb = (uint32_t)(32 * pr);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      wr[slot][h] = load_words<P, CPOL_NT>(rk, ok ? vk + (tb + 16 * h) * RB : OOB_OFFSET);
      if constexpr (QJL)
        sr[slot][h] = __builtin_amdgcn_raw_buffer_load_b32(rs, ok ? vs + (tb + 16 * h) * 4 : OOB_OFFSET, 0, CPOL_NT);
      else
        sr[slot][h] = __builtin_amdgcn_raw_buffer_load_b16(rs, ok ? vs + (tb + 16 * h) * 2 : OOB_OFFSET, 0, CPOL_NT);
    }
  };
  const uint8_t* pack = a.ws + (size_t)seg * pack_bytes(MT, F);
  const int mine = npairs > wave ? (npairs - wave + NWV - 1) / NWV : 0;
  // the first round's keys go out before the pack is read (pairs past the
  // span read zeros without memory traffic)
#pragma unroll
  for (int j = 0; j < RING; ++j) load_pair(j, wave + NWV * j);
  if constexpr (FUSED) {
    // 0: the pack is published; 1: this workgroup holds the claim and builds it
    int* build = reinterpret_cast<int*>(smem + SMEM);
    if (threadIdx.x == 0) {
      int bld = 0;
      if (!wait_ticket(&a.sync[seg].flag, a.ticket, a.wait_ticks)) {
        if (take_claim(&a.sync[seg], a.ticket))
          bld = 1;
        else
          wait_ticket(&a.sync[seg].flag, a.ticket, -1);   // the claimant is running and will publish
      }
      *build = bld;
    }
    __syncthreads();
    if (*build) {
      // the producer has not started: build the pack here (the only writer
      // of this launch), publish it, then request the first keys again
      prep_pack<HAD, S, CPOL_SC1, QJL, MW>(a.prep, seg, 1, *reinterpret_cast<PrepLds*>(smem),
                                           const_cast<uint8_t*>(pack));
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (threadIdx.x == 0) publish(&a.sync[seg], a.ticket);
#pragma unroll
      for (int j = 0; j < RING; ++j) load_pair(j, wave + NWV * j);
    }
  }

  // the pack: in the one-launch form it was written in this launch, possibly
  // through another XCD's L2, so the workgroup reads it once with
  // device-coherent loads into the LDS and the waves take their fragments
  // from there; otherwise each wave reads its fragments (L2 hits)
  const rsrc_t rp = make_rsrc(pack, (uint32_t)pack_bytes(MT, F));
  const uint8_t* lpack = reinterpret_cast<const uint8_t*>(smem);
  if constexpr (FUSED) {
    for (int u = threadIdx.x; u < PACKF / 4; u += NWV * 64)
      reinterpret_cast<i32x4*>(smem)[u] =
          __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, (uint32_t)(16 * u), 0, CPOL_SC1));
    __syncthreads();
  }
  i32x4 afr[MT][F];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const uint32_t off = (uint32_t)(((mt * F + f) * 64 + lane) * 16);
      if constexpr (FUSED)
        afr[mt][f] = *reinterpret_cast<const i32x4*>(lpack + off);
      else
        afr[mt][f] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, off, 0, 0));
    }
  // head 4 HL mt + HL kg + hh: sigma_mse, const_mse, kappa sigma_qjl, kappa const_qjl
  float cst[MT][HL][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int hh = 0; hh < HL; ++hh) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t off = (uint32_t)(pack_frag_bytes(MT, F) + ((4 * HL * mt + HL * kg + hh) * 4 + c) * 4);
        if constexpr (FUSED)
          cst[mt][hh][c] = *reinterpret_cast<const float*>(lpack + off);
        else
          cst[mt][hh][c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rp, off, 0, 0));
      }
      cst[mt][hh][2] *= a.kappa;
      cst[mt][hh][3] *= a.kappa;
    }
  if constexpr (FUSED) __syncthreads();   // every wave has its fragments: the LDS turns into output tiles
  float* sbuf = smem + wave * (NH * SROW);

  // one 16-token tile -> LDS rows (heads 4 mt + kg), columns col0 + t16
  auto compute = [&](wvec w, uint32_t scl, int col0) {
    if constexpr (MW == 2) w = rotate_late_groups<P>(w, kg >= 2);
    i32x4 am[MT], aq[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) am[mt] = aq[mt] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p < NP + QJL; ++p) {
      uint32_t word;
      if constexpr (QJL) {
        if (p == NP) {
          word = w[QJL ? BQ : 0];                        // QJL signs
        } else if (p < BQ) {
          word = w[p];                                   // single index bits
        } else {
          if constexpr (BQ == 3) word = w[0] ^ w[1] ^ w[2];   // parity of 3 bits
        }
      } else {
        word = plane_word<BQ, NP, false>(w, p);
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
    const float g = (float)__builtin_bit_cast(_Float16, (uint16_t)(scl >> 16));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int hh = 0; hh < HL; ++hh) {
        const float im = S == 2 ? (float)(am[mt][2 * hh] * 256 + am[mt][2 * hh + 1]) : mse_digits<NP>(am[mt]);
        const int iq = S == 2 ? aq[mt][2 * hh] * 256 + aq[mt][2 * hh + 1] : combine3(aq[mt]);
        const float mse = fmaf(im, cst[mt][hh][0], cst[mt][hh][1]);
        const float qjl = fmaf((float)iq, cst[mt][hh][2], cst[mt][hh][3]);
        sbuf[(4 * HL * mt + HL * kg + hh) * SROW + col0 + t16] = QJL ? n * fmaf(g, qjl, mse) : n * mse;
      }
    }
  };
  // lanes 8 h' + c store tokens 4c .. 4c+3 of head 8 r + h' of the pair;
  // padded heads and tokens past ntok get an offset past the descriptor
  const int hr = lane >> 3, c4 = 4 * (lane & 7);
  auto flush = [&](int pbase) {
    const bool full = pbase + 32 <= ntok;
#pragma unroll
    for (int rr = 0; rr < (NH + 7) / 8; ++rr) {
      const int head = rr * 8 + hr;
      const int hread = head < NH ? head : 0;
      const float4 v = *reinterpret_cast<const float4*>(&sbuf[hread * SROW + c4]);
      const uint32_t vo = (uint32_t)(head * a.T + pbase + c4) * 4u;
      const bool live = head < a.group;
      if (full) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), ro, live ? vo : OOB_OFFSET, 0, CPOL_SC1);
      } else {
        const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t o = live && pbase + c4 + e < ntok ? vo + 4 * e : OOB_OFFSET;
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, vv[e]), ro, o, 0, CPOL_SC1);
        }
      }
    }
  };

  // rounds of ROUND pairs per wave, straight-line inside a round: loads run
  // RING pairs ahead and never across a round boundary, so every wait on a
  // slot counts exactly the loads issued after it
  for (int r0 = 0; r0 < mine; r0 += ROUND) {
    if (r0 > 0) {
#pragma unroll
      for (int j = 0; j < RING; ++j) load_pair(j, wave + NWV * (r0 + j));
    }
#pragma unroll
    for (int j = 0; j < ROUND; ++j) {
      if (r0 + j >= mine) break;
      const int pr = wave + NWV * (r0 + j);
      compute(wr[j % RING][0], sr[j % RING][0], 0);
      compute(wr[j % RING][1], sr[j % RING][1], 16);
      if (j + RING < ROUND) load_pair(j % RING, pr + NWV * RING);
      flush(32 * pr);
    }
  }
  // done with the pack (read into the LDS at the start): count this consumer
  if constexpr (FUSED)
    if (threadIdx.x == 0) sync_done(&a.sync[seg], a.ticket, active_chunks(seg));
}

int device_cus();
int occupancy(const void* kernel, int threads);
int64_t split_span(int segs, int64_t T, int resident, int64_t gran, int64_t kmax);

// Workgroups of the score pass: enough to fill the device once, and more when
// a segment is long, so that no workgroup takes more than one straight-line
// round of its waves (pspan tokens: 8 pairs of 32 tokens per wave).  Many
// short workgroups keep every channel busy to the end of the pass: at 32
// layers x 8 heads x 32768 tokens, 16 8-wave workgroups per segment ran 14%
// faster than the 2 that fill the device once.
constexpr int64_t PASS_SPAN = (int64_t)SC_WAVES * 8 * 32;   // 8 waves x 8 pairs x 32 tokens
int pass_workgroups(int resident, int segs, int64_t T, int64_t pspan = PASS_SPAN) {
  const int64_t by_len = (int64_t)segs * ((T + pspan - 1) / pspan);
  return (int)std::min<int64_t>(std::max<int64_t>(resident, by_len), 1ll << 30);
}

// Grid: (workgroups per segment, segments); a workgroup's span is a multiple
// of its waves x 32 tokens.  A pass that takes more than one dispatch of
// 8-wave workgroups runs 4-wave workgroups with the same work per wave: at 92
// VGPRs a SIMD holds 5 waves, of which 8-wave workgroups use 4 (32 layers x 8
// heads x 32768 tokens: 87-89 us against 93-95 us); a shorter pass keeps the
// 8-wave form, whose workgroups fill the device once with longer spans
// (72 segments x 8192 tokens: 11.6 us against 12.3 us).
template <int BQ, int MT, int S, bool QJL, int MW, int NW>
hipError_t launch_scores_waves(Score128Args& s, int segs, hipStream_t stream) {
  static const int nb =
      occupancy(reinterpret_cast<const void*>(&scores128<BQ, MT, S, false, false, QJL, MW, NW>), NW * 64);
  const int64_t span = split_span(segs, s.T, pass_workgroups(nb * device_cus(), segs, s.T, (int64_t)NW * 8 * 32),
                                  32 * NW, (s.T + 255) / 256);
  s.chunk_tiles = (int)(span / 16);
  const int64_t chunks = (s.T + span - 1) / span;
  hipLaunchKernelGGL((scores128<BQ, MT, S, false, false, QJL, MW, NW>), dim3((unsigned)chunks, (unsigned)segs),
                     dim3(NW * 64), 0, stream, s);
  return hipGetLastError();
}

// Segments per query-prep workgroup: one while the segments fit one workgroup
// per compute unit (more compute units at work: 256 segments of 4 heads,
// 98.2 us per call against 99.1-99.5 us); beyond that, consecutive segments
// that share a rotation set fill the products' 16 head columns together (one
// read of Pi and S per workgroup: 512 segments of 4 heads, a 149.6 us batched
// step against 152.2 us).
int prep_segments_per_workgroup(int n_sets, int group, int segs) {
  if (n_sets > 1 || segs <= device_cus()) return 1;
  return MAXG / (group > 0 ? group : 1);
}

// True when the pass takes more than one dispatch of 8-wave workgroups.
template <int BQ, int MT, int S, bool QJL, int MW>
bool long_pass(int segs, int64_t T) {
  static const int nb8 =
      occupancy(reinterpret_cast<const void*>(&scores128<BQ, MT, S, false, false, QJL, MW, SC_WAVES>), SC_WAVES * 64);
  const int64_t by_len = (int64_t)segs * ((T + PASS_SPAN - 1) / PASS_SPAN);
  return by_len > (int64_t)nb8 * device_cus();
}

template <int BQ, int MT, int S, bool QJL = true, int MW = 4>
hipError_t launch_scores(Score128Args& s, int segs, hipStream_t stream) {
  if (long_pass<BQ, MT, S, QJL, MW>(segs, s.T)) return launch_scores_waves<BQ, MT, S, QJL, MW, PASS_WAVES>(s, segs, stream);
  return launch_scores_waves<BQ, MT, S, QJL, MW, SC_WAVES>(s, segs, stream);
}

// One-launch form: the producers take one resident slot per segment, the
// consumers split the tokens over the rest.
// A long pass runs as two launches instead, the query packs and then the
// pass: its 4-wave pass kernel outruns the one-launch form by more than the
// packs' own launch costs (32 layers x 8 heads x 32768 tokens: 97-99 us
// against 106-108 us per call), while a short pass keeps the one launch.
template <int BQ, int MT, int S, bool HAD, bool QJL = true, int MW = 4>
hipError_t launch_scores_fused(Score128Args& s, int segs, hipStream_t stream) {
  if (!s.one_launch && long_pass<BQ, MT, S, QJL, MW>(segs, s.T)) {
    PrepArgs p = s.prep;
    p.seg_per_wg = prep_segments_per_workgroup(p.n_sets, p.group, segs);
    hipLaunchKernelGGL((prep_queries128<HAD, S, QJL, MW>), dim3((unsigned)((segs + p.seg_per_wg - 1) / p.seg_per_wg)),
                       dim3(PREP_THREADS), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_scores<BQ, MT, S, QJL, MW>(s, segs, stream);
  }
  static const int nb =
      occupancy(reinterpret_cast<const void*>(&scores128<BQ, MT, S, true, HAD, QJL, MW>), SC_WAVES * 64);
  const int resident = nb * device_cus() - segs;
  const int64_t span = split_span(segs, s.T, pass_workgroups(resident > segs ? resident : segs, segs, s.T),
                                  32 * SC_WAVES, (s.T + 255) / 256);
  s.chunk_tiles = (int)(span / 16);
  s.chunks = (int)((s.T + span - 1) / span);
  const int64_t nwg = (int64_t)segs * (s.chunks + 1);
  hipLaunchKernelGGL((scores128<BQ, MT, S, true, HAD, QJL, MW>), dim3((unsigned)nwg), dim3(SC_WAVES * 64), 0, stream,
                     s);
  return hipGetLastError();
}

}  // namespace

void walsh_coefficients(const Codebook& cb, int bq, float u[8], float* usum) {
  // u_S = 2^-bq sum_idx c[idx] prod_{p in S} (2 bit_p(idx) - 1), odd S in the plane order
  const int K = 1 << bq;
  const int ns = mse_planes(bq);
  double tot = 0;
  for (int s = 0; s < 8; ++s) u[s] = 0.f;
  for (int s = 0; s < ns; ++s) {
    const int sub = plane_subset(bq, s);
    double acc = 0;
    for (int idx = 0; idx < K; ++idx) {
      double chi = 1;
      for (int p = 0; p < bq; ++p)
        if (sub >> p & 1) chi *= ((idx >> p) & 1) ? 1.0 : -1.0;
      acc += cb.c[idx] * chi;
    }
    u[s] = (float)(acc / K);
    tot += acc / K;
  }
  *usum = (float)tot;
}

namespace {

// Compute units of the current device (cached per device).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// Resident workgroups per compute unit of a kernel at the given block size.
int occupancy(const void* kernel, int threads) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, threads, 0) != hipSuccess || nb <= 0) nb = 1;
  return nb;
}

// Split each segment's T tokens over k workgroups so that segs * k fills the
// device once: span = tokens per workgroup, a multiple of gran.
int64_t split_span(int segs, int64_t T, int resident, int64_t gran, int64_t kmax) {
  int64_t k = resident / (segs > 0 ? segs : 1);
  if (k < 1) k = 1;
  if (k > kmax) k = kmax;
  const int64_t per = (T + k - 1) / k;
  int64_t span = (per + gran - 1) / gran * gran;
  return span < gran ? gran : span;
}

}  // namespace

// Query packs of every segment, sized for the widest pack (4 heads per
// 16-row tile, 16 fragments: MSE-only 4-bit keys in the attention pass; prod
// keys take at most 10), then the one-launch hand-over words.
static size_t scores128_pack_region(int segs, int group) {
  const int mt = (group + 3) / 4;
  return (size_t)segs * pack_bytes(mt, 2 * mse_planes(4));
}

size_t scores128_workspace(int segs, int group) {
  return scores128_pack_region(segs, group) + ((size_t)segs * sizeof(ScoreSync) + 255) / 256 * 256;
}

// ---------------------------------------------------------------------------
// tq_scores_noalloc: tq_scores with its workspace in a device array of this
// library instead of caller memory, for callers that cannot allocate (code
// under graph capture, tight serving loops).  The array is file-scope device
// memory, one copy per GPU, held until the process ends.  Host code never
// uses its name as an address: the device address is resolved once per device
// with hipGetSymbolAddress and kept.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[SCORES_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES];
}  // namespace

hipError_t scores_scratch(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  *bytes = SCORES_SCRATCH_BYTES;
  return hipSuccess;
}

// Per-call tickets of the one-launch form: odd (never the cleared value 0)
// and distinct from call to call, from the host's monotonic clock in
// nanoseconds (consecutive calls on one workspace are far more than a
// nanosecond apart).  No state is kept between calls.
static uint64_t call_ticket() {
  return (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() * 2 + 1;
}

// Digits per quantised query weight for the score pass: 2 for MSE-only keys
// and for prod keys with 1 or 2 MSE bits, else 3 (the attention pass always
// takes 3).
static int score_slices(const ScoreArgs& a) { return !a.qjl || a.bq <= 2 ? 2 : 3; }

static PrepArgs make_prep(const ScoreArgs& a, int slices) {
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
  p.n_sets = a.n_sets > 1 ? a.n_sets : 1;
  p.set_div = a.set_div > 1 ? a.set_div : 1;
  p.m_rows = a.qjl ? a.m : 0;
  walsh_coefficients(a.cb, a.bq, p.u, &p.usum);
  p.bq = a.bq;
  p.slices = slices;
  p.mt = slices == 2 ? (a.group + 7) / 8 : (a.group + 3) / 4;
  p.ws = static_cast<uint8_t*>(a.ws);
  p.seg_per_wg = 1;
  return p;
}

hipError_t launch_scores128_prep(const ScoreArgs& a, int slices, hipStream_t stream) {
  PrepArgs p = make_prep(a, slices);
  p.seg_per_wg = prep_segments_per_workgroup(p.n_sets, a.group, a.segs);
  const bool had = a.rot == TQ_ROT_HADAMARD;
  const dim3 grid((a.segs + p.seg_per_wg - 1) / p.seg_per_wg), block(PREP_THREADS);
  if (a.qjl && a.m == D / 2) {
    switch ((slices == 2 ? 0 : 2) + (had ? 1 : 0)) {
      case 0: hipLaunchKernelGGL((prep_queries128<false, 2, true, 2>), grid, block, 0, stream, p); break;
      case 1: hipLaunchKernelGGL((prep_queries128<true, 2, true, 2>), grid, block, 0, stream, p); break;
      case 2: hipLaunchKernelGGL((prep_queries128<false, 3, true, 2>), grid, block, 0, stream, p); break;
      case 3: hipLaunchKernelGGL((prep_queries128<true, 3, true, 2>), grid, block, 0, stream, p); break;
    }
    return hipGetLastError();
  }
  switch ((slices == 2 ? 0 : 4) + (had ? 2 : 0) + (a.qjl ? 1 : 0)) {
    case 0: hipLaunchKernelGGL((prep_queries128<false, 2, false>), grid, block, 0, stream, p); break;
    case 1: hipLaunchKernelGGL((prep_queries128<false, 2, true>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((prep_queries128<true, 2, false>), grid, block, 0, stream, p); break;
    case 3: hipLaunchKernelGGL((prep_queries128<true, 2, true>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((prep_queries128<false, 3, false>), grid, block, 0, stream, p); break;
    case 5: hipLaunchKernelGGL((prep_queries128<false, 3, true>), grid, block, 0, stream, p); break;
    case 6: hipLaunchKernelGGL((prep_queries128<true, 3, false>), grid, block, 0, stream, p); break;
    case 7: hipLaunchKernelGGL((prep_queries128<true, 3, true>), grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

static Score128Args score_pass_args(const ScoreArgs& a) {
  Score128Args s = {};
  s.ws = static_cast<const uint8_t*>(a.ws);
  s.planes = a.planes;
  s.scalars = a.scalars;
  s.seg_stride = a.seg_stride;
  s.len = a.len;
  s.T = a.T;
  s.group = a.group;
  s.kappa = (float)(std::sqrt(M_PI / 2.0) / (a.qjl ? a.m : D));
  s.scores = a.scores;
  s.chunk_tiles = 0;   // set by the launcher
  return s;
}

hipError_t launch_scores128(const ScoreArgs& a, hipStream_t stream) {
  const int slices = score_slices(a);
  const int mt = slices == 2 ? (a.group + 7) / 8 : (a.group + 3) / 4;
  Score128Args s = score_pass_args(a);
  s.prep = make_prep(a, slices);
  s.sync = reinterpret_cast<ScoreSync*>(static_cast<uint8_t*>(a.ws) + scores128_pack_region(a.segs, a.group));
  s.ticket = call_ticket();
  s.wait_ticks = 100LL * (a.wait_us < 0 ? 0 : a.wait_us);   // 100 MHz clock
  s.one_launch = a.one_launch;
  const bool had = a.rot == TQ_ROT_HADAMARD;
  if (a.qjl && a.m == D / 2) {
    // prod keys with m = d / 2 QJL rows
    switch (a.bq * 100 + mt * 10 + (had ? 1 : 0)) {
      case 110: return launch_scores_fused<1, 1, 2, false, true, 2>(s, a.segs, stream);
      case 111: return launch_scores_fused<1, 1, 2, true, true, 2>(s, a.segs, stream);
      case 120: return launch_scores_fused<1, 2, 2, false, true, 2>(s, a.segs, stream);
      case 121: return launch_scores_fused<1, 2, 2, true, true, 2>(s, a.segs, stream);
      case 210: return launch_scores_fused<2, 1, 2, false, true, 2>(s, a.segs, stream);
      case 211: return launch_scores_fused<2, 1, 2, true, true, 2>(s, a.segs, stream);
      case 220: return launch_scores_fused<2, 2, 2, false, true, 2>(s, a.segs, stream);
      case 221: return launch_scores_fused<2, 2, 2, true, true, 2>(s, a.segs, stream);
      case 310: return launch_scores_fused<3, 1, 3, false, true, 2>(s, a.segs, stream);
      case 311: return launch_scores_fused<3, 1, 3, true, true, 2>(s, a.segs, stream);
      case 320: return launch_scores_fused<3, 2, 3, false, true, 2>(s, a.segs, stream);
      case 321: return launch_scores_fused<3, 2, 3, true, true, 2>(s, a.segs, stream);
      case 330: return launch_scores_fused<3, 3, 3, false, true, 2>(s, a.segs, stream);
      case 331: return launch_scores_fused<3, 3, 3, true, true, 2>(s, a.segs, stream);
      case 340: return launch_scores_fused<3, 4, 3, false, true, 2>(s, a.segs, stream);
      case 341: return launch_scores_fused<3, 4, 3, true, true, 2>(s, a.segs, stream);
    }
    return hipErrorInvalidValue;
  }
  if (!a.qjl) {
    switch (a.bq * 100 + mt * 10 + (had ? 1 : 0)) {
      case 110: return launch_scores_fused<1, 1, 2, false, false>(s, a.segs, stream);
      case 111: return launch_scores_fused<1, 1, 2, true, false>(s, a.segs, stream);
      case 120: return launch_scores_fused<1, 2, 2, false, false>(s, a.segs, stream);
      case 121: return launch_scores_fused<1, 2, 2, true, false>(s, a.segs, stream);
      case 210: return launch_scores_fused<2, 1, 2, false, false>(s, a.segs, stream);
      case 211: return launch_scores_fused<2, 1, 2, true, false>(s, a.segs, stream);
      case 220: return launch_scores_fused<2, 2, 2, false, false>(s, a.segs, stream);
      case 221: return launch_scores_fused<2, 2, 2, true, false>(s, a.segs, stream);
      case 310: return launch_scores_fused<3, 1, 2, false, false>(s, a.segs, stream);
      case 311: return launch_scores_fused<3, 1, 2, true, false>(s, a.segs, stream);
      case 320: return launch_scores_fused<3, 2, 2, false, false>(s, a.segs, stream);
      case 321: return launch_scores_fused<3, 2, 2, true, false>(s, a.segs, stream);
      case 410: return launch_scores_fused<4, 1, 2, false, false>(s, a.segs, stream);
      case 411: return launch_scores_fused<4, 1, 2, true, false>(s, a.segs, stream);
      case 420: return launch_scores_fused<4, 2, 2, false, false>(s, a.segs, stream);
      case 421: return launch_scores_fused<4, 2, 2, true, false>(s, a.segs, stream);
    }
    return hipErrorInvalidValue;
  }
  switch (a.bq * 100 + mt * 10 + (had ? 1 : 0)) {
    case 110: return launch_scores_fused<1, 1, 2, false>(s, a.segs, stream);
    case 111: return launch_scores_fused<1, 1, 2, true>(s, a.segs, stream);
    case 120: return launch_scores_fused<1, 2, 2, false>(s, a.segs, stream);
    case 121: return launch_scores_fused<1, 2, 2, true>(s, a.segs, stream);
    case 210: return launch_scores_fused<2, 1, 2, false>(s, a.segs, stream);
    case 211: return launch_scores_fused<2, 1, 2, true>(s, a.segs, stream);
    case 220: return launch_scores_fused<2, 2, 2, false>(s, a.segs, stream);
    case 221: return launch_scores_fused<2, 2, 2, true>(s, a.segs, stream);
    case 310: return launch_scores_fused<3, 1, 3, false>(s, a.segs, stream);
    case 311: return launch_scores_fused<3, 1, 3, true>(s, a.segs, stream);
    case 320: return launch_scores_fused<3, 2, 3, false>(s, a.segs, stream);
    case 321: return launch_scores_fused<3, 2, 3, true>(s, a.segs, stream);
    case 330: return launch_scores_fused<3, 3, 3, false>(s, a.segs, stream);
    case 331: return launch_scores_fused<3, 3, 3, true>(s, a.segs, stream);
    case 340: return launch_scores_fused<3, 4, 3, false>(s, a.segs, stream);
    case 341: return launch_scores_fused<3, 4, 3, true>(s, a.segs, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_scores128_prepare(const ScoreArgs& a, hipStream_t stream) {
  return launch_scores128_prep(a, score_slices(a), stream);
}

hipError_t launch_scores128_prepared(const ScoreArgs& a, hipStream_t stream) {
  const int slices = score_slices(a);
  const int mt = slices == 2 ? (a.group + 7) / 8 : (a.group + 3) / 4;
  Score128Args s = score_pass_args(a);
  if (a.qjl && a.m == D / 2) {
    switch (a.bq * 10 + mt) {
      case 11: return launch_scores<1, 1, 2, true, 2>(s, a.segs, stream);
      case 12: return launch_scores<1, 2, 2, true, 2>(s, a.segs, stream);
      case 21: return launch_scores<2, 1, 2, true, 2>(s, a.segs, stream);
      case 22: return launch_scores<2, 2, 2, true, 2>(s, a.segs, stream);
      case 31: return launch_scores<3, 1, 3, true, 2>(s, a.segs, stream);
      case 32: return launch_scores<3, 2, 3, true, 2>(s, a.segs, stream);
      case 33: return launch_scores<3, 3, 3, true, 2>(s, a.segs, stream);
      case 34: return launch_scores<3, 4, 3, true, 2>(s, a.segs, stream);
    }
    return hipErrorInvalidValue;
  }
  if (!a.qjl) {
    switch (a.bq * 10 + mt) {
      case 11: return launch_scores<1, 1, 2, false>(s, a.segs, stream);
      case 12: return launch_scores<1, 2, 2, false>(s, a.segs, stream);
      case 21: return launch_scores<2, 1, 2, false>(s, a.segs, stream);
      case 22: return launch_scores<2, 2, 2, false>(s, a.segs, stream);
      case 31: return launch_scores<3, 1, 2, false>(s, a.segs, stream);
      case 32: return launch_scores<3, 2, 2, false>(s, a.segs, stream);
      case 41: return launch_scores<4, 1, 2, false>(s, a.segs, stream);
      case 42: return launch_scores<4, 2, 2, false>(s, a.segs, stream);
    }
    return hipErrorInvalidValue;
  }
  switch (a.bq * 10 + mt) {
    case 11: return launch_scores<1, 1, 2>(s, a.segs, stream);
    case 12: return launch_scores<1, 2, 2>(s, a.segs, stream);
    case 21: return launch_scores<2, 1, 2>(s, a.segs, stream);
    case 22: return launch_scores<2, 2, 2>(s, a.segs, stream);
    case 31: return launch_scores<3, 1, 3>(s, a.segs, stream);
    case 32: return launch_scores<3, 2, 3>(s, a.segs, stream);
    case 33: return launch_scores<3, 3, 3>(s, a.segs, stream);
    case 34: return launch_scores<3, 4, 3>(s, a.segs, stream);
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
// P'_t = p_t n_v,t, a contraction over tokens: A = P' (two base-256 int8
// digits per head, 16 bits relative to the group maximum: a weight error of
// 2^-16 moves the output by at most that fraction, unlike a score error,
// which the exponential amplifies, so the key side keeps three digits), B =
// value bits, whose block layout gives each lane one coordinate across 32
// tokens in one word.  One 16-row value tile holds 8 heads: head 4 mt + kg,
// digit d in row 4 kg + 2 (mt % 2) + d of tile mt / 2, so its results land in
// the lane group that holds the head's softmax state.  The constant term uses
// the same quantised P' as the bit sums, so quantisation errors enter only
// through the zero-mean centroids.
//
// Work split: grid (chunks, segments); a workgroup (4 waves) covers `span`
// tokens of one segment, sized so that the grid is resident at once, and a
// wave takes its 128-token groups w, w + 4, ... (8 key tiles; 4 value blocks),
// folding each into a running (m, l, o~) (online softmax).  The next group's
// key words are requested once the current scores exist and its value words
// once the current value sums are done, so loads overlap the arithmetic.  The
// waves' partials merge in LDS, one partial per (segment, chunk, head) goes to
// the workspace, and attend_combine128 merges the chunks (log-sum-exp),
// normalises and applies Pi_v^T.
// ---------------------------------------------------------------------------
constexpr int PST = 132;        // partial: m, l, 2 pad, o~[128]
constexpr int AGRAN = 512;      // span granule: 4 waves x 128 tokens

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
  float vu[8];                  // value Walsh coefficients, odd subsets
  float vusum;
  float* part;                  // [segs][nchunks][group][PST]
  int nchunks;                  // workgroups per segment
  int64_t span;                 // tokens per workgroup (multiple of AGRAN)
  int kv_div;                   // query segments per cache segment (1, or 2 when a segment's heads run as halves)
  // one workgroup per segment (nchunks = 1): the workgroup normalises and
  // applies the value rotation itself, as attend_combine128 would
  int solo;
  float* out;                   // [segs][group][128]
  const float* pi_v;            // value rotations (dense), [sets][128][128]
  const float* eps_v;           // or their signs (Hadamard), [sets][128]
  int rot_v;
  int n_sets_v, set_div_v;      // value rotation set of query segment seg: (seg / set_div_v) % n_sets_v
};

__device__ __forceinline__ float f16lo(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffff)); }
__device__ __forceinline__ float f16hi(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); }

// The P' A operand: row 4 kg + slice, byte position of group token tt
//   32 (tt / 32) + 16 m + 4 k + i,  b = tt % 32 = 8 i + 4 m + k
// (the value expansion's K-slot order).  Lane (t16, kg) owns tokens
// 16 tile + t16; tiles 2 c and 2 c + 1 land in bytes i and i + 2 of dword
// 8 c + 4 m + k with i = t16 / 8, and lane t16 ^ 8 owns the other two bytes,
// so one rotate by 8 within a 16-lane row completes the dword.
__device__ __forceinline__ uint32_t pair_bytes(int lo, int hi, int shift) {
  return ((uint32_t)(lo & 0xff) | ((uint32_t)(hi & 0xff) << 16)) << shift;
}
__device__ __forceinline__ uint32_t row_ror8(uint32_t v) {
  // DPP row_ror:8 (0x128): lane i of each 16-lane row reads lane (i + 8) % 16
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false);
}

// QJL: prod keys; without it MSE-only keys (BQK index planes and n).  MW: QJL
// sign words per key record (as in scores128; 2 for m = d / 2).
template <int BQK, int BQV, int KMT, bool QJL = true, int MW = 4>
__global__ __launch_bounds__(256, KMT <= 2 ? 2 : 1) void attend128(Attend128Args a) {
  constexpr int NPK = mse_planes(BQK);
  constexpr int FK = 2 * (NPK + QJL);
  constexpr int PK = BQK + QJL;
  constexpr int KSB = QJL ? 4 : 2;            // key scalar bytes per record
  constexpr uint32_t RBK = MW == 4 ? 16 * PK : 4 * (4 * BQK + MW);   // key plane bytes per record
  constexpr int NPV = mse_planes(BQV);
  constexpr int PV = BQV;
  constexpr uint32_t VBB = D * PV * 4;        // value bytes per 32-token block
  constexpr int NH = KMT * 4;                 // heads of the 16-row tiles (4 each)
  constexpr int VMT = (KMT + 1) / 2;          // value-side tiles: 8 heads x 2 digits of P' each
  typedef typename Words<PK>::v kvec;
  typedef typename Words<PV>::v vvec;
  __shared__ float sred[4][NH][PST];
  __shared__ __align__(16) uint32_t pq[4][VMT][16][32];   // A rows of P', 128 bytes each
  __shared__ float vnorm[4][128];
  const int seg = blockIdx.y;
  const int chunk = blockIdx.x;
  const int kseg = seg / a.kv_div;   // the cache segment this query segment reads
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t16 = lane & 15;
  const int kg = lane >> 4;
  const int64_t len = a.len ? (int64_t)a.len[kseg] : a.T;
  const int64_t c0 = (int64_t)chunk * a.span;
  const int64_t c1 = len < c0 + a.span ? len : c0 + a.span;
  const int ngroups = c1 > c0 ? (int)((c1 - c0 + 127) / 128) : 0;

  // lane group kg holds head 4 mt + kg on both sides
  float o_st[KMT][8], m_st[KMT], l_st[KMT];
#pragma unroll
  for (int mt = 0; mt < KMT; ++mt) {
    m_st[mt] = -INFINITY;
    l_st[mt] = 0.f;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) o_st[mt][nt] = 0.f;
  }
  // value tile vt holds head 4 mt + kg (mt = 2 vt + j) digit d in row
  // 4 kg + 2 j + d; the rows of a missing second head (odd KMT) stay zero
  if constexpr (KMT % 2) *reinterpret_cast<uint4*>(&pq[wave][VMT - 1][4 * kg + 2 + (t16 >> 3)][4 * (t16 & 7)]) =
      make_uint4(0u, 0u, 0u, 0u);

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
  for (int mt = 0; mt < KMT; ++mt) {
#pragma unroll
    for (int c = 0; c < 4; ++c) cst[mt][c] = consts[(mt * 4 + kg) * 4 + c] * (c < 2 ? a.scale2 : a.scale2 * a.kappa);
  }

  const int64_t krec0 = kseg * a.kstride + c0;
  const rsrc_t rk = make_rsrc(a.kplanes + krec0 * (RBK / 4), clamp_bytes((a.kstride - c0) * RBK));
  const rsrc_t rks = make_rsrc(a.kscal + krec0 * (KSB / 2), clamp_bytes((a.kstride - c0) * KSB));
  const int64_t vrec0 = kseg * a.vstride + c0;   // multiple of 32
  const rsrc_t rv = make_rsrc(a.vplanes + (vrec0 / 32) * (D * PV), clamp_bytes((a.vstride - c0) / 32 * VBB));
  const rsrc_t rvs = make_rsrc(a.vscal + vrec0, clamp_bytes((a.vstride - c0) * 2));
  const uint32_t vko = t16 * RBK + (MW == 4 ? kg * (PK * 4) : (kg < 2 ? kg * PK : kg * BQK + 1) * 4);
  const uint32_t vkso = t16 * KSB;
  const uint32_t vvo = (kg * D + t16) * (PV * 4);
  const uint32_t vno = lane * 4;

  kvec kw[8];
  uint32_t ks[8];
  vvec vw[8];
  uint32_t vn2;
  // the issue order is pinned (scheduling barriers) so that the prologue and
  // the loop body leave the same outstanding loads at the loop header, which
  // lets each wait count only the loads it needs
  // groups past the span get the out-of-range offset (zeros, no traffic)
  auto load_keys = [&](int g) {
    const bool ok = g < ngroups;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int tile = 0; tile < 8; ++tile) {
      const uint32_t tok = (uint32_t)(128 * g + 16 * tile);
      kw[tile] = load_words<PK>(rk, ok ? vko + tok * RBK : OOB_OFFSET);
      // (the offset written out in each branch: a shared offset variable here
      // crashes this compiler's AGPR-copy rewrite on the 4-tile kernels)
      if constexpr (QJL) ks[tile] = __builtin_amdgcn_raw_buffer_load_b32(rks, ok ? vkso + tok * 4 : OOB_OFFSET, 0, 0);
      else ks[tile] = __builtin_amdgcn_raw_buffer_load_b16(rks, ok ? vkso + tok * 2 : OOB_OFFSET, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto load_vals = [&](int g) {
    const bool ok = g < ngroups;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
      vw[nt] = load_words<PV>(rv, ok ? vvo + (uint32_t)(4 * g) * VBB + nt * 16 * (PV * 4) : OOB_OFFSET);
    vn2 = __builtin_amdgcn_raw_buffer_load_b32(rvs, ok ? vno + (uint32_t)(256 * g) : OOB_OFFSET, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  load_keys(wave);
  load_vals(wave);

  for (int g = wave; g < ngroups; g += 4) {
    const int ntok = (int)(c1 - c0 - 128 * g < 128 ? c1 - c0 - 128 * g : 128);

    // ---- phase 1: logits (log2 units) of the 8 key tiles, token t16 + 16 tile ----
    float sc[8][KMT];
#pragma unroll
    for (int tile = 0; tile < 8; ++tile) {
      if constexpr (MW == 2) kw[tile] = rotate_late_groups<PK>(kw[tile], kg >= 2);
      i32x4 am[KMT], aq[KMT];
#pragma unroll
      for (int mt = 0; mt < KMT; ++mt) am[mt] = aq[mt] = i32x4{0, 0, 0, 0};
#pragma unroll
      for (int p = 0; p < NPK + QJL; ++p) {
        uint32_t word;
        if constexpr (QJL) {
          if (p == NPK) {
            word = kw[tile][QJL ? BQK : 0];
          } else if (p < BQK) {
            word = kw[tile][p];
          } else {
            if constexpr (BQK == 3) word = kw[tile][0] ^ kw[tile][1] ^ kw[tile][2];
          }
        } else {
          word = plane_word<BQK, NPK, false>(kw[tile], p);
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
      const bool valid = tile * 16 + t16 < ntok;
      const float n = f16lo(ks[tile]), gm = f16hi(ks[tile]);
#pragma unroll
      for (int mt = 0; mt < KMT; ++mt) {
        const float mse = fmaf(mse_digits<NPK>(am[mt]), cst[mt][0], cst[mt][1]);
        const float qjl = fmaf((float)combine3(aq[mt]), cst[mt][2], cst[mt][3]);
        sc[tile][mt] = valid ? (QJL ? n * fmaf(gm, qjl, mse) : n * mse) : -INFINITY;
      }
    }
    load_keys(g + 4);

    // ---- phase 2: softmax statistics and the int8 P' rows ----
    vnorm[wave][2 * lane] = 2 * lane < ntok ? f16lo(vn2) : 0.f;
    vnorm[wave][2 * lane + 1] = 2 * lane + 1 < ntok ? f16hi(vn2) : 0.f;
    float vn[8];
#pragma unroll
    for (int tile = 0; tile < 8; ++tile) vn[tile] = vnorm[wave][tile * 16 + t16];
    float fsig[KMT];
    const int bsh = 8 * (t16 >> 3);
    const int dw0 = 4 * ((t16 >> 2) & 1) + (t16 & 3);
#pragma unroll
    for (int mt = 0; mt < KMT; ++mt) {
      float mx = -INFINITY;
#pragma unroll
      for (int tile = 0; tile < 8; ++tile) mx = fmaxf(mx, sc[tile][mt]);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      const float mref = fmaxf(m_st[mt], mx);           // running reference
      const float alpha = __builtin_amdgcn_exp2f(m_st[mt] - mref);   // 0 on the first group
      float pv[8], ls = 0.f, pmax = 0.f;
#pragma unroll
      for (int tile = 0; tile < 8; ++tile) {
        const float pp = __builtin_amdgcn_exp2f(sc[tile][mt] - mref);
        ls += pp;
        pv[tile] = pp * vn[tile];
        pmax = fmaxf(pmax, pv[tile]);
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        ls += __shfl_xor(ls, o, 64);
        pmax = fmaxf(pmax, __shfl_xor(pmax, o, 64));
      }
      const float sig = pmax > 0.f ? pmax / QMAX2 : 1.f;
      const float inv = 1.f / sig;
      int qsum = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        int s0[2], s1[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int qi = (int)rintf(fminf(pv[2 * c + h] * inv, QMAX2));
          qsum += qi;                                   // <= 128 * 127 * 2^8
          s0[h] = (qi + 128) >> 8;                      // balanced digits, as slices2
          s1[h] = qi - 256 * s0[h];
        }
        const uint32_t d0 = pair_bytes(s0[0], s0[1], bsh);
        const uint32_t d1 = pair_bytes(s1[0], s1[1], bsh);
        const int dw = 8 * c + dw0;
        pq[wave][mt / 2][4 * kg + 2 * (mt % 2)][dw] = d0 | row_ror8(d0);
        pq[wave][mt / 2][4 * kg + 2 * (mt % 2) + 1][dw] = d1 | row_ror8(d1);
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) qsum += __shfl_xor(qsum, o, 64);
      m_st[mt] = mref;
      l_st[mt] = fmaf(alpha, l_st[mt], ls);
      fsig[mt] = sig;
      const float cv0 = -a.vusum * sig * (float)qsum;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) o_st[mt][nt] = fmaf(alpha, o_st[mt][nt], cv0);
    }

    // ---- phase 3: A operands (row = lane % 16, token bytes of block kg) ----
    i32x4 pa[VMT][2];
#pragma unroll
    for (int vt = 0; vt < VMT; ++vt)
#pragma unroll
      for (int m = 0; m < 2; ++m) pa[vt][m] = *reinterpret_cast<const i32x4*>(&pq[wave][vt][t16][8 * kg + 4 * m]);

    // ---- phase 4: value planes, each folded with its Walsh weight ----
#pragma unroll
    for (int sp = 0; sp < NPV; ++sp) {
      i32x4 acc[VMT][8];
#pragma unroll
      for (int vt = 0; vt < VMT; ++vt)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) acc[vt][nt] = i32x4{0, 0, 0, 0};
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        uint32_t word;
        if (sp < BQV) {
          word = vw[nt][sp];
        } else {
          word = 0u;
#pragma unroll
          for (int p = 0; p < BQV; ++p)
            if (plane_subset(BQV, sp) >> p & 1) word ^= vw[nt][p];
        }
        uint32_t e8[8];
        expand8(word, e8);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const i32x4 bv = {(int)e8[4 * m], (int)e8[4 * m + 1], (int)e8[4 * m + 2], (int)e8[4 * m + 3]};
#pragma unroll
          for (int vt = 0; vt < VMT; ++vt) acc[vt][nt] = mfma16x16x64i8(pa[vt][m], bv, acc[vt][nt]);
        }
      }
      const float w2 = 2.f * a.vu[sp];
      // accumulator register 2 j + d of lane group kg: head 4 (2 vt + j) + kg, digit d
#pragma unroll
      for (int mt = 0; mt < KMT; ++mt) {
        const float f = w2 * fsig[mt];
        const int vt = mt / 2, j = mt % 2;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
          o_st[mt][nt] = fmaf((float)(acc[vt][nt][2 * j] * 256 + acc[vt][nt][2 * j + 1]), f, o_st[mt][nt]);
      }
    }
    load_vals(g + 4);
  }

  // ---- phase 5: merge the four waves' partials in LDS, publish the chunk's ----
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
  if (a.solo) {
    // the segment's only workgroup: o~ / l per head into the LDS (the P'
    // rows are free now), then o = Pi_v^T (o~ / l), lane (j = 32 wave +
    // lane % 32, k half kh) summing its 64 rotation entries, the halves
    // joined by one shuffle
    float* ot = reinterpret_cast<float*>(&pq[0][0][0][0]);     // [nh][128]
    static_assert(sizeof(pq) >= sizeof(float) * NH * D, "o~ fits the P' rows");
    for (int i = threadIdx.x; i < nh * D; i += blockDim.x) {
      const int h = i / D, k = i % D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, sred[w][h][0]);
      float l = 0.f, o = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float wt = __builtin_amdgcn_exp2f(sred[w][h][0] - M);   // 0 for empty waves
          l += wt * sred[w][h][1];
          o += wt * sred[w][h][4 + k];
        }
      }
      const float inv = l > 0.f ? 1.f / l : 0.f;
      ot[h * D + k] = o * inv;
    }
    const int set = a.n_sets_v > 1 ? (seg / a.set_div_v) % a.n_sets_v : 0;
    const int j = 32 * wave + (lane & 31), kh = lane >> 5;
    float pj[64];
    if (a.rot_v == TQ_ROT_DENSE) {
      const float* pv = a.pi_v + (size_t)set * D * D + (size_t)(64 * kh) * D + j;
#pragma unroll
      for (int kk = 0; kk < 64; ++kk) pj[kk] = pv[(size_t)kk * D];
    } else {
      const float sg = a.eps_v[(size_t)set * D + j] * rsqrtf((float)D);
#pragma unroll
      for (int kk = 0; kk < 64; ++kk) pj[kk] = (__popc(j & (64 * kh + kk)) & 1) ? -sg : sg;
    }
    __syncthreads();
    for (int h = 0; h < nh; ++h) {
      const float4* src = reinterpret_cast<const float4*>(ot + h * D + 64 * kh);
      float acc = 0.f;
#pragma unroll
      for (int k4 = 0; k4 < 16; ++k4) {
        const float4 x = src[k4];
        acc = fmaf(pj[4 * k4], x.x, acc);
        acc = fmaf(pj[4 * k4 + 1], x.y, acc);
        acc = fmaf(pj[4 * k4 + 2], x.z, acc);
        acc = fmaf(pj[4 * k4 + 3], x.w, acc);
      }
      acc += __shfl_xor(acc, 32, 64);
      if (kh == 0) a.out[((size_t)seg * a.group + h) * D + j] = acc;
    }
    return;
  }
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
          const float wt = __builtin_amdgcn_exp2f(sred[w][h][0] - M);     // 0 for empty waves
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
  int rot;
  const float* pi_v;
  const float* eps_v;
  float* out;
  int n_sets, set_div;   // value rotation sets: segment seg uses set (seg / set_div) % n_sets
};

// One workgroup (256 threads) per segment: log-sum-exp merge of the chunk
// partials of every head into LDS, then o = Pi_v^T o~ with Pi_v staged in
// LDS (dense) or the inverse sign-flipped Hadamard transform.  Pi_v and the
// partials of up to 8 chunks are requested together, so a segment with at
// most 8 chunks costs one memory round trip.
constexpr int CMB_G = 16;
constexpr int CMB_B = 8;       // chunks merged per batch of loads
__global__ __launch_bounds__(256, 1) void attend_combine128(Combine128Args a) {
  __shared__ __align__(16) float pis[D * D];
  __shared__ __align__(16) float ot[CMB_G][D];
  const int seg = blockIdx.x;
  const int t = threadIdx.x;
  const bool dense = a.rot == TQ_ROT_DENSE;
  const int set = a.n_sets > 1 ? (seg / a.set_div) % a.n_sets : 0;
  const float* pi_v = a.pi_v ? a.pi_v + (size_t)set * D * D : nullptr;
  const float* eps_v = a.eps_v ? a.eps_v + (size_t)set * D : nullptr;
  if (dense) {
    // Pi_v -> LDS by the direct global-to-LDS path: lane i of a wave's
    // instruction fills 16 bytes at the wave's LDS base + 16 i
    const int w = t >> 6;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(pi_v + (size_t)(256 * i + t) * 4),
          (__attribute__((address_space(3))) void*)(pis + (256 * i + 64 * w) * 4), 16, 0, 0);
  }
  const float* pseg = a.part + (size_t)seg * a.nchunks * a.group * PST;
  const int j4 = 4 * (t & 31);
  for (int hb = 0; hb < a.group; hb += 8) {
    const int h = hb + (t >> 5);
    const int hc = h < a.group ? h : a.group - 1;
    float M = -INFINITY, L = 0.f;
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int cb = 0; cb < a.nchunks; cb += CMB_B) {
      float mc[CMB_B], lc[CMB_B];
      float4 oc[CMB_B];
#pragma unroll
      for (int u = 0; u < CMB_B; ++u) {
        const int c = cb + u < a.nchunks ? cb + u : a.nchunks - 1;
        const float* pc = pseg + ((size_t)c * a.group + hc) * PST;
        mc[u] = pc[0];
        lc[u] = pc[1];
        oc[u] = *reinterpret_cast<const float4*>(pc + 4 + j4);
      }
      float Mb = M;
#pragma unroll
      for (int u = 0; u < CMB_B; ++u) {
        if (cb + u >= a.nchunks) mc[u] = -INFINITY;
        Mb = fmaxf(Mb, mc[u]);
      }
      if (Mb == -INFINITY) continue;
      const float r = __builtin_amdgcn_exp2f(M - Mb);      // 0 while M is -inf
      L *= r;
      acc.x *= r;
      acc.y *= r;
      acc.z *= r;
      acc.w *= r;
#pragma unroll
      for (int u = 0; u < CMB_B; ++u) {
        const float wt = __builtin_amdgcn_exp2f(mc[u] - Mb);   // 0 for empty chunks
        L = fmaf(wt, lc[u], L);
        acc.x = fmaf(wt, oc[u].x, acc.x);
        acc.y = fmaf(wt, oc[u].y, acc.y);
        acc.z = fmaf(wt, oc[u].z, acc.z);
        acc.w = fmaf(wt, oc[u].w, acc.w);
      }
      M = Mb;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    if (h < a.group)
      *reinterpret_cast<float4*>(&ot[h][j4]) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
  __builtin_amdgcn_s_waitcnt(0);   // the direct-to-LDS loads have landed
  __syncthreads();
  const int j = t & (D - 1), h0 = t >> 7;
  if (j >= a.d) return;
  for (int hb = 0; hb < a.group; hb += 8) {
    float o[4] = {0.f, 0.f, 0.f, 0.f};     // heads hb + h0 + 2 i
    int hh[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) hh[i] = hb + h0 + 2 * i < a.group ? hb + h0 + 2 * i : 0;
    if (dense) {
      for (int k = 0; k < D; k += 4) {
        const float p0 = pis[k * D + j], p1 = pis[(k + 1) * D + j];
        const float p2 = pis[(k + 2) * D + j], p3 = pis[(k + 3) * D + j];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 v = *reinterpret_cast<const float4*>(&ot[hh[i]][k]);
          o[i] = fmaf(p0, v.x, fmaf(p1, v.y, fmaf(p2, v.z, fmaf(p3, v.w, o[i]))));
        }
      }
    } else {
      for (int k = 0; k < D; ++k) {
        const bool neg = __popc(j & k) & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = ot[hh[i]][k];
          o[i] += neg ? -v : v;
        }
      }
      const float sg = eps_v[j] * rsqrtf((float)D);
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] *= sg;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = hb + h0 + 2 * i;
      if (h < a.group) a.out[((size_t)seg * a.group + h) * a.d + j] = o[i];
    }
  }
}

// Most workgroups per segment the workspace provides for: enough to fill a
// device of 4096 resident workgroups, never more than T / AGRAN.
int64_t attend_kmax(int segs, int64_t T) {
  int64_t k = (4096 + segs - 1) / (segs > 0 ? segs : 1);
  const int64_t kt = (T + AGRAN - 1) / AGRAN;
  if (k > kt) k = kt;
  return k < 1 ? 1 : k;
}

template <int BQK, int BQV, int MT, bool QJL = true, int MW = 4>
hipError_t launch_attend(Attend128Args& s, int segs, hipStream_t stream) {
  static const int nb = occupancy(reinterpret_cast<const void*>(&attend128<BQK, BQV, MT, QJL, MW>), 256);
  s.span = split_span(segs, s.T, nb * device_cus(), AGRAN, attend_kmax(segs, s.T));
  s.nchunks = (int)((s.T + s.span - 1) / s.span);
  s.solo = s.nchunks == 1;
  hipLaunchKernelGGL((attend128<BQK, BQV, MT, QJL, MW>), dim3((unsigned)s.nchunks, (unsigned)segs), dim3(256), 0,
                     stream, s);
  return hipGetLastError();
}

// Prod keys with m = d / 2 QJL rows against values of 2..4 bits.
template <int BQK, int BQV>
hipError_t launch_attend_half(Attend128Args& s, int segs, int mt, hipStream_t stream) {
  switch (mt) {
    case 1: return launch_attend<BQK, BQV, 1, true, 2>(s, segs, stream);
    case 2: return launch_attend<BQK, BQV, 2, true, 2>(s, segs, stream);
    case 3: return launch_attend<BQK, BQV, 3, true, 2>(s, segs, stream);
    case 4: return launch_attend<BQK, BQV, 4, true, 2>(s, segs, stream);
  }
  return hipErrorInvalidValue;
}

// MSE-only keys of BQK bits (2..4) against values of 2..4 bits; 4-bit keys
// take at most two 16-row tiles (8 query heads: their 16 fragments per tile
// fill the registers).
template <int BQK, int BQV>
hipError_t launch_attend_mse_keys(Attend128Args& s, int segs, int mt, hipStream_t stream) {
  switch (mt) {
    case 1: return launch_attend<BQK, BQV, 1, false>(s, segs, stream);
    case 2: return launch_attend<BQK, BQV, 2, false>(s, segs, stream);
    case 3: if constexpr (BQK < 4) return launch_attend<BQK, BQV, 3, false>(s, segs, stream); break;
    case 4: if constexpr (BQK < 4) return launch_attend<BQK, BQV, 4, false>(s, segs, stream); break;
  }
  return hipErrorInvalidValue;
}

size_t attend_pack_bytes(int segs, int group) { return scores128_workspace(segs, group); }

size_t attend_part_bytes(int segs, int group, int64_t T) {
  return ((size_t)segs * attend_kmax(segs, T) * group * PST * sizeof(float) + 255) / 256 * 256;
}

}  // namespace

size_t attend128_workspace(int segs, int group, int64_t T) {
  return attend_pack_bytes(segs, group) + attend_part_bytes(segs, group, T);
}

hipError_t launch_attend128_prepare(const AttendArgs& a, hipStream_t stream) {
  return launch_scores128_prep(a.k, 3, stream);
}

hipError_t launch_attend128(const AttendArgs& a, hipStream_t stream) {
  uint8_t* ws = static_cast<uint8_t*>(a.ws);
  hipError_t e = a.prepared ? hipSuccess : launch_scores128_prep(a.k, 3, stream);
  if (e != hipSuccess) return e;
  Attend128Args s;
  s.pack = ws;
  s.kplanes = a.k.planes;
  s.kscal = a.k.scalars;
  s.kstride = a.k.seg_stride;
  s.vplanes = a.planes_v;
  s.vscal = a.scalars_v;
  s.vstride = a.seg_stride_v;
  s.len = a.k.len;
  s.T = a.k.T;
  s.group = a.k.group;
  s.kappa = (float)(std::sqrt(M_PI / 2.0) / (a.k.qjl ? a.k.m : D));
  s.scale2 = a.scale * 1.4426950408889634f;
  walsh_coefficients(a.cb_v, a.bq_v, s.vu, &s.vusum);
  s.part = reinterpret_cast<float*>(ws + attend_pack_bytes(a.k.segs, a.k.group));
  s.nchunks = 0;   // set by the launcher
  s.span = 0;
  s.kv_div = a.kv_div;
  s.solo = 0;   // set by the launcher
  s.out = a.out;
  s.pi_v = a.pi_v;
  s.eps_v = a.eps_v;
  s.rot_v = a.rot_v;
  s.n_sets_v = a.n_sets_v > 1 ? a.n_sets_v : 1;
  s.set_div_v = (a.set_div_v > 1 ? a.set_div_v : 1) * a.kv_div;
  const int mt = (a.k.group + 3) / 4;
  if (a.k.qjl && a.k.m == D / 2) {
    switch (a.k.bq * 10 + a.bq_v) {
      case 12: e = launch_attend_half<1, 2>(s, a.k.segs, mt, stream); break;
      case 13: e = launch_attend_half<1, 3>(s, a.k.segs, mt, stream); break;
      case 14: e = launch_attend_half<1, 4>(s, a.k.segs, mt, stream); break;
      case 22: e = launch_attend_half<2, 2>(s, a.k.segs, mt, stream); break;
      case 23: e = launch_attend_half<2, 3>(s, a.k.segs, mt, stream); break;
      case 24: e = launch_attend_half<2, 4>(s, a.k.segs, mt, stream); break;
      case 32: e = launch_attend_half<3, 2>(s, a.k.segs, mt, stream); break;
      case 33: e = launch_attend_half<3, 3>(s, a.k.segs, mt, stream); break;
      case 34: e = launch_attend_half<3, 4>(s, a.k.segs, mt, stream); break;
      default: return hipErrorInvalidValue;
    }
  } else if (!a.k.qjl) {
    switch (a.k.bq * 10 + a.bq_v) {
      case 22: e = launch_attend_mse_keys<2, 2>(s, a.k.segs, mt, stream); break;
      case 23: e = launch_attend_mse_keys<2, 3>(s, a.k.segs, mt, stream); break;
      case 24: e = launch_attend_mse_keys<2, 4>(s, a.k.segs, mt, stream); break;
      case 32: e = launch_attend_mse_keys<3, 2>(s, a.k.segs, mt, stream); break;
      case 33: e = launch_attend_mse_keys<3, 3>(s, a.k.segs, mt, stream); break;
      case 34: e = launch_attend_mse_keys<3, 4>(s, a.k.segs, mt, stream); break;
      case 42: e = launch_attend_mse_keys<4, 2>(s, a.k.segs, mt, stream); break;
      case 43: e = launch_attend_mse_keys<4, 3>(s, a.k.segs, mt, stream); break;
      case 44: e = launch_attend_mse_keys<4, 4>(s, a.k.segs, mt, stream); break;
      default: return hipErrorInvalidValue;
    }
  } else switch ((a.k.bq * 10 + a.bq_v) * 10 + mt) {
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
    case 141: e = launch_attend<1, 4, 1>(s, a.k.segs, stream); break;
    case 142: e = launch_attend<1, 4, 2>(s, a.k.segs, stream); break;
    case 143: e = launch_attend<1, 4, 3>(s, a.k.segs, stream); break;
    case 144: e = launch_attend<1, 4, 4>(s, a.k.segs, stream); break;
    case 241: e = launch_attend<2, 4, 1>(s, a.k.segs, stream); break;
    case 242: e = launch_attend<2, 4, 2>(s, a.k.segs, stream); break;
    case 243: e = launch_attend<2, 4, 3>(s, a.k.segs, stream); break;
    case 244: e = launch_attend<2, 4, 4>(s, a.k.segs, stream); break;
    case 341: e = launch_attend<3, 4, 1>(s, a.k.segs, stream); break;
    case 342: e = launch_attend<3, 4, 2>(s, a.k.segs, stream); break;
    case 343: e = launch_attend<3, 4, 3>(s, a.k.segs, stream); break;
    case 344: e = launch_attend<3, 4, 4>(s, a.k.segs, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  if (s.solo) return hipSuccess;   // each segment's workgroup finished it
  Combine128Args c;
  c.part = s.part;
  c.nchunks = s.nchunks;
  c.group = a.k.group;
  c.d = a.k.d;
  c.rot = a.rot_v;
  c.pi_v = a.pi_v;
  c.eps_v = a.eps_v;
  c.n_sets = a.n_sets_v > 1 ? a.n_sets_v : 1;
  c.set_div = (a.set_div_v > 1 ? a.set_div_v : 1) * a.kv_div;
  c.out = a.out;
  hipLaunchKernelGGL(attend_combine128, dim3((unsigned)a.k.segs), dim3(256), 0, stream, c);
  return hipGetLastError();
}

}  // namespace tq
