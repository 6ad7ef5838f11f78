// TurboQuant encode kernels for gfx950 (MI355X), d = d_rot = 128, dense or
// sign-flipped Hadamard rotation.
//
// Per vector x (blog notes on the TurboQuant paper: Q_mse and Q_prod; the
// explainer page, sections 6 and 8):
//   n = ||x||, u = x / n, y = Pi u, idx_j = #{beta_k <= y_j}           (Q_mse)
//   r = y - c[idx], gamma = ||r||, z = [S r >= 0]                        (Q_prod)
//
// Layout of the work: one wave owns a tile of 32 vectors (NT = 1) or 64
// (NT = 2).  Both rotations are dense 128x128 contractions on the matrix cores
// (v_mfma_f32_32x32x16_f16):
//   GEMM1  Y^T = (16 Pi) . X^T      A = Pi fragments from LDS, B = x rows
//   GEMM2  Z^T = S . (256 R)^T      A = S fragments from LDS, B = residuals
// Float32 accuracy comes from splitting the fixed matrices into fp16 hi + lo
// (and fp32 operands likewise): Pi_hi x + Pi_lo x for fp16 inputs (x is exact
// in fp16), three products for fp32 operands (the lo*lo term, ~2^-22, is
// dropped).  The power-of-two prescales keep the lo parts out of the fp16
// subnormal range and are undone exactly.
//
// Sign-flipped Hadamard rotation (explainer page, the random Hadamard variant;
// blog notes, the fast rotation): y = H diag(eps) u / sqrt(128) with the
// Sylvester H, H[j][k] = (-1)^popcount(j & k).  At d = 128 it runs through the
// same GEMM1 as the matrix 16 H diag(eps), whose entries +-16 are exact in
// fp16 (no lo part, one pass for fp16 inputs); 1/sqrt(128) joins the output
// scale.
//
// The A rows are permuted so that, in the accumulator layout, lane
// (v = lane % 32, h = lane / 32) holds coordinates 64 h + 16 mt + r of vector
// v in register r of row tile mt.  A lane therefore owns the whole 32-bit
// plane words 2h and 2h+1 of its vector (a contiguous 8P bytes of the record,
// whose planes are interleaved word by word): bit packing is a shift-or per
// coordinate with no cross-lane traffic, and the GEMM1 accumulators are
// already in the B layout GEMM2 needs (K slot e of MFMA ks2 in lane half h is
// coordinate 64 h + 8 ks2 + e, the same map GEMM1 uses for x).
#include <algorithm>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int D = 128;
constexpr float PI_SCALE = 16.f;   // 2^4
constexpr float R_SCALE = 256.f;   // 2^8
constexpr float U_SCALE = 64.f;    // 2^6 (fp32 inputs, after normalising)
constexpr float HAD_SCALE = 0.08838834764831845f;   // 1 / sqrt(128)
constexpr int FRAGS = 4 * 8 * 2 * 64;  // half8 per 128x128 matrix (hi and lo)

__device__ __forceinline__ int frag_index(int mt, int ks, int part, int lane) {
  return ((mt * 8 + ks) * 2 + part) * 64 + lane;
}

// Output row rho of a 32-row tile -> the coordinate it stands for.
__device__ __forceinline__ int row_coord(int rho, int mt) {
  int h = (rho >> 2) & 1;
  int r = ((rho >> 3) << 2) | (rho & 3);
  return 64 * h + 16 * mt + r;
}
// The same for a 64-row QJL matrix (m = d / 2) in two row tiles: lane half h
// holds projection rows 32 h + 16 mt + r, i.e. all 32 bits of sign word h.
__device__ __forceinline__ int row_half(int rho, int mt) {
  int h = (rho >> 2) & 1;
  int r = ((rho >> 3) << 2) | (rho & 3);
  return 32 * h + 16 * mt + r;
}

// M is [128][128] float32 row-major (or, with eps, the matrix H diag(eps)).
// Fragment (mt, ks) of lane l holds scale * M[row_coord(l % 32, mt)][64 (l / 32)
// + 8 ks + e], e = 0..7, as hi, lo.  NTHR threads build the 2048 fragments,
// each requesting up to 8 fragments' operands before splitting any of them
// (a small workgroup would otherwise wait out one memory round trip per
// fragment).
// HALF: a 64-row matrix in two row tiles (row_half); fragments of row tiles
// 2 and 3 are not built.
template <int NTHR, bool HALF = false>
__device__ void build_frags(half8* lds, const float* __restrict__ M, float scale, const float* eps = nullptr) {
  constexpr int TOTAL = (HALF ? 2 : 4) * 8 * 64;
  constexpr int PER = TOTAL / NTHR;
  constexpr int U = PER < 8 ? PER : 8;
  static_assert(TOTAL % NTHR == 0 && PER % U == 0, "fragments per thread");
  for (int b0 = 0; b0 < PER; b0 += U) {
    float4 p[U], q[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int f = threadIdx.x + (b0 + u) * NTHR;
      const int lane = f & 63, ks = (f >> 6) & 7, mt = f >> 9;
      const int row = HALF ? row_half(lane & 31, mt) : row_coord(lane & 31, mt);
      const int k0 = 64 * (lane >> 5) + 8 * ks;
      const float4* src = reinterpret_cast<const float4*>(eps ? eps + k0 : M + row * D + k0);
      p[u] = src[0];
      q[u] = src[1];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int f = threadIdx.x + (b0 + u) * NTHR;
      const int lane = f & 63, ks = (f >> 6) & 7, mt = f >> 9;
      const int row = HALF ? row_half(lane & 31, mt) : row_coord(lane & 31, mt);
      const int k0 = 64 * (lane >> 5) + 8 * ks;
      float v[8] = {p[u].x, p[u].y, p[u].z, p[u].w, q[u].x, q[u].y, q[u].z, q[u].w};
      if (eps) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (__popc(row & (k0 + e)) & 1) ? -v[e] : v[e];
      }
      half8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        _Float16 h, l;
        split_f16(v[e] * scale, h, l);
        hi[e] = h;
        lo[e] = l;
      }
      lds[frag_index(mt, ks, 0, lane)] = hi;
      lds[frag_index(mt, ks, 1, lane)] = lo;
    }
  }
}

// Lane mask of [y >= b] (ordered: false for NaN), one v_cmp into an SGPR pair.
__device__ __forceinline__ uint64_t ge_mask(float y, float b) { return __builtin_amdgcn_fcmpf(y, b, 3); }

// m[lane] ? t : f
__device__ __forceinline__ float select_mask(uint64_t m, float t, float f) {
  float r;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(f), "v"(t), "s"(m));
  return r;
}

// 2 w + m[lane]: one add with the mask as carry-in
__device__ __forceinline__ uint32_t shift_in(uint32_t w, uint64_t m) {
  uint32_t r;
  uint64_t carry;
  asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(carry) : "v"(w), "s"(m));
  return r;
}

template <int BQ>
__device__ __forceinline__ void quantize(float y, const Codebook& cb, int& idx, float& chat) {
  idx = 0;
  chat = cb.c[0];
#pragma unroll
  for (int k = 0; k < (1 << BQ) - 1; ++k) {
    const bool ge = y >= cb.b[k];
    idx += ge ? 1 : 0;
    chat = ge ? cb.c[k + 1] : chat;
  }
}

// PROD: per-record key layout (in-lane packing); with QJL the residual's
// sign projection follows (prod keys), without it the record holds the BQ
// index planes and the norm only (MSE-only keys).  !PROD: values in the
// token-blocked layout.
// SLOTS: values written through a slot map (any record order), whose tiles
// may take the per-bit path; without it only a ragged last tile can.
// EDEN: an MSE record stores the unbiased per-vector scale n / <y, c[idx]>
// instead of n (EDEN's scale; DRIVE's at one bit).
// MW: QJL sign words per key record, m / 32 (4: m = d; 2: m = d / 2, whose
// record holds for each 32-coordinate group w the index words, then sign word
// w if w < 2).
template <bool PROD, bool QJL, int BQ, bool F16IN, int NT, int WAVES, bool HAD, bool SLOTS, bool EDEN = false,
          int MW = 4>
__global__ __launch_bounds__(64 * WAVES, 1) void encode_dense128(EncodeArgs a) {
  static_assert(PROD || !QJL, "values carry no QJL bits");
  static_assert(!(EDEN && QJL), "the scale replaces the norm of MSE records only");
  static_assert(MW == 4 || (QJL && MW == 2), "m = d / 2 is a prod-key form");
  extern __shared__ half8 lds[];
  half8* fpi = lds;
  half8* fs = lds + FRAGS;
  build_frags<64 * WAVES>(fpi, a.pi, PI_SCALE, HAD ? a.eps : nullptr);
  if (QJL) build_frags<64 * WAVES, MW == 2>(fs, a.s, 1.f);
  __syncthreads();

  constexpr int P = QJL ? BQ + 1 : BQ;      // planes per record
  constexpr int VT = 32 * NT;               // vectors per wave tile
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int v = lane & 31;
  const int h = lane >> 5;
  const int64_t ntiles = (a.n + VT - 1) / VT;
  const int64_t stride = (int64_t)gridDim.x * WAVES;

  // The codebook in VGPRs: as kernel arguments it would hold 32 SGPRs, which
  // the comparison masks of the quantiser need.
  Codebook cbv;
#pragma unroll
  for (int k = 0; k < (1 << BQ); ++k) asm volatile("v_mov_b32 %0, %1" : "=v"(cbv.c[k]) : "s"(a.cb.c[k]));
#pragma unroll
  for (int k = 0; k < (1 << BQ) - 1; ++k) asm volatile("v_mov_b32 %0, %1" : "=v"(cbv.b[k]) : "s"(a.cb.b[k]));

  for (int64_t tile = (int64_t)blockIdx.x * WAVES + wave; tile < ntiles; tile += stride) {
    // The fragment reads below are loop-invariant; without this barrier the
    // compiler hoists all of them (256 registers) out of the loop and spills.
    asm volatile("" ::: "memory");
    // ---- load 64 coordinates (64 h .. 64 h + 63) of each vector, norms ----
    half8 xh[NT][8];
    half8 xl[NT][8];   // fp32 inputs only
    // ysc: output scale of GEMM1 (y = ysc acc); inv = 1 / ysc.  A zero vector
    // (acc = 0) takes ysc = inv = 1, so that y = 0 and r = -c[idx] as defined.
    float ysc[NT], inv[NT], nrm[NT];
    int64_t vec[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      vec[nt] = tile * VT + nt * 32 + v;
      const bool valid = vec[nt] < a.n;
      float s2 = 0.f;
      if (F16IN) {
        const uint4* src = reinterpret_cast<const uint4*>(
            static_cast<const _Float16*>(a.x) + (valid ? vec[nt] : 0) * a.ld_x + 64 * h);
        float s4[4] = {0.f, 0.f, 0.f, 0.f};   // four chains instead of one 64-long one
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          half8 hv = __builtin_bit_cast(half8, valid ? src[ks] : make_uint4(0, 0, 0, 0));
          xh[nt][ks] = hv;
#pragma unroll
          for (int e = 0; e < 8; ++e) s4[e & 3] += (float)hv[e] * (float)hv[e];
        }
        s2 = (s4[0] + s4[1]) + (s4[2] + s4[3]);
      } else {
        const float4* src = reinterpret_cast<const float4*>(
            static_cast<const float*>(a.x) + (valid ? vec[nt] : 0) * a.ld_x + 64 * h);
        float xv[64];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float4 w = valid ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
          xv[4 * i] = w.x; xv[4 * i + 1] = w.y; xv[4 * i + 2] = w.z; xv[4 * i + 3] = w.w;
        }
        float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 64; ++i) s4[i & 3] += xv[i] * xv[i];
        s2 = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        s2 += shfl_xor_f(s2, 32);
        const float n = sqrtf(s2);
        const float un = n > 0.f ? U_SCALE / n : 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            _Float16 hi, lo;
            split_f16(xv[8 * ks + e] * un, hi, lo);
            xh[nt][ks][e] = hi;
            xl[nt][ks][e] = lo;
          }
        }
        nrm[nt] = n;
        ysc[nt] = (HAD ? HAD_SCALE : 1.f) / (U_SCALE * PI_SCALE);
        inv[nt] = (U_SCALE * PI_SCALE) / (HAD ? HAD_SCALE : 1.f);
        continue;
      }
      s2 += shfl_xor_f(s2, 32);
      const float n = sqrtf(s2);
      nrm[nt] = n;
      ysc[nt] = n > 0.f ? (HAD ? HAD_SCALE : 1.f) / (n * PI_SCALE) : 1.f;
      inv[nt] = n > 0.f ? (n * PI_SCALE) / (HAD ? HAD_SCALE : 1.f) : 1.f;
    }
    // keys: the scale goes into the codebook instead of every coordinate, so
    // the raw accumulator is compared with beta / ysc and the residual is
    // ysc (acc - c[idx] / ysc), scaled once in its fp16 split (the decisions
    // move by a rounding step at most, inside the boundary band)
    float bsc[NT][(1 << BQ) - 1], csc[NT][1 << BQ], rsc[NT];
    if (PROD) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int k = 0; k < (1 << BQ) - 1; ++k) bsc[nt][k] = cbv.b[k] * inv[nt];
#pragma unroll
        for (int k = 0; k < (1 << BQ); ++k) csc[nt][k] = cbv.c[k] * inv[nt];
        rsc[nt] = R_SCALE * ysc[nt];
      }
    }

    // ---- values: one aligned, fully valid 32-record block per tile? ----
    bool vfast = false;
    int64_t vblock = 0, vrec = 0;
    uint32_t vlo[BQ], vhi[BQ];
    if (!PROD) {
      static_assert(PROD || NT == 1, "value tiles are 32 vectors");
      const int64_t r0 = a.slot ? a.slot[tile * 32 < a.n ? tile * 32 : 0] : tile * 32;
      // this lane's record, read once (the per-bit path below would otherwise
      // re-read it after every batch of atomics)
      vrec = vec[0] < a.n ? (a.slot ? a.slot[vec[0]] : vec[0]) : 0;
      const bool mine = vec[0] < a.n && vrec == r0 + v;
      vfast = (r0 % 32) == 0 && __all(mine);
      vblock = r0 / 32;
#pragma unroll
      for (int p = 0; p < BQ; ++p) vlo[p] = vhi[p] = 0u;
    }
    // ---- GEMM1 per row tile, then quantize, pack, residual ----
    uint32_t iw[NT][BQ][2];
    half8 rh[NT][8], rl[NT][8];
    float g2[NT];
    float yc[NT];   // EDEN: this lane's part of <y, c[idx]> (keys: in accumulator x scaled-centroid units)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      g2[nt] = 0.f;
      yc[nt] = 0.f;
#pragma unroll
      for (int p = 0; p < BQ; ++p) iw[nt][p][0] = iw[nt][p][1] = 0u;
    }
    // GEMM1 software-pipelined: the 16 products of row tile mt + 1 are
    // issued between the epilogue steps of row tile mt
    auto mma = [&](f32x16* acc, int mt, int ks) {
      const half8 ahi = fpi[frag_index(mt, ks, 0, lane)];
      const half8 alo = fpi[frag_index(mt, ks, 1, lane)];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        acc[nt] = mfma32x32x16(ahi, xh[nt][ks], acc[nt]);
        if (!HAD) acc[nt] = mfma32x32x16(alo, xh[nt][ks], acc[nt]);   // +-16 has no lo part
        if (!F16IN) acc[nt] = mfma32x32x16(ahi, xl[nt][ks], acc[nt]);
      }
    };
    // per-bit value path: this lane's current words of the 16 coordinates of
    // a row tile, read before its epilogue.  Only this lane writes its bit of
    // a word (records are distinct), so a plain read shows that bit exactly
    // and only the bits that change need an atomic.
    uint32_t oldw[SLOTS ? 16 * BQ : 1];
    auto load_old = [&](int mt) {
      if (PROD || !SLOTS || vfast || vec[0] >= a.n) return;
      const uint4* src = reinterpret_cast<const uint4*>(a.planes + (vrec >> 5) * (D * BQ) + (64 * h + 16 * mt) * BQ);
#pragma unroll
      for (int q = 0; q < 4 * BQ; ++q) {
        const uint4 w = src[q];
        oldw[4 * q] = w.x;
        oldw[4 * q + 1] = w.y;
        oldw[4 * q + 2] = w.z;
        oldw[4 * q + 3] = w.w;
      }
    };
    auto epi = [&](const f32x16* acc, int mt, int nt, int r) {
          const float y = PROD ? acc[nt][r] : acc[nt][r] * ysc[nt];   // keys: unscaled
          if (!PROD && vfast) {
            // The comparison masks are wave ballots of [y >= beta_k] (bit v:
            // vector v at coordinate 16 mt + r for lanes 0-31, 64 + 16 mt + r
            // for lanes 32-63).  The index is their count c, a thermometer
            // code: bit p of c = (sum over j >= 1 of [c >= j 2^p]) mod 2, the
            // xor of the masks k with k + 1 a multiple of 2^p.  Each plane's
            // two block words come from scalar xors, written into lane
            // 16 mt + r.
            uint64_t ge[(1 << BQ) - 1];
#pragma unroll
            for (int k = 0; k < (1 << BQ) - 1; ++k) ge[k] = __ballot(y >= cbv.b[k]);
            if constexpr (EDEN) {
              float cv = cbv.c[0];
#pragma unroll
              for (int k = 0; k < (1 << BQ) - 1; ++k) cv = select_mask(ge[k], cbv.c[k + 1], cv);
              yc[nt] = fmaf(y, cv, yc[nt]);
            }
#pragma unroll
            for (int p = 0; p < BQ; ++p) {
              uint64_t m = 0;
#pragma unroll
              for (int k = 0; k < (1 << BQ) - 1; ++k)
                if (((k + 1) & ((1 << p) - 1)) == 0) m ^= ge[k];
              const uint32_t mlo = (uint32_t)m, mhi = (uint32_t)(m >> 32);
              // the mask may come straight from a VALU compare (one plane: m
              // is the comparison itself); a writelane reading an SGPR that a
              // VALU instruction has just written needs wait states, which the
              // compiler does not insert in front of inline asm
              if (p == 0)
                asm volatile("s_nop 4\n\tv_writelane_b32 %0, %2, %4\n\tv_writelane_b32 %1, %3, %4"
                             : "+v"(vlo[p]), "+v"(vhi[p])
                             : "s"(mlo), "s"(mhi), "i"(16 * mt + r));
              else
                asm volatile("v_writelane_b32 %0, %2, %4\n\tv_writelane_b32 %1, %3, %4"
                             : "+v"(vlo[p]), "+v"(vhi[p])
                             : "s"(mlo), "s"(mhi), "i"(16 * mt + r));
            }
            return;
          }
          // idx = #{k : y >= beta_k} is a thermometer code, so bit p of idx
          // is the xor of the comparisons k with k + 1 a multiple of 2^p (the
          // xors run on the lane masks).  Each plane word takes its bits in
          // ascending coordinate order as w = 2 w + bit (one carry-in add per
          // bit) and is bit-reversed once before the store.
          uint64_t ge[(1 << BQ) - 1];
          float chat = PROD ? csc[nt][0] : cbv.c[0];
#pragma unroll
          for (int k = 0; k < (1 << BQ) - 1; ++k) {
            ge[k] = ge_mask(y, PROD ? bsc[nt][k] : cbv.b[k]);
            chat = select_mask(ge[k], PROD ? csc[nt][k + 1] : cbv.c[k + 1], chat);
          }
          if constexpr (EDEN) yc[nt] = fmaf(y, chat, yc[nt]);
          uint64_t bit[BQ];
#pragma unroll
          for (int p = 0; p < BQ; ++p) {
            uint64_t x = 0;
#pragma unroll
            for (int k = 0; k < (1 << BQ) - 1; ++k)
              if (((k + 1) & ((1 << p) - 1)) == 0) x ^= ge[k];
            bit[p] = x;
            iw[nt][p][mt >> 1] = shift_in(iw[nt][p][mt >> 1], x);
          }
          if (!PROD) {
            if (vec[nt] < a.n) {
              // blocks shared with other vectors: an atomic for each bit
              // that changes (with a slot map), else one per bit
              uint32_t* wp = a.planes + (vrec >> 5) * (D * BQ) + (64 * h + 16 * mt + r) * BQ;
              const uint32_t sh = (uint32_t)(vrec & 31);
#pragma unroll
              for (int p = 0; p < BQ; ++p) {
                const uint32_t nb = (uint32_t)(bit[p] >> lane) & 1u;
                const bool change = SLOTS ? nb != ((oldw[r * BQ + p] >> sh) & 1u) : true;
                if (change) {
                  if (nb) atomicOr(wp + p, 1u << sh);
                  else atomicAnd(wp + p, ~(1u << sh));
                }
              }
            }
          }
          if (QJL) {
            const float d = y - chat;      // residual / ysc
            g2[nt] += d * d;
            _Float16 hi, lo;
            split_f16(d * rsc[nt], hi, lo);
            const int ks2 = 2 * mt + (r >> 3);
            rh[nt][ks2][r & 7] = hi;
            rl[nt][ks2][r & 7] = lo;
          }
    };
    f32x16 accA[NT], accB[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) accA[nt] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) mma(accA, 0, ks);
#pragma unroll
    for (int mt = 1; mt < 4; ++mt) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) accB[nt] = f32x16{};
      load_old(mt - 1);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if ((i & 1) == 0) mma(accB, mt, i >> 1);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) epi(accA, mt - 1, nt, i);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) accA[nt] = accB[nt];
    }
    load_old(3);
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) epi(accA, 3, nt, i);

    // ---- GEMM2 (QJL signs) ----
    uint32_t sw[NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) sw[nt][0] = sw[nt][1] = 0u;
    if (QJL) {
      // m = d: row tiles 0-3, lane half h collects sign words 2h, 2h + 1;
      // m = d / 2: row tiles 0-1, lane half h collects sign word h
#pragma unroll
      for (int it = 0; it < MW; ++it) {
        f32x16 acc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const half8 shi = fs[frag_index(it, ks, 0, lane)];
          const half8 slo = fs[frag_index(it, ks, 1, lane)];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            acc[nt] = mfma32x32x16(shi, rh[nt][ks], acc[nt]);
            acc[nt] = mfma32x32x16(slo, rh[nt][ks], acc[nt]);
            acc[nt] = mfma32x32x16(shi, rl[nt][ks], acc[nt]);
          }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
          for (int r = 0; r < 16; ++r)   // ascending coordinate order, reversed before the store
            sw[nt][it >> 1] = shift_in(sw[nt][it >> 1], ge_mask(acc[nt][r], 0.f));
        }
      }
    }

    // ---- store records ----
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float g = 0.f;
      if (QJL) {
        float t = g2[nt] + shfl_xor_f(g2[nt], 32);
        g = sqrtf(t) * ysc[nt];
      }
      if (!PROD) {
        if (vfast) {
          // lane L holds the words of coordinates L and 64 + L, planes contiguous
          uint32_t* base = a.planes + vblock * (D * BQ);
#pragma unroll
          for (int p = 0; p < BQ; ++p) {
            base[lane * BQ + p] = vlo[p];
            base[(64 + lane) * BQ + p] = vhi[p];
          }
        }
        float sv = nrm[nt];
        if constexpr (EDEN) {
          const float t = yc[nt] + shfl_xor_f(yc[nt], 32);    // <y, c[idx]>, y on the unit sphere
          sv = nrm[nt] > 0.f && t > 0.f ? nrm[nt] / t : 0.f;
        }
        if (vec[nt] < a.n && h == 0) a.scalars[a.slot ? a.slot[vec[nt]] : vec[nt]] = f16_bits(sv);
        continue;
      }
      // MSE-only key scalar: n, or with EDEN n / <y, c[idx]> (the sum over both
      // half-waves runs on every lane)
      float ks = nrm[nt];
      if constexpr (EDEN) {
        const float t = (yc[nt] + shfl_xor_f(yc[nt], 32)) * (ysc[nt] * ysc[nt]);
        ks = nrm[nt] > 0.f && t > 0.f ? nrm[nt] / t : 0.f;
      }
      if constexpr (QJL && MW == 2) {
        // lane half 0 writes groups 0 and 1 with sign words 0 and 1 (the
        // latter from lane half 1); lane half 1 writes groups 2 and 3
        const uint32_t s1 = __shfl_xor(sw[nt][0], 32, 64);
        if (vec[nt] < a.n) {
          const int64_t rec = a.slot ? a.slot[vec[nt]] : vec[nt];
          constexpr int RW = 4 * BQ + 2;
          uint32_t out[2 * BQ + 2];
#pragma unroll
          for (int p = 0; p < BQ; ++p) {
            out[p] = __builtin_bitreverse32(iw[nt][p][0]);
            out[BQ + 1 + p] = __builtin_bitreverse32(iw[nt][p][1]);
          }
          out[BQ] = __builtin_bitreverse32(sw[nt][0]);
          out[2 * BQ + 1] = __builtin_bitreverse32(s1);
          if (h == 1) {
#pragma unroll
            for (int p = 0; p < BQ; ++p) out[BQ + p] = __builtin_bitreverse32(iw[nt][p][1]);
          }
          uint2* dst = reinterpret_cast<uint2*>(a.planes + rec * RW + (h ? 2 * BQ + 2 : 0));
#pragma unroll
          for (int i = 0; i < BQ + 1; ++i)
            if (h == 0 || i < BQ) dst[i] = make_uint2(out[2 * i], out[2 * i + 1]);
          if (h == 0)
            reinterpret_cast<uint32_t*>(a.scalars)[rec] =
                (uint32_t)f16_bits(nrm[nt]) | ((uint32_t)f16_bits(g) << 16);
        }
        continue;
      }
      if (vec[nt] < a.n) {
        const int64_t rec = a.slot ? a.slot[vec[nt]] : vec[nt];
        // record order: word w of plane p at w * P + p; this lane owns words
        // 2h and 2h+1 of every plane, i.e. the 2P contiguous u32 from 2h * P
        uint32_t out[2 * P];
#pragma unroll
        for (int p = 0; p < BQ; ++p) {
          out[p] = __builtin_bitreverse32(iw[nt][p][0]);
          out[P + p] = __builtin_bitreverse32(iw[nt][p][1]);
        }
        if (QJL) {
          out[BQ] = __builtin_bitreverse32(sw[nt][0]);
          out[P + BQ] = __builtin_bitreverse32(sw[nt][1]);
        }
        uint2* dst = reinterpret_cast<uint2*>(a.planes + rec * (P * 4) + 2 * h * P);
#pragma unroll
        for (int i = 0; i < P; ++i) dst[i] = make_uint2(out[2 * i], out[2 * i + 1]);
        if (h == 0) {
          if (QJL) {
            reinterpret_cast<uint32_t*>(a.scalars)[rec] =
                (uint32_t)f16_bits(nrm[nt]) | ((uint32_t)f16_bits(g) << 16);
          } else {
            a.scalars[rec] = f16_bits(ks);
          }
        }
      }
    }
  }
}

template <bool PROD, bool QJL, int BQ, bool F16IN, bool HAD, int WAVES, bool EDEN = false, int MW = 4>
hipError_t launch_waves(const EncodeArgs& a, int cus, hipStream_t stream) {
  constexpr int NT = 1;
  // EDEN values always take the slot-capable form (one kernel for both)
  auto kern = MW != 4 ? encode_dense128<PROD, QJL, BQ, F16IN, NT, WAVES, HAD, false, false, MW>
              : EDEN ? encode_dense128<PROD, QJL, BQ, F16IN, NT, WAVES, HAD, !PROD, EDEN>
              : PROD || !a.slot ? encode_dense128<PROD, QJL, BQ, F16IN, NT, WAVES, HAD, false>
                                : encode_dense128<PROD, QJL, BQ, F16IN, NT, WAVES, HAD, !PROD>;
  const size_t lds = (QJL ? 2 : 1) * FRAGS * sizeof(half8);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t ntiles = (a.n + 32 * NT - 1) / (32 * NT);
  const int64_t want = (ntiles + WAVES - 1) / WAVES;
  const int blocks_per_cu = PROD ? 1 : 2;
  const int grid = (int)std::min<int64_t>(want, (int64_t)cus * blocks_per_cu);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * WAVES), lds, stream, a);
  return hipGetLastError();
}

// Workgroups of 8 waves share one copy of the fragments per compute unit; a
// small batch (under two tiles per compute unit, e.g. one appended token per
// sequence) takes one-wave workgroups instead, so that its tiles (and, for
// values written through a slot map, their per-bit atomics) spread over as
// many compute units as there are tiles.
template <bool PROD, bool QJL, int BQ, bool F16IN, bool HAD, int MW = 4>
hipError_t launch_one(const EncodeArgs& a, hipStream_t stream) {
  int dev = 0, cus = 256;
  hipGetDevice(&dev);
  hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int64_t ntiles = (a.n + 31) / 32;
  if (ntiles < 2 * (int64_t)cus) return launch_waves<PROD, QJL, BQ, F16IN, HAD, 1, false, MW>(a, cus, stream);
  return launch_waves<PROD, QJL, BQ, F16IN, HAD, 8, false, MW>(a, cus, stream);
}

// Prod keys with m = d / 2 QJL rows
template <bool F16IN, bool HAD>
hipError_t launch_prod_half(const EncodeArgs& a, hipStream_t stream) {
  switch (a.bq) {
    case 1: return launch_one<true, true, 1, F16IN, HAD, 2>(a, stream);
    case 2: return launch_one<true, true, 2, F16IN, HAD, 2>(a, stream);
    case 3: return launch_one<true, true, 3, F16IN, HAD, 2>(a, stream);
  }
  return hipErrorInvalidValue;
}

// EDEN-scaled MSE records (keys in the per-record layout, or values), b
// index bits; one launch shape (8-wave workgroups) for every batch size
template <bool PROD, bool F16IN, bool HAD>
hipError_t launch_eden(const EncodeArgs& a, hipStream_t stream) {
  int dev = 0, cus = 256;
  hipGetDevice(&dev);
  hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  switch (a.bq) {
    case 1: return launch_waves<PROD, false, 1, F16IN, HAD, 8, true>(a, cus, stream);
    case 2: return launch_waves<PROD, false, 2, F16IN, HAD, 8, true>(a, cus, stream);
    case 3: return launch_waves<PROD, false, 3, F16IN, HAD, 8, true>(a, cus, stream);
    case 4: return launch_waves<PROD, false, 4, F16IN, HAD, 8, true>(a, cus, stream);
  }
  return hipErrorInvalidValue;
}

// MSE-only keys: b index bits in the per-record layout
template <bool F16IN, bool HAD>
hipError_t launch_mse_keys(const EncodeArgs& a, hipStream_t stream) {
  switch (a.bq) {
    case 1: return launch_one<true, false, 1, F16IN, HAD>(a, stream);
    case 2: return launch_one<true, false, 2, F16IN, HAD>(a, stream);
    case 3: return launch_one<true, false, 3, F16IN, HAD>(a, stream);
    case 4: return launch_one<true, false, 4, F16IN, HAD>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <bool HAD>
hipError_t launch_rot(const EncodeArgs& a, hipStream_t stream) {
  if (a.eden) {
    if (a.prod) return a.f16_in ? launch_eden<true, true, HAD>(a, stream) : launch_eden<true, false, HAD>(a, stream);
    return a.f16_in ? launch_eden<false, true, HAD>(a, stream) : launch_eden<false, false, HAD>(a, stream);
  }
  if (a.prod && !a.qjl) return a.f16_in ? launch_mse_keys<true, HAD>(a, stream) : launch_mse_keys<false, HAD>(a, stream);
  if (a.prod && a.m == D / 2)
    return a.f16_in ? launch_prod_half<true, HAD>(a, stream) : launch_prod_half<false, HAD>(a, stream);
  if (a.prod) {
    if (a.f16_in) {
      switch (a.bq) {
        case 1: return launch_one<true, true, 1, true, HAD>(a, stream);
        case 2: return launch_one<true, true, 2, true, HAD>(a, stream);
        case 3: return launch_one<true, true, 3, true, HAD>(a, stream);
      }
    } else {
      switch (a.bq) {
        case 1: return launch_one<true, true, 1, false, HAD>(a, stream);
        case 2: return launch_one<true, true, 2, false, HAD>(a, stream);
        case 3: return launch_one<true, true, 3, false, HAD>(a, stream);
      }
    }
  } else {
    if (a.f16_in) {
      switch (a.bq) {
        case 1: return launch_one<false, false, 1, true, HAD>(a, stream);
        case 2: return launch_one<false, false, 2, true, HAD>(a, stream);
        case 3: return launch_one<false, false, 3, true, HAD>(a, stream);
        case 4: return launch_one<false, false, 4, true, HAD>(a, stream);
      }
    } else {
      switch (a.bq) {
        case 1: return launch_one<false, false, 1, false, HAD>(a, stream);
        case 2: return launch_one<false, false, 2, false, HAD>(a, stream);
        case 3: return launch_one<false, false, 3, false, HAD>(a, stream);
        case 4: return launch_one<false, false, 4, false, HAD>(a, stream);
      }
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_encode_dense128(const EncodeArgs& a, hipStream_t stream) {
  return a.had ? launch_rot<true>(a, stream) : launch_rot<false>(a, stream);
}

}  // namespace tq
