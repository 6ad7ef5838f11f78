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
#include <cmath>

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
constexpr int64_t VSCAN_MAX = 4096;    // value records a small-batch workgroup scans for shared blocks

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
// Values of a tile that is not one aligned, fully valid 32-record block (a
// slot map in any order, a ragged tail) set or clear their bits in the
// epilogue, one atomic or / and per plane word with nothing read first (a
// record's bit has one writer; other records of the block may be written at
// the same time).
// EDEN: an MSE record stores the unbiased per-vector scale n / <y, c[idx]>
// instead of n (EDEN's scale; DRIVE's at one bit).
// MW: QJL sign words per key record, m / 32 (4: m = d; 2: m = d / 2, whose
// record holds for each 32-coordinate group w the index words, then sign word
// w if w < 2).
template <bool PROD, bool QJL, int BQ, bool F16IN, int NT, int WAVES, bool HAD, bool EDEN = false, int MW = 4>
__global__ __launch_bounds__(64 * WAVES, 1) void encode_dense128(EncodeArgs a) {
  static_assert(PROD || !QJL, "values carry no QJL bits");
  static_assert(!(EDEN && QJL), "the scale replaces the norm of MSE records only");
  static_assert(MW == 4 || (QJL && MW == 2), "m = d / 2 is a prod-key form");
  extern __shared__ half8 lds[];
  half8* fpi = lds;
  half8* fs = lds + FRAGS;
  // values, one tile per workgroup: the tile's plane words [32][2 halves][BQ][2],
  // records, same-block masks and shared flags, for the bit writes after the tile
  uint32_t* vbits = reinterpret_cast<uint32_t*>(lds + FRAGS);
  int64_t* vrecs = reinterpret_cast<int64_t*>(vbits + 32 * 2 * BQ * 2);
  uint32_t* vmask = reinterpret_cast<uint32_t*>(vrecs + 32);
  int* vshared = reinterpret_cast<int*>(vmask + 32);
  build_frags<64 * WAVES>(fpi, a.pi, PI_SCALE, HAD ? a.eps : nullptr);
  if (QJL) build_frags<64 * WAVES, MW == 2>(fs, a.s, 1.f);
  if (!PROD && threadIdx.x < 32) vshared[threadIdx.x] = 0;
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

  // tiles: consecutive per workgroup, or (interleave) one per workgroup in
  // wave 0 first, so that a small batch takes one tile per workgroup while all
  // its waves build the fragments
  // (values: `split` workgroups share each small-batch tile, each computing
  // it and writing its share of the tile's words)
  const int split = a.interleave ? a.split : 1;
  const int part = (int)(blockIdx.x % split);
  const int64_t wg = blockIdx.x / split, ngroups = gridDim.x / split;
  if constexpr (!PROD) {
    // one tile per workgroup (values, small batch): while wave 0 encodes it,
    // the other waves look for records of the call outside the tile that share
    // a block with it (the tile's records from the slot map, lane u of each
    // wave holding record u)
    if (a.interleave && wave > 0 && wg < ntiles && a.n <= VSCAN_MAX) {
      const int64_t tile0 = wg * 32;
      const int64_t iu = tile0 + (lane & 31);
      const int64_t mine = iu < a.n ? (a.slot ? a.slot[iu] : iu) : -1;
      // 64-record chunks per wave, the same trip count on every lane (the
      // shuffles read lanes 0..31)
      for (int64_t i0 = 64 * (int64_t)(wave - 1); i0 < a.n; i0 += 64 * (WAVES - 1)) {
        const int64_t i = i0 + lane;
        const int64_t r = i < a.n && (i < tile0 || i >= tile0 + 32) ? (a.slot ? a.slot[i] : i) : -1;
        const bool lr = (uint64_t)r < (uint64_t)a.records;
        for (int u = 0; u < 32; ++u) {
          const int64_t q = __shfl((long long)mine, u, 64);
          if (lr && (uint64_t)q < (uint64_t)a.records && (q >> 5) == (r >> 5)) vshared[u] = 1;
        }
      }
    }
  }
  for (int64_t tile = a.interleave ? wg + ngroups * wave : (int64_t)blockIdx.x * WAVES + wave;
       tile < ntiles; tile += stride) {
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
      // this lane's record (-1 past n)
      vrec = vec[0] < a.n ? (a.slot ? a.slot[vec[0]] : vec[0]) : -1;
      const bool mine = vec[0] < a.n && vrec == r0 + v;
      // whole-block stores only for a block inside the cache's capacity
      vfast = (r0 % 32) == 0 && r0 >= 0 && r0 + 32 <= a.records && __all(mine);
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
              // lane 16 mt + r takes the block's words of this coordinate (a
              // plain select: the mask may come straight from a VALU compare,
              // and the compiler places whatever wait states that needs)
              const bool here = lane == 16 * mt + r;
              vlo[p] = here ? mlo : vlo[p];
              vhi[p] = here ? mhi : vhi[p];
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
          if (!PROD && !(a.interleave && wave == 0) && vec[nt] < a.n && (uint64_t)vrec < (uint64_t)a.records) {
            // this record's bit of each plane word of coordinate 64 h + 16 mt + r:
            // one atomic or / and per word, nothing read first; the 64 lanes
            // of each atomic hit 64 different words of 32 records' blocks
            // (with one tile per workgroup, wave 0's tile, the whole workgroup
            // issues them after the tile instead)
            uint32_t* wp = a.planes + (vrec >> 5) * (D * BQ) + (64 * h + 16 * mt + r) * BQ;
            const uint32_t sh = 1u << (uint32_t)(vrec & 31);
#pragma unroll
            for (int p = 0; p < BQ; ++p) {
              if ((bit[p] >> lane) & 1u) atomicOr(wp + p, sh);
              else atomicAnd(wp + p, ~sh);
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
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if ((i & 1) == 0) mma(accB, mt, i >> 1);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) epi(accA, mt - 1, nt, i);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) accA[nt] = accB[nt];
    }
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
        if (vfast && part == 0) {
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
        if (vec[nt] < a.n && h == 0 && part == 0) {
          const int64_t rec = a.slot ? a.slot[vec[nt]] : vec[nt];
          if ((uint64_t)rec < (uint64_t)a.records) a.scalars[rec] = f16_bits(sv);
        }
        if (a.interleave && wave == 0) {
#pragma unroll
          for (int p = 0; p < BQ; ++p)
#pragma unroll
            for (int w = 0; w < 2; ++w) vbits[((v * 2 + h) * BQ + p) * 2 + w] = __builtin_bitreverse32(iw[nt][p][w]);
          if (h == 0) vrecs[v] = vfast ? -1 : vrec;     // an aligned block is already written
        }
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
        const int64_t rec = vec[nt] < a.n ? (a.slot ? a.slot[vec[nt]] : vec[nt]) : -1;
        if ((uint64_t)rec < (uint64_t)a.records) {
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
      const int64_t rec = vec[nt] < a.n ? (a.slot ? a.slot[vec[nt]] : vec[nt]) : -1;
      if ((uint64_t)rec < (uint64_t)a.records) {
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
  if constexpr (!PROD) {
    // One tile per workgroup (wave 0's): the workgroup writes the tile's value
    // bits.  A block that no record of the call outside this tile touches
    // (found by scanning the call's records, for calls of up to VSCAN_MAX) has
    // this workgroup as its only writer: one thread per plane word reads it,
    // sets or clears the bits of every tile record in the block, and stores it.
    // Other blocks take one atomic or / and per record and word.
    if (a.interleave && wg < ntiles) {
      constexpr int NW = D * BQ;    // plane words of a block
      __syncthreads();              // wave 0's vbits, vrecs
      const int t = threadIdx.x;
      auto live = [&](int64_t r) { return (uint64_t)r < (uint64_t)a.records; };
      if (t < 32) {
        const int64_t r = vrecs[t];
        uint32_t m = 0;
        if (live(r)) {
          for (int u = 0; u < 32; ++u)
            if (live(vrecs[u]) && (vrecs[u] >> 5) == (r >> 5)) m |= 1u << u;
        }
        vmask[t] = m;       // the tile's records in the same block (itself included)
      }
      __syncthreads();
      const bool scan = a.n <= VSCAN_MAX;
      // this workgroup's share of the tile's words (split = 1, 2, 4 or 8), every
      // thread's words in flight together: reads first, then the writes
      constexpr int PER = 32 * NW / (64 * WAVES * 8);
      static_assert(PER * 64 * WAVES * 8 == 32 * NW, "a whole number of words per thread");
      const int per = PER * (8 / split);
      const int fbase = part * (32 * NW / split);
      uint32_t old[8 * PER];
#pragma unroll
      for (int k = 0; k < 8 * PER; ++k) {
        if (k >= per) break;
        const int f = fbase + t + 64 * WAVES * k, u = f & 31, w = f >> 5;
        const int64_t rec = vrecs[u];
        const bool rmw = live(rec) && scan && !vshared[u] && (int)__builtin_ctz(vmask[u]) == u;
        old[k] = rmw ? a.planes[(rec >> 5) * NW + w] : 0u;
      }
#pragma unroll
      for (int k = 0; k < 8 * PER; ++k) {
        if (k >= per) break;
        const int f = fbase + t + 64 * WAVES * k, u = f & 31, w = f >> 5;
        const int64_t rec = vrecs[u];
        if (!live(rec)) continue;
        const int c = w / BQ, p = w - c * BQ;
        const int vi = (c >> 6) * BQ * 2 + p * 2 + ((c >> 5) & 1);   // (half, plane, word) within a record's vbits
        uint32_t* wp = a.planes + (rec >> 5) * NW + w;
        if (scan && !vshared[u]) {
          const uint32_t m = vmask[u];
          if ((int)__builtin_ctz(m) != u) continue;      // the block's first tile record writes its words
          uint32_t word = old[k];
          for (uint32_t mm = m; mm; mm &= mm - 1) {
            const int u2 = __builtin_ctz(mm);
            const uint32_t bit = 1u << (uint32_t)(vrecs[u2] & 31);
            word = (vbits[u2 * 4 * BQ + vi] >> (c & 31)) & 1u ? word | bit : word & ~bit;
          }
          *wp = word;
        } else {
          const uint32_t bit = 1u << (uint32_t)(rec & 31);
          if ((vbits[u * 4 * BQ + vi] >> (c & 31)) & 1u) atomicOr(wp, bit);
          else atomicAnd(wp, ~bit);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Small batches (an append of a few hundred vectors, the 4096-vector tiny
// workload): one 32-vector tile per workgroup of four waves, wave mt computing
// row tile mt of both products, so a tile takes a quarter of the matrix-core
// chain it takes in one wave, and no workgroup builds a shared fragment copy:
// each lane splits its own 64 entries of the matrix rows it needs (16 KB of
// fp32 per wave and matrix, L2 hits after the first workgroup).  The
// arithmetic is the one of encode_dense128 (same products in the same order,
// same quantiser), so records match the large-batch path; only the norm of the
// residual is summed in another order.
//   keys:   the waves exchange the residual's fp16 split (the B operand of the
//           sign product) and their 16-bit parts of the plane words in LDS;
//           wave 0 writes the records.
//   values: an aligned, fully valid 32-record block is written whole (each
//           wave its 32 coordinates); otherwise every wave updates its
//           coordinates' words of the tile's records: a block that no other
//           record of the call touches (found by the four waves scanning the
//           call's records, for calls of up to VSCAN_MAX) by reading,
//           changing and storing whole words, other blocks with one atomic
//           or / and per record and word.
constexpr int ROWS_THREADS = 256;

template <int BQ>
struct RowsLds {
  half8 res[8][2][64];             // keys: residual split, [k step][hi, lo][lane]
  uint32_t part[4][BQ + 1][64];    // keys: 16-bit parts of the index (and sign) words, [row tile][plane][lane]
  float g2[4][64];                 // keys: partial squared residual norms
  uint32_t vb[4][32][2][BQ];       // values: [row tile][record][lane half][plane] bits r of coordinates 64 h + 16 mt + r
  int64_t vrecs[32];               // values: the tile's records (-1: none)
  uint32_t vmask[32];              // values: tile records in the same block
  uint32_t vshmask;                // values: tile records whose block another record of the call shares
};

template <bool PROD, bool QJL, int BQ, bool F16IN, bool HAD, int MW = 4>
__global__ __launch_bounds__(ROWS_THREADS, 1) void encode_rows128(EncodeArgs a) {
  static_assert(PROD || !QJL, "values carry no QJL bits");
  static_assert(MW == 4 || (QJL && MW == 2), "m = d / 2 is a prod-key form");
  constexpr int P = QJL ? BQ + 1 : BQ;
  __shared__ RowsLds<BQ> L;
  const int lane = threadIdx.x & 63;
  const int mt = threadIdx.x >> 6;      // the wave's row tile
  const int v = lane & 31, h = lane >> 5;
  const int64_t tile = blockIdx.x;
  const int64_t vec = tile * 32 + v;
  const bool valid = vec < a.n;
  if (!PROD && threadIdx.x == 0) L.vshmask = 0u;

  // ---- operands: x (coordinates 64 h .. 64 h + 63 of vector v) and this
  // lane's rows of Pi (and S), all requested before any is used ----
  float4 pm[16], sm[16];
  {
    const int row = row_coord(v, mt);
    const float4* src = reinterpret_cast<const float4*>(HAD ? a.eps + 64 * h : a.pi + row * D + 64 * h);
#pragma unroll
    for (int i = 0; i < 16; ++i) pm[i] = src[i];
  }
  if constexpr (QJL) {
    if (mt < MW) {
      const int row = MW == 2 ? row_half(v, mt) : row_coord(v, mt);
      const float4* src = reinterpret_cast<const float4*>(a.s + row * D + 64 * h);
#pragma unroll
      for (int i = 0; i < 16; ++i) sm[i] = src[i];
    }
  }
  half8 xh[8], xl[8];
  float ysc, inv, nrm;
  if (F16IN) {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const _Float16*>(a.x) + (valid ? vec : 0) * a.ld_x + 64 * h);
    float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      half8 hv = __builtin_bit_cast(half8, valid ? src[ks] : make_uint4(0, 0, 0, 0));
      xh[ks] = hv;
#pragma unroll
      for (int e = 0; e < 8; ++e) s4[e & 3] += (float)hv[e] * (float)hv[e];
    }
    float s2 = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    s2 += shfl_xor_f(s2, 32);
    const float n = sqrtf(s2);
    nrm = n;
    ysc = n > 0.f ? (HAD ? HAD_SCALE : 1.f) / (n * PI_SCALE) : 1.f;
    inv = n > 0.f ? (n * PI_SCALE) / (HAD ? HAD_SCALE : 1.f) : 1.f;
  } else {
    const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(a.x) + (valid ? vec : 0) * a.ld_x + 64 * h);
    float xv[64];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float4 w = valid ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      xv[4 * i] = w.x; xv[4 * i + 1] = w.y; xv[4 * i + 2] = w.z; xv[4 * i + 3] = w.w;
    }
    float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 64; ++i) s4[i & 3] += xv[i] * xv[i];
    float s2 = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    s2 += shfl_xor_f(s2, 32);
    const float n = sqrtf(s2);
    const float un = n > 0.f ? U_SCALE / n : 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        _Float16 hi, lo;
        split_f16(xv[8 * ks + e] * un, hi, lo);
        xh[ks][e] = hi;
        xl[ks][e] = lo;
      }
    }
    nrm = n;
    ysc = (HAD ? HAD_SCALE : 1.f) / (U_SCALE * PI_SCALE);
    inv = (U_SCALE * PI_SCALE) / (HAD ? HAD_SCALE : 1.f);
  }

  // ---- values: this lane's record and the tile's block case; the records
  // of the call the scan for shared blocks compares (first chunks requested
  // now, compared after the products); the words a single writer will
  // rewrite, requested before the products as well ----
  constexpr int NQ = 16 * BQ / 4;    // 16-byte groups of a lane's run of plane words
  constexpr int SPRE = 4;            // scan chunks requested up front
  int64_t vrec = -1;
  bool vfast = false;
  int64_t vblock = 0;
  int64_t spre[SPRE];
  uint4 w4[NQ];
  const bool scan = a.n <= VSCAN_MAX;
  if constexpr (!PROD) {
#pragma unroll
    for (int c = 0; c < SPRE; ++c) {
      const int64_t i = 64 * (int64_t)(mt + 4 * c) + lane;
      spre[c] = i < a.n ? (a.slot ? a.slot[i] : i) : -1;
    }
    const int64_t r0 = a.slot ? a.slot[tile * 32 < a.n ? tile * 32 : 0] : tile * 32;
    vrec = valid ? (a.slot ? a.slot[vec] : vec) : -1;
    const bool mine = valid && vrec == r0 + v;
    vfast = (r0 % 32) == 0 && r0 >= 0 && r0 + 32 <= a.records && __all(mine);
    vblock = r0 / 32;
    if (mt == 0 && h == 0) L.vrecs[v] = vfast || (uint64_t)vrec >= (uint64_t)a.records ? -1 : vrec;
    __syncthreads();   // vshmask cleared, vrecs set
    // lane (record u = lane % 32, half hh = lane / 32) owns the 16 BQ words of
    // coordinates 64 hh + 16 mt .. + 15 in u's block
    const int64_t rec = L.vrecs[lane & 31];
    if (!vfast && scan && rec >= 0) {
      const uint4* wp = reinterpret_cast<const uint4*>(a.planes + (rec >> 5) * (D * BQ) + (64 * h + 16 * mt) * BQ);
#pragma unroll
      for (int q = 0; q < NQ; ++q) w4[q] = wp[q];
    }
  }

  // ---- A fragments of this wave's row tile (and of its sign row tile) ----
  half8 ph[8], pl[8], sh[8], sl[8];
  {
    const int row = row_coord(v, mt);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const float* f = reinterpret_cast<const float*>(&pm[2 * ks]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float val = f[e];
        if (HAD) val = (__popc(row & (64 * h + 8 * ks + e)) & 1) ? -val : val;
        _Float16 hi, lo;
        split_f16(val * PI_SCALE, hi, lo);
        ph[ks][e] = hi;
        pl[ks][e] = lo;
      }
    }
  }
  if constexpr (QJL) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const float* f = reinterpret_cast<const float*>(&sm[2 * ks]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        _Float16 hi, lo;
        split_f16(mt < MW ? f[e] : 0.f, hi, lo);
        sh[ks][e] = hi;
        sl[ks][e] = lo;
      }
    }
  }

  // ---- GEMM1, row tile mt ----
  f32x16 acc = f32x16{};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    acc = mfma32x32x16(ph[ks], xh[ks], acc);
    if (!HAD) acc = mfma32x32x16(pl[ks], xh[ks], acc);   // +-16 has no lo part
    if (!F16IN) acc = mfma32x32x16(ph[ks], xl[ks], acc);
  }

  // ---- quantise, pack, residual (as the large-batch epilogue) ----
  Codebook cbv;
#pragma unroll
  for (int k = 0; k < (1 << BQ); ++k) asm volatile("v_mov_b32 %0, %1" : "=v"(cbv.c[k]) : "s"(a.cb.c[k]));
#pragma unroll
  for (int k = 0; k < (1 << BQ) - 1; ++k) asm volatile("v_mov_b32 %0, %1" : "=v"(cbv.b[k]) : "s"(a.cb.b[k]));
  float bsc[(1 << BQ) - 1], csc[1 << BQ];
  const float rsc = R_SCALE * ysc;
  if (PROD) {
#pragma unroll
    for (int k = 0; k < (1 << BQ) - 1; ++k) bsc[k] = cbv.b[k] * inv;
#pragma unroll
    for (int k = 0; k < (1 << BQ); ++k) csc[k] = cbv.c[k] * inv;
  }
  uint32_t iw[BQ];
  uint32_t vlo[BQ], vhi[BQ];
#pragma unroll
  for (int p = 0; p < BQ; ++p) iw[p] = vlo[p] = vhi[p] = 0u;
  half8 rh[2], rl[2];
  float g2 = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float y = PROD ? acc[r] : acc[r] * ysc;
    if (!PROD && vfast) {
      // ballots of [y >= beta_k]; the xors of the thermometer code give each
      // plane's two block words of coordinate 16 mt + r, kept by lane 16 mt + r
      uint64_t ge[(1 << BQ) - 1];
#pragma unroll
      for (int k = 0; k < (1 << BQ) - 1; ++k) ge[k] = __ballot(y >= cbv.b[k]);
#pragma unroll
      for (int p = 0; p < BQ; ++p) {
        uint64_t m = 0;
#pragma unroll
        for (int k = 0; k < (1 << BQ) - 1; ++k)
          if (((k + 1) & ((1 << p) - 1)) == 0) m ^= ge[k];
        const bool here = lane == 16 * mt + r;
        vlo[p] = here ? (uint32_t)m : vlo[p];
        vhi[p] = here ? (uint32_t)(m >> 32) : vhi[p];
      }
      continue;
    }
    uint64_t ge[(1 << BQ) - 1];
    float chat = PROD ? csc[0] : cbv.c[0];
#pragma unroll
    for (int k = 0; k < (1 << BQ) - 1; ++k) {
      ge[k] = ge_mask(y, PROD ? bsc[k] : cbv.b[k]);
      chat = select_mask(ge[k], PROD ? csc[k + 1] : cbv.c[k + 1], chat);
    }
#pragma unroll
    for (int p = 0; p < BQ; ++p) {
      uint64_t x = 0;
#pragma unroll
      for (int k = 0; k < (1 << BQ) - 1; ++k)
        if (((k + 1) & ((1 << p) - 1)) == 0) x ^= ge[k];
      iw[p] = shift_in(iw[p], x);
    }
    if (QJL) {
      const float d = y - chat;      // residual / ysc
      g2 += d * d;
      _Float16 hi, lo;
      split_f16(d * rsc, hi, lo);
      rh[r >> 3][r & 7] = hi;
      rl[r >> 3][r & 7] = lo;
    }
  }
  // the 16 bits of this row tile, bit r = coordinate 64 h + 16 mt + r, at
  // bit 16 (mt % 2) + r of plane word 2 h + mt / 2
  auto place = [&](uint32_t w16) { return (mt & 1) ? __builtin_bitreverse32(w16) : __builtin_bitreverse32(w16) >> 16; };

  if constexpr (PROD) {
#pragma unroll
    for (int p = 0; p < BQ; ++p) L.part[mt][p][lane] = place(iw[p]);
    if constexpr (QJL) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        L.res[2 * mt + j][0][lane] = rh[j];
        L.res[2 * mt + j][1][lane] = rl[j];
      }
      L.g2[mt][lane] = g2;
    }
    __syncthreads();
    // ---- GEMM2 (QJL signs), row tile mt of S ----
    if constexpr (QJL) {
      if (mt < MW) {
        f32x16 acc2 = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const half8 bh = L.res[ks][0][lane], bl = L.res[ks][1][lane];
          acc2 = mfma32x32x16(sh[ks], bh, acc2);
          acc2 = mfma32x32x16(sl[ks], bh, acc2);
          acc2 = mfma32x32x16(sh[ks], bl, acc2);
        }
        uint32_t sw = 0u;
#pragma unroll
        for (int r = 0; r < 16; ++r) sw = shift_in(sw, ge_mask(acc2[r], 0.f));
        L.part[mt][BQ][lane] = place(sw);
      }
      __syncthreads();
    }
    if (mt != 0) return;
    // ---- wave 0: the records ----
    uint32_t wd[P][2];
#pragma unroll
    for (int p = 0; p < BQ; ++p)
#pragma unroll
      for (int j = 0; j < 2; ++j) wd[p][j] = L.part[2 * j][p][lane] | L.part[2 * j + 1][p][lane];
    float g = 0.f;
    if constexpr (QJL) {
      if (MW == 4) {
#pragma unroll
        for (int j = 0; j < 2; ++j) wd[BQ][j] = L.part[2 * j][BQ][lane] | L.part[2 * j + 1][BQ][lane];
      } else {
        // m = d / 2: sign word hh from row tiles 0, 1 of lane half hh
        const int o = lane ^ 32;
        wd[BQ][0] = L.part[0][BQ][lane] | L.part[1][BQ][lane];
        wd[BQ][1] = L.part[0][BQ][o] | L.part[1][BQ][o];
      }
      float t = ((L.g2[0][lane] + L.g2[1][lane]) + (L.g2[2][lane] + L.g2[3][lane]));
      t += shfl_xor_f(t, 32);
      g = sqrtf(t) * ysc;
    }
    const int64_t rec = valid ? (a.slot ? a.slot[vec] : vec) : -1;
    if ((uint64_t)rec >= (uint64_t)a.records) return;
    if constexpr (QJL && MW == 2) {
      // per coordinate group: the index words, then sign word w for w < 2;
      // lane half 0 writes groups 0 and 1, lane half 1 groups 2 and 3
      constexpr int RW = 4 * BQ + 2;
      uint32_t out[2 * BQ + 2];
#pragma unroll
      for (int p = 0; p < BQ; ++p) {
        out[p] = wd[p][0];
        out[BQ + 1 + p] = wd[p][1];
      }
      out[BQ] = wd[BQ][0];
      out[2 * BQ + 1] = wd[BQ][1];
      if (h == 1) {
#pragma unroll
        for (int p = 0; p < BQ; ++p) out[BQ + p] = wd[p][1];
      }
      uint2* dst = reinterpret_cast<uint2*>(a.planes + rec * RW + (h ? 2 * BQ + 2 : 0));
#pragma unroll
      for (int i = 0; i < BQ + 1; ++i)
        if (h == 0 || i < BQ) dst[i] = make_uint2(out[2 * i], out[2 * i + 1]);
    } else {
      // word w of plane p at w * P + p: this lane owns words 2 h and 2 h + 1
      uint32_t out[2 * P];
#pragma unroll
      for (int p = 0; p < P; ++p) {
        out[p] = wd[p][0];
        out[P + p] = wd[p][1];
      }
      uint2* dst = reinterpret_cast<uint2*>(a.planes + rec * (P * 4) + 2 * h * P);
#pragma unroll
      for (int i = 0; i < P; ++i) dst[i] = make_uint2(out[2 * i], out[2 * i + 1]);
    }
    if (h == 0) {
      if (QJL)
        reinterpret_cast<uint32_t*>(a.scalars)[rec] = (uint32_t)f16_bits(nrm) | ((uint32_t)f16_bits(g) << 16);
      else
        a.scalars[rec] = f16_bits(nrm);
    }
  } else {
    constexpr int NW = D * BQ;    // plane words of a value block
    if (mt == 0 && h == 0 && valid && (uint64_t)vrec < (uint64_t)a.records) a.scalars[vrec] = f16_bits(nrm);
    if (vfast) {
      // lane 16 mt + r holds the words of coordinates 16 mt + r and 64 + 16 mt + r
      if ((lane >> 4) == mt) {
        uint32_t* base = a.planes + vblock * NW;
#pragma unroll
        for (int p = 0; p < BQ; ++p) {
          base[lane * BQ + p] = vlo[p];
          base[(64 + lane) * BQ + p] = vhi[p];
        }
      }
      return;
    }
    if (scan) {
      // records of the call outside the tile that share a block with it:
      // each lane compares its record's block with the tile's 32 (LDS
      // broadcasts) and ors the hits into one mask
      const int64_t tile0 = tile * 32;
      int64_t tb[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const int64_t q = L.vrecs[u];
        tb[u] = q >= 0 ? q >> 5 : -1;
      }
      uint32_t hit = 0u;
      for (int c = 0; 64 * (int64_t)(mt + 4 * c) < a.n; ++c) {
        const int64_t i = 64 * (int64_t)(mt + 4 * c) + lane;
        int64_t r = -1;
#pragma unroll
        for (int k = 0; k < SPRE; ++k)
          if (k == c) r = spre[k];
        if (c >= SPRE) r = i < a.n ? (a.slot ? a.slot[i] : i) : -1;
        if (i >= tile0 && i < tile0 + 32) r = -1;
        if ((uint64_t)r < (uint64_t)a.records) {
          const int64_t blk = r >> 5;
#pragma unroll
          for (int u = 0; u < 32; ++u) hit |= blk == tb[u] ? 1u << u : 0u;
        }
      }
      if (hit) atomicOr(&L.vshmask, hit);
    }
#pragma unroll
    for (int p = 0; p < BQ; ++p) L.vb[mt][v][h][p] = __builtin_bitreverse32(iw[p]) >> 16;
    if (threadIdx.x < 32) {
      const int64_t r = L.vrecs[threadIdx.x];
      uint32_t m = 0;
      if (r >= 0) {
        for (int u = 0; u < 32; ++u)
          if (L.vrecs[u] >= 0 && (L.vrecs[u] >> 5) == (r >> 5)) m |= 1u << u;
      }
      L.vmask[threadIdx.x] = m;
    }
    __syncthreads();
    const int u = lane & 31, hh = lane >> 5;
    const int64_t rec = L.vrecs[u];
    if (rec < 0) return;
    const uint32_t m = L.vmask[u];
    uint32_t* wp = a.planes + (rec >> 5) * NW + (64 * hh + 16 * mt) * BQ;
    if (scan && !((L.vshmask >> u) & 1u)) {
      // the block's first tile record merges the bits of every tile record
      // in the block into the words it read and stores them
      if ((int)__builtin_ctz(m) != u) return;
      for (uint32_t mm = m; mm; mm &= mm - 1) {
        const int u2 = __builtin_ctz(mm);
        const uint32_t bit = 1u << (uint32_t)(L.vrecs[u2] & 31);
        uint32_t bits[BQ];
#pragma unroll
        for (int p = 0; p < BQ; ++p) bits[p] = L.vb[mt][u2][hh][p];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int w = 4 * q + e, ci = w / BQ, p = w % BQ;
            uint32_t& word = e == 0 ? w4[q].x : e == 1 ? w4[q].y : e == 2 ? w4[q].z : w4[q].w;
            word = (bits[p] >> ci) & 1u ? word | bit : word & ~bit;
          }
        }
      }
#pragma unroll
      for (int q = 0; q < NQ; ++q) reinterpret_cast<uint4*>(wp)[q] = w4[q];
    } else {
      const uint32_t bit = 1u << (uint32_t)(rec & 31);
      uint32_t bits[BQ];
#pragma unroll
      for (int p = 0; p < BQ; ++p) bits[p] = L.vb[mt][u][hh][p];
#pragma unroll
      for (int w = 0; w < 16 * BQ; ++w) {
        const int ci = w / BQ, p = w % BQ;
        if ((bits[p] >> ci) & 1u) atomicOr(wp + w, bit);
        else atomicAnd(wp + w, ~bit);
      }
    }
  }
}

template <bool PROD, bool QJL, int BQ, bool F16IN, bool HAD, int MW = 4>
hipError_t launch_rows(const EncodeArgs& a, hipStream_t stream) {
  const int64_t ntiles = (a.n + 31) / 32;
  hipLaunchKernelGGL((encode_rows128<PROD, QJL, BQ, F16IN, HAD, MW>), dim3((unsigned)ntiles), dim3(ROWS_THREADS), 0,
                     stream, a);
  return hipGetLastError();
}

template <bool PROD, bool QJL, int BQ, bool F16IN, bool HAD, int WAVES, bool EDEN = false, int MW = 4>
hipError_t launch_waves(const EncodeArgs& a, int cus, hipStream_t stream) {
  constexpr int NT = 1;
  auto kern = encode_dense128<PROD, QJL, BQ, F16IN, NT, WAVES, HAD, EDEN, MW>;
  // fragments; values also the tile's plane words and records (one tile per workgroup)
  const size_t lds = (QJL ? 2 : 1) * FRAGS * sizeof(half8) + (PROD ? 0 : 32 * 2 * BQ * 2 * 4 + 32 * 8 + 32 * 8);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t ntiles = (a.n + 32 * NT - 1) / (32 * NT);
  const int blocks_per_cu = PROD ? 1 : 2;
  EncodeArgs b = a;
  // values in a small batch: 1, 2, 4 or 8 workgroups per tile, as the device
  // holds them, sharing the tile's scattered bit writes
  b.split = 1;
  if (!PROD && a.interleave && a.slot)    // (without a slot map at most the last tile is not one block)
    while (b.split < 8 && ntiles * b.split * 2 <= (int64_t)cus * blocks_per_cu) b.split *= 2;
  const int64_t want = a.interleave ? ntiles * b.split : (ntiles + WAVES - 1) / WAVES;
  const int grid = (int)std::min<int64_t>(want, (int64_t)cus * blocks_per_cu);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * WAVES), lds, stream, b);
  return hipGetLastError();
}

// Workgroups of 8 waves share one copy of the fragments per compute unit.  A
// small batch (under two tiles per compute unit, e.g. one appended token per
// sequence) takes the row-split kernel instead: one tile per four-wave
// workgroup, spread over as many compute units as there are tiles.
template <bool PROD, bool QJL, int BQ, bool F16IN, bool HAD, int MW = 4>
hipError_t launch_one(const EncodeArgs& a, hipStream_t stream) {
  int dev = 0, cus = 256;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int64_t ntiles = (a.n + 31) / 32;
  if (ntiles < 2 * (int64_t)cus) return launch_rows<PROD, QJL, BQ, F16IN, HAD, MW>(a, stream);
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
// index bits; 8-wave workgroups, one tile each for a small batch
template <bool PROD, bool F16IN, bool HAD>
hipError_t launch_eden(const EncodeArgs& a, hipStream_t stream) {
  int dev = 0, cus = 256;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  EncodeArgs b = a;
  b.interleave = (a.n + 31) / 32 < 2 * (int64_t)cus;   // small batches: one tile per workgroup
  switch (a.bq) {
    case 1: return launch_waves<PROD, false, 1, F16IN, HAD, 8, true>(b, cus, stream);
    case 2: return launch_waves<PROD, false, 2, F16IN, HAD, 8, true>(b, cus, stream);
    case 3: return launch_waves<PROD, false, 3, F16IN, HAD, 8, true>(b, cus, stream);
    case 4: return launch_waves<PROD, false, 4, F16IN, HAD, 8, true>(b, cus, stream);
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

// ---------------------------------------------------------------------------
// PolarQuant as stage 1 at d = 128 (FastVQ README, "PolarQuant Algorithm" in
// its recursive form; "TurboQuant Combination" for the QJL stage).
//
// GEMM1 is the one above, so lane (v, h) holds coordinates 64 h + i of vector
// v, i = 16 mt + r in register r of row tile mt.  The transform therefore runs
// inside the lane up to level 6 (its 64 coordinates), and level 7 combines the
// lane halves.  Level-1 angles come from atan2 of the pair; an angle above
// level 1 is coded without trigonometry, psi >= beta <=> P_b cos^2 beta >
// P_a sin^2 beta with P the squared lengths of its two children (strict, so two
// empty children give code 0, as atan2(0, 0) = 0 does).  Every decision is
// scale-free, so it runs on the raw accumulators.  The reconstruction walks
// back down with the centroid (cos, sin) pairs from the LDS, the residual
// y - y~ feeds GEMM2 exactly as the prod residual does.
// ---------------------------------------------------------------------------

namespace {

// OR code c (W bits) into a little-endian word stream at bit pos (constant
// after unrolling), spilling into the next word when it straddles.
template <int W, int N>
__device__ __forceinline__ void put_code(uint32_t (&w)[N], int pos, uint32_t c) {
  w[pos >> 5] |= c << (pos & 31);
  if ((pos & 31) + W > 32) w[(pos >> 5) + 1] |= c >> (32 - (pos & 31));
}
template <int W, int N>
__device__ __forceinline__ uint32_t get_code(const uint32_t (&w)[N], int pos) {
  uint32_t c = w[pos >> 5] >> (pos & 31);
  if ((pos & 31) + W > 32) c |= w[(pos >> 5) + 1] << (32 - (pos & 31));
  return c & ((1u << W) - 1);
}

// Code the NP angles of one upper level from the 2 NP squared lengths below
// them (children 2j, 2j+1 of angle j), into nibble slot OFF + j of uw, and
// form the squared lengths of this level.
template <int NP, int LI, int OFF, int KU>
__device__ __forceinline__ void polar_level(const float (&pin)[2 * NP], float (&pout)[NP], uint32_t (&uw)[4],
                                            const PolarBook& bk) {
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const float pa = pin[2 * j], pb = pin[2 * j + 1];
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < KU - 1; ++k) c += pb * bk.bc[LI][k] > pa * bk.bs[LI][k] ? 1u : 0u;
    uw[(OFF + j) >> 3] |= c << (4 * ((OFF + j) & 7));
    pout[j] = pa + pb;
  }
}

// Split NP lengths of one level into the 2 NP lengths below with the
// centroid pairs of the level's codes (nibble slots OFF + j of uw).
template <int NP, int LI, int OFF>
__device__ __forceinline__ void polar_split(const float (&rin)[NP], float (&rout)[2 * NP], const uint32_t (&uw)[4],
                                            const float2* tabu) {
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const uint32_t c = (uw[(OFF + j) >> 3] >> (4 * ((OFF + j) & 7))) & 15u;
    const float2 t = tabu[16 * LI + c];
    rout[2 * j] = rin[j] * t.x;
    rout[2 * j + 1] = rin[j] * t.y;
  }
}

// Nibble slots of a lane's upper codes (levels 2..6) and their offsets in the
// record's upper stream (level l starts at 64 - 128 / 2^(l-1); the lane half h
// holds the second half of each level's positions when h = 1).
constexpr int PL_LOCAL[5] = {0, 16, 24, 28, 30};
constexpr int PL_STREAM[5] = {0, 32, 48, 56, 60};
constexpr int PL_HALF[5] = {16, 8, 4, 2, 1};

template <int B1, int B, bool QJL, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 1) void polar_encode128(PolarArgs a) {
  constexpr int K1 = 1 << B1, KU = 1 << B;
  constexpr int P = 2 * B1 + 2 * B + (QJL ? 4 : 0);     // record words
  extern __shared__ half8 lds[];
  half8* fpi = lds;
  half8* fs = lds + FRAGS;
  float2* tab1 = reinterpret_cast<float2*>(lds + (QJL ? 2 : 1) * FRAGS);   // [16] level 1
  float2* tabu = tab1 + 16;                                                 // [6][16] levels 2..7
  build_frags<64 * WAVES>(fpi, a.pi, PI_SCALE, a.had ? a.eps : nullptr);
  if (QJL) build_frags<64 * WAVES>(fs, a.s, 1.f);
  polar_tables_to_lds(a.book, tab1);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int v = lane & 31;
  const int h = lane >> 5;
  const float hs = a.had ? HAD_SCALE : 1.f;
  const int64_t ntiles = (a.n + 31) / 32;
  for (int64_t tile = (int64_t)blockIdx.x * WAVES + wave; tile < ntiles; tile += (int64_t)gridDim.x * WAVES) {
    asm volatile("" ::: "memory");   // keep the fragment reads inside the loop
    const int64_t vec = tile * 32 + v;
    const bool valid = vec < a.n;
    // ---- load, norm, GEMM1 operands (fp32 inputs normalised, in hi + lo) ----
    half8 xh[8], xl[8];
    float nrm, ysc, inv;
    if (a.f16_in) {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const _Float16*>(a.x) +
                                                        (valid ? vec : 0) * a.ld_x + 64 * h);
      float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const half8 hv = __builtin_bit_cast(half8, valid ? src[ks] : make_uint4(0, 0, 0, 0));
        xh[ks] = hv;
#pragma unroll
        for (int e = 0; e < 8; ++e) s4[e & 3] += (float)hv[e] * (float)hv[e];
      }
      float s2 = (s4[0] + s4[1]) + (s4[2] + s4[3]);
      s2 += shfl_xor_f(s2, 32);
      nrm = sqrtf(s2);
      ysc = nrm > 0.f ? hs / (nrm * PI_SCALE) : 1.f;
      inv = nrm > 0.f ? (nrm * PI_SCALE) / hs : 1.f;
    } else {
      const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(a.x) +
                                                          (valid ? vec : 0) * a.ld_x + 64 * h);
      float xv[64];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float4 w = valid ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        xv[4 * i] = w.x; xv[4 * i + 1] = w.y; xv[4 * i + 2] = w.z; xv[4 * i + 3] = w.w;
      }
      float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 64; ++i) s4[i & 3] += xv[i] * xv[i];
      float s2 = (s4[0] + s4[1]) + (s4[2] + s4[3]);
      s2 += shfl_xor_f(s2, 32);
      nrm = sqrtf(s2);
      const float un = nrm > 0.f ? U_SCALE / nrm : 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          _Float16 hi, lo;
          split_f16(xv[8 * ks + e] * un, hi, lo);
          xh[ks][e] = hi;
          xl[ks][e] = lo;
        }
      }
      ysc = hs / (U_SCALE * PI_SCALE);
      inv = (U_SCALE * PI_SCALE) / hs;
    }
    // ---- GEMM1: all four row tiles (the transform needs the lane's 64 coordinates) ----
    f32x16 acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      acc[mt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const half8 ahi = fpi[frag_index(mt, ks, 0, lane)];
        const half8 alo = fpi[frag_index(mt, ks, 1, lane)];
        acc[mt] = mfma32x32x16(ahi, xh[ks], acc[mt]);
        acc[mt] = mfma32x32x16(alo, xh[ks], acc[mt]);     // zero for the +-16 Hadamard entries
        if (!a.f16_in) acc[mt] = mfma32x32x16(ahi, xl[ks], acc[mt]);
      }
    }
    auto yv = [&](int i) { return acc[i >> 4][i & 15]; };   // coordinate 64 h + i, in accumulator units

    // ---- level 1: 32 pairs; codes straight into the lane's B1 stream words ----
    uint32_t w1[B1];
#pragma unroll
    for (int i = 0; i < B1; ++i) w1[i] = 0u;
    float p1[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float y0 = yv(2 * j), y1 = yv(2 * j + 1);
      const float psi = atan2f(y1, y0);
      uint32_t c = 0;
#pragma unroll
      for (int k = 0; k < K1 - 1; ++k) c += psi >= a.book.b1[k] ? 1u : 0u;
      put_code<B1>(w1, j * B1, c);
      p1[j] = y0 * y0 + y1 * y1;
    }
    // ---- levels 2..6 in the lane, level 7 across the halves ----
    uint32_t uw[4] = {0u, 0u, 0u, 0u};
    float p2[16], p3[8], p4[4], p5[2], p6[1];
    polar_level<16, 0, 0, KU>(p1, p2, uw, a.book);
    polar_level<8, 1, 16, KU>(p2, p3, uw, a.book);
    polar_level<4, 2, 24, KU>(p3, p4, uw, a.book);
    polar_level<2, 3, 28, KU>(p4, p5, uw, a.book);
    polar_level<1, 4, 30, KU>(p5, p6, uw, a.book);
    const float po = shfl_xor_f(p6[0], 32);
    const float pa = h ? po : p6[0], pb = h ? p6[0] : po;
    uint32_t c7 = 0;
#pragma unroll
    for (int k = 0; k < KU - 1; ++k) c7 += pb * a.book.bc[5][k] > pa * a.book.bs[5][k] ? 1u : 0u;

    // ---- reconstruction from the unit length down, residual fragments ----
    const float2 t7 = tabu[16 * 5 + c7];
    float r6[1] = {h ? t7.y : t7.x};
    float r5[2], r4[4], r3[8], r2[16], r1[32];
    polar_split<1, 4, 30>(r6, r5, uw, tabu);
    polar_split<2, 3, 28>(r5, r4, uw, tabu);
    polar_split<4, 2, 24>(r4, r3, uw, tabu);
    polar_split<8, 1, 16>(r3, r2, uw, tabu);
    polar_split<16, 0, 0>(r2, r1, uw, tabu);
    float g2 = 0.f;
    half8 rh[8], rl[8];
    const float rsc = R_SCALE * ysc;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float2 t = tab1[get_code<B1>(w1, j * B1)];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int i = 2 * j + e;
        const float d = yv(i) - r1[j] * (e ? t.y : t.x) * inv;    // (y - y~) / ysc
        g2 += d * d;
        if (QJL) {
          _Float16 hi, lo;
          split_f16(d * rsc, hi, lo);
          rh[i >> 3][i & 7] = hi;
          rl[i >> 3][i & 7] = lo;
        }
      }
    }
    // ---- GEMM2: QJL signs of the residual; lane half h collects words 2h, 2h + 1 ----
    uint32_t sw[2] = {0u, 0u};
    if (QJL) {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        f32x16 acc2 = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const half8 shi = fs[frag_index(it, ks, 0, lane)];
          const half8 slo = fs[frag_index(it, ks, 1, lane)];
          acc2 = mfma32x32x16(shi, rh[ks], acc2);
          acc2 = mfma32x32x16(slo, rh[ks], acc2);
          acc2 = mfma32x32x16(shi, rl[ks], acc2);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sw[it >> 1] = shift_in(sw[it >> 1], ge_mask(acc2[r], 0.f));
      }
    }
    // ---- store: the lane half's level-1 words, half 0 the upper stream and scalars ----
    uint32_t ou[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ou[i] = shfl_xor_u(uw[i], 32);
    const float gam = sqrtf(g2 + shfl_xor_f(g2, 32)) * ysc;
    const int64_t rec = valid ? (a.slot ? a.slot[vec] : vec) : -1;
    if ((uint64_t)rec < (uint64_t)a.records) {
      uint32_t* dst = a.planes + rec * P;
#pragma unroll
      for (int i = 0; i < B1; ++i) dst[h * B1 + i] = w1[i];
      if (QJL) {
        dst[2 * B1 + 2 * B + 2 * h] = __builtin_bitreverse32(sw[0]);
        dst[2 * B1 + 2 * B + 2 * h + 1] = __builtin_bitreverse32(sw[1]);
      }
      if (h == 0) {
        uint32_t us[2 * B];
#pragma unroll
        for (int i = 0; i < 2 * B; ++i) us[i] = 0u;
#pragma unroll
        for (int li = 0; li < 5; ++li) {
#pragma unroll
          for (int src = 0; src < 2; ++src) {
#pragma unroll
            for (int j = 0; j < PL_HALF[li]; ++j) {
              const int slot = PL_LOCAL[li] + j;
              const uint32_t c = ((src ? ou : uw)[slot >> 3] >> (4 * (slot & 7))) & 15u;
              put_code<B>(us, (PL_STREAM[li] + src * PL_HALF[li] + j) * B, c);
            }
          }
        }
        put_code<B>(us, 62 * B, c7);
#pragma unroll
        for (int i = 0; i < 2 * B; ++i) dst[2 * B1 + i] = us[i];
        if (QJL)
          reinterpret_cast<uint32_t*>(a.scalars)[rec] = (uint32_t)f16_bits(nrm) | ((uint32_t)f16_bits(gam) << 16);
        else
          a.scalars[rec] = f16_bits(nrm);
      }
    }
  }
}

template <int B1, int B, bool QJL>
hipError_t launch_polar3(const PolarArgs& a, hipStream_t stream) {
  int dev = 0, cus = 256;
  hipGetDevice(&dev);
  hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const size_t lds = (QJL ? 2 : 1) * FRAGS * sizeof(half8) + 16 * 7 * sizeof(float2);
  const int64_t ntiles = (a.n + 31) / 32;
  auto go = [&](auto kern, int waves) -> hipError_t {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const int grid = (int)std::min<int64_t>((ntiles + waves - 1) / waves, (int64_t)cus);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * waves), lds, stream, a);
    return hipGetLastError();
  };
  // eight-wave workgroups share the fragments; a small batch spreads one-wave
  // workgroups over the compute units instead
  if (ntiles < 2 * (int64_t)cus) return go(polar_encode128<B1, B, QJL, 1>, 1);
  return go(polar_encode128<B1, B, QJL, 8>, 8);
}

template <int B1, int B>
hipError_t launch_polar2(const PolarArgs& a, hipStream_t stream) {
  return a.qjl ? launch_polar3<B1, B, true>(a, stream) : launch_polar3<B1, B, false>(a, stream);
}

template <int B1>
hipError_t launch_polar1(const PolarArgs& a, hipStream_t stream) {
  switch (a.b) {
    case 1: return launch_polar2<B1, 1>(a, stream);
    case 2: return launch_polar2<B1, 2>(a, stream);
    case 3: return launch_polar2<B1, 3>(a, stream);
    case 4: return launch_polar2<B1, 4>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_polar_encode128(const PolarArgs& a, hipStream_t stream) {
  switch (a.b1) {
    case 1: return launch_polar1<1>(a, stream);
    case 2: return launch_polar1<2>(a, stream);
    case 3: return launch_polar1<3>(a, stream);
    case 4: return launch_polar1<4>(a, stream);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// The explicit R-round Hadamard matrix (tq_hadamard_matrix): one workgroup per
// column j, the transform of e_j in the LDS, rounds of sign flip then an
// in-place butterfly pass per index bit; the unscaled values are integers
// (exact in float32 up to 2048^2), and the scale d_rot^(-R/2) is applied once.
// ---------------------------------------------------------------------------
namespace {
__global__ __launch_bounds__(256) void hadamard_matrix_kernel(const float* eps, int rounds, int d, int d_rot,
                                                              float scale, float* out) {
  __shared__ float v[2048];
  const int j = blockIdx.x;
  for (int i = threadIdx.x; i < d_rot; i += 256) v[i] = i == j ? 1.f : 0.f;
  __syncthreads();
  for (int r = 0; r < rounds; ++r) {
    for (int i = threadIdx.x; i < d_rot; i += 256) v[i] *= eps[(size_t)r * d_rot + i];
    __syncthreads();
    for (int h = 1; h < d_rot; h <<= 1) {
      for (int p = threadIdx.x; p < d_rot / 2; p += 256) {
        const int lo = (p / h) * 2 * h + (p % h), hi = lo + h;
        const float a = v[lo], b = v[hi];
        v[lo] = a + b;
        v[hi] = a - b;
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < d_rot; i += 256) out[(size_t)i * d + j] = v[i] * scale;
}
}  // namespace

hipError_t launch_hadamard_matrix(const float* eps, int rounds, int d, int d_rot, float* out, hipStream_t stream) {
  double sc = 1.0;
  for (int r = 0; r < rounds; ++r) sc /= std::sqrt((double)d_rot);
  hipLaunchKernelGGL(hadamard_matrix_kernel, dim3((unsigned)d), dim3(256), 0, stream, eps, rounds, d, d_rot,
                     (float)sc, out);
  return hipGetLastError();
}

}  // namespace tq
