// TurboQuant-prod encode at d_rot = 2048, sign-flipped Hadamard rotation
// (retrieval embeddings: d <= 2048, zero-padded to the Hadamard order).
//
// Per vector x (blog notes on the paper: Q_prod; explainer page, the random
// Hadamard rotation):
//   n = ||x||, u = x / n, y = H diag(eps) pad(u) / sqrt(2048),
//   idx_j = #{beta_k <= y_j}, r = y - c[idx], gamma = ||r||, z = [S r >= 0].
//
// Pass 1, one wave per vector: lane l holds coordinates 32 l .. 32 l + 31.
// The Walsh-Hadamard transform runs in registers: butterflies on index bits
// 0..4 stay inside a lane, bits 5..10 pair lane l with lane l ^ 2^(b-5)
// (cross-lane shuffles).  Plane word w of a record covers coordinates
// 32 w .. 32 w + 31, so lane l builds word l of every index plane by itself.
// The residual goes to the workspace as fp16 hi + lo (prescaled by 2^8).
//
// Pass 2, the QJL projection of a chunk of residuals, C = R S^T (M = vectors,
// N = m, K = 2048), on v_mfma_f32_32x32x16_f16 with fp16 hi/lo operands (three
// products, ~2^-22 relative).  A workgroup (8 waves) owns a 256 x 128 tile of
// C, staged through the LDS in K blocks of 32; a wave owns 64 x 64.  Lane l
// of a 32 x 32 accumulator holds column l % 32 for 16 rows, so the sign bits
// of a row's 32 columns are one ballot: the epilogue writes whole QJL plane
// words.  Consecutive workgroups share an M tile and the workgroup-to-XCD
// assignment (id mod 8) gives each XCD fixed 128-row slices of S, which stay
// in its L2.
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

struct Encode2kArgs {
  const void* x;
  int rounds;          // Hadamard rounds (eps holds rounds x 2048 signs)
  int m;               // QJL rows (prod): 2048, or 1024 (sign words in coordinate groups 0..31 only)
  int64_t ld_x;
  int d;
  int64_t n;           // vectors in the call
  int64_t v0, cn;      // current chunk: first vector, count
  int64_t chunk;       // vectors per chunk (multiple of 128 rows of residual space)
  const float* eps;
  Codebook cb;
  uint32_t* planes;
  uint16_t* scalars;
  const int64_t* slot;
  int64_t records;         // capacity in records (records at or past it are not written)
  _Float16 *s_hi, *s_lo;   // [2048][2048]
  _Float16 *r_hi, *r_lo;   // [chunk][2048], prescaled residuals
};

namespace {

constexpr int D2 = 2048;
constexpr int VPL = 32;                  // coordinates per lane
// Prod records with m QJL rows: for each 32-coordinate group g, its BQ index
// words, then sign word g while g < m / 32.  Word offset of group g and the
// record's length in words.
__device__ __forceinline__ int group_offset(int g, int bq, int mw) { return g < mw ? g * (bq + 1) : mw * (bq + 1) + (g - mw) * bq; }
__device__ __forceinline__ int record_words(int bq, int mw) { return 64 * bq + mw; }

constexpr float R2_SCALE = 256.f;        // 2^8, keeps the residual's lo part normal in fp16
constexpr float INV_SQRT_D2 = 0.02209708691207961f;   // 1 / sqrt(2048)

__global__ __launch_bounds__(256) void split_s_f16(const float* __restrict__ s, _Float16* hi, _Float16* lo,
                                                    int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256) {
    _Float16 h, l;
    split_f16(s[i], h, l);
    hi[i] = h;
    lo[i] = l;
  }
}

template <int BQ>
__device__ __forceinline__ void quantize2k(float y, const Codebook& cb, int& idx, float& chat) {
  idx = 0;
  chat = cb.c[0];
#pragma unroll
  for (int k = 0; k < (1 << BQ) - 1; ++k) {
    const bool ge = y >= cb.b[k];
    idx += ge ? 1 : 0;
    chat = ge ? cb.c[k + 1] : chat;
  }
}

// PROD: key records (BQ index planes + the QJL plane, written by the
// projection pass; scalars n and gamma) with the residual to the workspace;
// otherwise MSE records (BQ planes, scalar n, or with EDEN the unbiased
// per-vector scale n / <y, c[idx]>) and nothing else.
template <int BQ, bool F16IN, bool PROD, bool EDEN = false>
__global__ __launch_bounds__(256) void encode2k_pass1(Encode2kArgs a) {
  static_assert(!(EDEN && PROD), "the scale replaces the norm of MSE records only");
  constexpr int P = PROD ? BQ + 1 : BQ;
  // EDEN reads c[idx] from an LDS table (a select chain over the centroids
  // would hold them all in registers); every wave passes the barrier before
  // any wave leaves
  __shared__ float ctab[16];
  if constexpr (EDEN) {
    if (threadIdx.x < (1 << BQ)) ctab[threadIdx.x] = a.cb.c[threadIdx.x];
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const int64_t vec = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);    // chunk-local
  if (vec >= a.cn) return;
  const int64_t gv = a.v0 + vec;
  const int j0 = VPL * lane;
  float v[VPL];
  if (F16IN) {
    const _Float16* src = static_cast<const _Float16*>(a.x) + gv * a.ld_x + j0;
#pragma unroll
    for (int i = 0; i < VPL; i += 8) {
      half8 h = {};
      if (j0 + i < a.d) h = *reinterpret_cast<const half8*>(src + i);   // d is a multiple of 8
#pragma unroll
      for (int e = 0; e < 8; ++e) v[i + e] = (float)h[e];
    }
  } else {
    const float* src = static_cast<const float*>(a.x) + gv * a.ld_x + j0;
#pragma unroll
    for (int i = 0; i < VPL; i += 4) {
      float4 f = {0.f, 0.f, 0.f, 0.f};
      if (j0 + i < a.d) f = *reinterpret_cast<const float4*>(src + i);   // d is a multiple of 4
      v[i] = f.x; v[i + 1] = f.y; v[i + 2] = f.z; v[i + 3] = f.w;
    }
  }
  float s2 = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) s2 = fmaf(v[i], v[i], s2);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) s2 += shfl_xor_f(s2, o);
  const float n = sqrtf(s2);
  const float inv = n > 0.f ? 1.f / n : 0.f;
  {
    const float4* e4 = reinterpret_cast<const float4*>(a.eps + j0);
#pragma unroll
    for (int i = 0; i < VPL; i += 4) {
      const float4 e = e4[i / 4];
      v[i] *= inv * e.x; v[i + 1] *= inv * e.y; v[i + 2] *= inv * e.z; v[i + 3] *= inv * e.w;
    }
  }
  fwht2048_wave(v, lane);
  // further rounds: scale, this round's signs, transform again
#pragma unroll 1
  for (int r = 1; r < a.rounds; ++r) {
    const float4* er = reinterpret_cast<const float4*>(a.eps + (size_t)r * D2 + j0);
#pragma unroll
    for (int i = 0; i < VPL; i += 4) {
      const float4 e = er[i / 4];
      v[i] *= INV_SQRT_D2 * e.x; v[i + 1] *= INV_SQRT_D2 * e.y; v[i + 2] *= INV_SQRT_D2 * e.z;
      v[i + 3] *= INV_SQRT_D2 * e.w;
    }
    fwht2048_wave(v, lane);
  }
  // quantise, pack this lane's plane words, residual
  uint32_t w[BQ];
#pragma unroll
  for (int p = 0; p < BQ; ++p) w[p] = 0u;
  float g2 = 0.f;
  float yc = 0.f;   // EDEN: this lane's part of <y, c[idx]>
  half8 rh[VPL / 8], rl[VPL / 8];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const float y = v[i] * INV_SQRT_D2;
    int idx;
    float chat;
    quantize2k<BQ>(y, a.cb, idx, chat);
#pragma unroll
    for (int p = 0; p < BQ; ++p) w[p] |= (uint32_t)((idx >> p) & 1) << i;
    if (EDEN) yc = fmaf(y, ctab[idx], yc);
    if (PROD) {
      const float r = y - chat;
      g2 = fmaf(r, r, g2);
      _Float16 h, l;
      split_f16(r * R2_SCALE, h, l);
      rh[i / 8][i % 8] = h;
      rl[i / 8][i % 8] = l;
    }
  }
  if (PROD) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) g2 += shfl_xor_f(g2, o);
    half8* rhi = reinterpret_cast<half8*>(a.r_hi + vec * D2 + j0);
    half8* rlo = reinterpret_cast<half8*>(a.r_lo + vec * D2 + j0);
#pragma unroll
    for (int q = 0; q < VPL / 8; ++q) {
      rhi[q] = rh[q];
      rlo[q] = rl[q];
    }
  }
  float scale = n;
  if (EDEN) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) yc += shfl_xor_f(yc, o);
    scale = n > 0.f && yc > 0.f ? n / yc : 0.f;
  }
  const int64_t rec = a.slot ? a.slot[gv] : gv;
  if ((uint64_t)rec >= (uint64_t)a.records) return;      // past the cache's capacity: not written
  uint32_t* dst = PROD ? a.planes + rec * record_words(BQ, a.m / 32) + group_offset(lane, BQ, a.m / 32)
                       : a.planes + rec * (P * (D2 / 32)) + lane * P;
#pragma unroll
  for (int p = 0; p < BQ; ++p) dst[p] = w[p];
  if (lane == 0) {
    if (PROD)
      reinterpret_cast<uint32_t*>(a.scalars)[rec] = (uint32_t)f16_bits(n) | ((uint32_t)f16_bits(sqrtf(g2)) << 16);
    else
      a.scalars[rec] = f16_bits(scale);
  }
}

// Workgroup tile 256 vectors x 128 projection rows, 8 waves of 64 x 64;
// K in stages of 32, double-buffered in the LDS (rows padded to 80 bytes, so
// the 16-byte fragment reads of 16 lanes cover all 64 banks once), the next
// stage's global loads in flight while the current one is multiplied.
constexpr int SG_M = 256, SG_N = 128, SG_K = 32, SG_LD = 40, SG_THREADS = 512;
constexpr int SG_A = SG_M * SG_LD, SG_B = SG_N * SG_LD;   // halfs per operand copy
constexpr int SG_STAGE = 2 * SG_A + 2 * SG_B;             // A hi, A lo, B hi, B lo
constexpr size_t SG_LDS = 2 * SG_STAGE * sizeof(_Float16);

template <int P>
__global__ __launch_bounds__(SG_THREADS) void encode2k_signs(Encode2kArgs a) {
  extern __shared__ half8 sg8[];
  _Float16* sg = reinterpret_cast<_Float16*>(sg8);
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int64_t mrow0 = (int64_t)blockIdx.y * SG_M;   // chunk-local vector rows of the tile
  const int nrow0 = blockIdx.x * SG_N;                // projection rows of the tile
  // copy items (16 bytes each): k = 0, 1 A hi rows 0..255; 2, 3 A lo; 4 B hi;
  // 5 B lo.  Global offsets from the two bases, LDS offsets, per item.
  const int crow = t >> 2, cc = (t & 3) * 8;
  const int64_t aoff0 = (mrow0 + crow) * D2 + cc, aoff1 = aoff0 + (int64_t)128 * D2;
  const int64_t boff = (int64_t)(nrow0 + crow) * D2 + cc;
  const int l0 = crow * SG_LD + cc, l1 = l0 + 128 * SG_LD;
  uint4 stg[6];
#define SG_GLOAD(kb)                                                                                    \
  do {                                                                                                  \
    const int64_t ko = (int64_t)SG_K * (kb);                                                            \
    stg[0] = *reinterpret_cast<const uint4*>(a.r_hi + aoff0 + ko);                                      \
    stg[1] = *reinterpret_cast<const uint4*>(a.r_hi + aoff1 + ko);                                      \
    stg[2] = *reinterpret_cast<const uint4*>(a.r_lo + aoff0 + ko);                                      \
    stg[3] = *reinterpret_cast<const uint4*>(a.r_lo + aoff1 + ko);                                      \
    stg[4] = *reinterpret_cast<const uint4*>(a.s_hi + boff + ko);                                       \
    stg[5] = *reinterpret_cast<const uint4*>(a.s_lo + boff + ko);                                       \
  } while (0)
#define SG_LSTORE(stage)                                                                                \
  do {                                                                                                  \
    _Float16* d = sg + (stage) * SG_STAGE;                                                              \
    *reinterpret_cast<uint4*>(d + l0) = stg[0];                                                         \
    *reinterpret_cast<uint4*>(d + l1) = stg[1];                                                         \
    *reinterpret_cast<uint4*>(d + SG_A + l0) = stg[2];                                                  \
    *reinterpret_cast<uint4*>(d + SG_A + l1) = stg[3];                                                  \
    *reinterpret_cast<uint4*>(d + 2 * SG_A + l0) = stg[4];                                              \
    *reinterpret_cast<uint4*>(d + 2 * SG_A + SG_B + l0) = stg[5];                                       \
  } while (0)
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, kh = lane >> 5;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  constexpr int KB = D2 / SG_K;
  SG_GLOAD(0);
  SG_LSTORE(0);
  __syncthreads();
  for (int kb = 0; kb < KB; ++kb) {
    if (kb + 1 < KB) SG_GLOAD(kb + 1);
    const _Float16* st = sg + (kb & 1) * SG_STAGE;
#pragma unroll
    for (int ks = 0; ks < SG_K / 16; ++ks) {
      const int k0 = 16 * ks + 8 * kh;
      half8 ah[2], al[2], bh[2], bl[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ra = (64 * wm + 32 * i + l32) * SG_LD + k0;
        ah[i] = *reinterpret_cast<const half8*>(st + ra);
        al[i] = *reinterpret_cast<const half8*>(st + SG_A + ra);
        const int rb = (64 * wn + 32 * i + l32) * SG_LD + k0;
        bh[i] = *reinterpret_cast<const half8*>(st + 2 * SG_A + rb);
        bl[i] = *reinterpret_cast<const half8*>(st + 2 * SG_A + SG_B + rb);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = mfma32x32x16(ah[i], bh[j], acc[i][j]);
          acc[i][j] = mfma32x32x16(al[i], bh[j], acc[i][j]);
          acc[i][j] = mfma32x32x16(ah[i], bl[j], acc[i][j]);
        }
    }
    if (kb + 1 < KB) SG_LSTORE((kb + 1) & 1);
    __syncthreads();
  }
#undef SG_GLOAD
#undef SG_LSTORE
  // signs: ballot over the 32 columns of each accumulator row
  const int64_t mw = mrow0 + 64 * wm;    // chunk-local vector rows of this wave
  const int iw = nrow0 + 64 * wn;        // projection rows of this wave
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t word = 0u;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint64_t m = __ballot(acc[i][j][r] >= 0.f);
        word = lane == r ? (uint32_t)m : word;
        word = lane == 32 + r ? (uint32_t)(m >> 32) : word;
      }
      // lane r (< 16) holds row 8 (r / 4) + r % 4, lane 32 + r row 8 (r / 4) + 4 + r % 4
      const int r = lane & 31;
      if (r < 16) {
        const int row = 8 * (r >> 2) + 4 * kh + (r & 3);
        const int64_t m = mw + 32 * i + row;
        if (m < a.cn) {
          const int64_t gv = a.v0 + m;
          const int64_t rec = a.slot ? a.slot[gv] : gv;
          if ((uint64_t)rec < (uint64_t)a.records)
            a.planes[rec * record_words(P - 1, a.m / 32) + group_offset((iw + 32 * j) / 32, P - 1, a.m / 32) + (P - 1)] =
                word;
        }
      }
    }
}

template <int BQ>
hipError_t run_chunks(const Encode2kArgs& base, bool f16, hipStream_t stream) {
  Encode2kArgs a = base;
  for (int64_t v0 = 0; v0 < base.n; v0 += base.chunk) {
    a.v0 = v0;
    a.cn = base.n - v0 < base.chunk ? base.n - v0 : base.chunk;
    const unsigned g1 = (unsigned)((a.cn + 3) / 4);
    if (f16)
      hipLaunchKernelGGL((encode2k_pass1<BQ, true, true>), dim3(g1), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((encode2k_pass1<BQ, false, true>), dim3(g1), dim3(256), 0, stream, a);
    const dim3 g2((unsigned)(a.m / SG_N), (unsigned)((a.cn + SG_M - 1) / SG_M));
    hipError_t e0 = hipFuncSetAttribute(reinterpret_cast<const void*>(&encode2k_signs<BQ + 1>),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)SG_LDS);
    if (e0 != hipSuccess) return e0;
    hipLaunchKernelGGL((encode2k_signs<BQ + 1>), g2, dim3(SG_THREADS), SG_LDS, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

int64_t encode2k_chunk(int64_t n) { return n < 32768 ? (n + SG_M - 1) / SG_M * SG_M : 32768; }

size_t encode2k_workspace(int64_t n) {
  // S hi + lo, then the residual chunk hi + lo, all fp16
  return (size_t)2 * D2 * D2 * sizeof(_Float16) + (size_t)2 * encode2k_chunk(n) * D2 * sizeof(_Float16);
}

template <int BQ>
hipError_t run_mse(const Encode2kArgs& a, bool f16, bool eden, hipStream_t stream) {
  const unsigned g1 = (unsigned)((a.cn + 3) / 4);
  if (eden) {
    if (f16)
      hipLaunchKernelGGL((encode2k_pass1<BQ, true, false, true>), dim3(g1), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((encode2k_pass1<BQ, false, false, true>), dim3(g1), dim3(256), 0, stream, a);
  } else if (f16) {
    hipLaunchKernelGGL((encode2k_pass1<BQ, true, false>), dim3(g1), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((encode2k_pass1<BQ, false, false>), dim3(g1), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_encode2k_mse(const EncodeArgs& e, hipStream_t stream) {
  Encode2kArgs a = {};
  a.x = e.x;
  a.ld_x = e.ld_x;
  a.d = e.d;
  a.n = e.n;
  a.eps = e.eps;
  a.rounds = e.rounds;
  a.m = e.m > 0 ? e.m : D2;
  a.cb = e.cb;
  a.planes = e.planes;
  a.scalars = e.scalars;
  a.slot = e.slot;
  a.records = e.records;
  a.v0 = 0;
  a.cn = e.n;
  switch (e.bq) {
    case 1: return run_mse<1>(a, e.f16_in, e.eden, stream);
    case 2: return run_mse<2>(a, e.f16_in, e.eden, stream);
    case 3: return run_mse<3>(a, e.f16_in, e.eden, stream);
    case 4: return run_mse<4>(a, e.f16_in, e.eden, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_encode2k(const EncodeArgs& e, void* ws, hipStream_t stream) {
  Encode2kArgs a;
  a.x = e.x;
  a.ld_x = e.ld_x;
  a.d = e.d;
  a.n = e.n;
  a.eps = e.eps;
  a.rounds = e.rounds;
  a.m = e.m > 0 ? e.m : D2;
  a.cb = e.cb;
  a.planes = e.planes;
  a.scalars = e.scalars;
  a.slot = e.slot;
  a.records = e.records;
  a.chunk = encode2k_chunk(e.n);
  _Float16* w = static_cast<_Float16*>(ws);
  a.s_hi = w;
  a.s_lo = w + (size_t)D2 * D2;
  a.r_hi = w + (size_t)2 * D2 * D2;
  a.r_lo = a.r_hi + (size_t)a.chunk * D2;
  a.v0 = 0;
  a.cn = 0;
  hipLaunchKernelGGL(split_s_f16, dim3(1024), dim3(256), 0, stream, e.s, a.s_hi, a.s_lo, (int64_t)a.m * D2);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  switch (e.bq) {
    case 1: return run_chunks<1>(a, e.f16_in, stream);
    case 2: return run_chunks<2>(a, e.f16_in, stream);
    case 3: return run_chunks<3>(a, e.f16_in, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
