// Internal declarations shared by the host API and the HIP kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tq.h"

namespace tq {

tq_status build_codebook(int d, int bits, double* centroids, double* boundaries);

// Codebook by value: it travels in the kernel argument buffer (scalar
// registers / constant cache), never in device memory.
struct Codebook {
  float c[16];   // centroids, ascending
  float b[16];   // boundaries (2^bq - 1 used)
};

struct EncodeArgs {
  const void* x;
  int f16_in;          // 1: x is float16, 0: float32
  int64_t n;
  int64_t ld_x;        // elements between rows of x
  int d;               // input dimension (<= d_rot)
  const float* pi;     // dense rotation [d_rot][d]
  const float* eps;    // hadamard signs [d_rot]
  const float* s;      // QJL matrix [m][d_rot] (prod only)
  int m;               // QJL rows: d_rot, or d_rot / 2 at d_rot = 128
  Codebook cb;
  int bq;              // index bits
  int prod;            // 1: per-record key layout, 0: values (mse, token-blocked)
  int qjl;             // with prod: 1 = QJL signs and gamma (prod keys), 0 = MSE-only keys
  int eden;            // MSE records: store n / <y, c[idx]> (EDEN's unbiased scale) instead of n
  int had;             // 1: sign-flipped Hadamard rotation (eps), 0: dense (pi)
  uint32_t* planes;    // [records][P][d_rot/32]
  uint16_t* scalars;   // [records][S] float16 bit patterns
  const int64_t* slot; // record of vector i, or null
};

hipError_t launch_encode_dense128(const EncodeArgs& a, hipStream_t stream);

// Prod encode at d_rot = 2048 (Hadamard): chunked two-pass path with a workspace.
struct Encode2kArgs {
  const void* x;
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
  _Float16 *s_hi, *s_lo;   // [2048][2048]
  _Float16 *r_hi, *r_lo;   // [chunk][2048], prescaled residuals
};
size_t encode2k_workspace(int64_t n);

// Walsh coefficients u_S of the odd subsets of an odd-symmetric codebook of bq
// index bits (plane order) and their sum.
void walsh_coefficients(const Codebook& cb, int bq, float u[8], float* usum);

// Top-k retrieval at d_rot = 2048 (Hadamard records): prod keys (qjl = 1,
// bq = b - 1 index planes + the QJL plane, scalars n and gamma) or MSE-only
// records (qjl = 0, bq = b planes, scalar n).
struct TopkLaunch {
  const float* q;          // [nq][d]
  int nq, d, bq, k;
  int qjl;
  const float* eps;
  const float* s;          // prod only
  float u[8];
  float usum;
  const uint32_t* planes;  // records, key layout with W = 64
  const uint16_t* scalars;
  int64_t T;
  int64_t* idx;            // [nq][k]
  float* val;              // [nq][k]
  void* ws;
};
size_t topk2k_workspace(int nq, int64_t T, int k, int bq, int qjl);
hipError_t launch_topk2k(const TopkLaunch& L, hipStream_t stream);
hipError_t launch_encode2k(const EncodeArgs& a, void* ws, hipStream_t stream);
// MSE records at d_rot = 2048 (Hadamard): one pass, no workspace.
hipError_t launch_encode2k_mse(const EncodeArgs& a, hipStream_t stream);

struct ScoreArgs {
  const float* q;        // [segs*group][d]
  int segs, group, d;
  const float* pi;       // rotation of the keys (dense)
  const float* eps;      // hadamard signs
  int rot;
  const float* s;        // QJL matrix [m][d] (prod keys) or NULL (MSE-only keys)
  int m;                 // QJL rows: d, or d / 2
  Codebook cb;
  int bq;                // index bits
  int qjl;               // 1: prod keys (QJL plane, n and gamma); 0: MSE-only keys (n only)
  const uint32_t* planes;
  const uint16_t* scalars;
  int64_t seg_stride;
  const int32_t* len;
  int64_t T;
  float* scores;
  void* ws;
};

hipError_t launch_scores128(const ScoreArgs& a, hipStream_t stream);
hipError_t launch_scores128_prepare(const ScoreArgs& a, hipStream_t stream);    // query pack only
hipError_t launch_scores128_prepared(const ScoreArgs& a, hipStream_t stream);   // score pass only
hipError_t launch_scores128_prep(const ScoreArgs& a, int slices, hipStream_t stream);
size_t scores128_workspace(int segs, int group);
void set_pack_wait_us(int us);   // one-launch scores: consumers' wait bound

struct AttendArgs {
  ScoreArgs k;           // query + key side (scores field unused)
  const float* pi_v;     // value rotation (dense)
  const float* eps_v;
  int rot_v;
  Codebook cb_v;
  int bq_v;
  const uint32_t* planes_v;
  const uint16_t* scalars_v;
  int64_t seg_stride_v;
  float scale;
  float* out;
  void* ws;
};

hipError_t launch_attend128(const AttendArgs& a, hipStream_t stream);
size_t attend128_workspace(int segs, int group, int64_t T);

}  // namespace tq
