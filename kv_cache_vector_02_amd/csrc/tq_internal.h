// Internal declarations shared by the host API and the HIP kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tq.h"

namespace tq {

tq_status build_codebook(int d, int bits, double* centroids, double* boundaries);
tq_status build_polar_codebook(int level, int bits, double* centroids, double* boundaries);

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
  int m;               // QJL rows: d_rot, or d_rot / 2 (d_rot = 128 or 2048)
  Codebook cb;
  int bq;              // index bits
  int prod;            // 1: per-record key layout, 0: values (mse, token-blocked)
  int qjl;             // with prod: 1 = QJL signs and gamma (prod keys), 0 = MSE-only keys
  int eden;            // MSE records: store n / <y, c[idx]> (EDEN's unbiased scale) instead of n
  int had;             // 1: sign-flipped Hadamard rotation (eps), 0: dense (pi)
  int rounds;          // Hadamard rounds (eps holds rounds x d_rot signs)
  uint32_t* planes;    // [records][P][d_rot/32]
  uint16_t* scalars;   // [records][S] float16 bit patterns
  const int64_t* slot; // record of vector i, or null
  int64_t records;     // capacity of planes / scalars in records: records at or past it are not written
  int interleave;      // d = 128 encode launch: 1 = one tile per workgroup (set by the launcher)
  int split;           // with interleave, values: workgroups per tile (set by the launcher)
};

hipError_t launch_encode_dense128(const EncodeArgs& a, hipStream_t stream);
// The explicit R-round Hadamard matrix [d_rot][d] (tq_hadamard_matrix).
hipError_t launch_hadamard_matrix(const float* eps, int rounds, int d, int d_rot, float* out, hipStream_t stream);

// Prod encode at d_rot = 2048 (Hadamard): chunked two-pass path with a workspace.
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
  const float* eps;        // [rounds][2048]
  int rounds;
  const float* s;          // prod only, [m][2048]
  int m;                   // QJL rows: 2048 or 1024
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
  int wait_us;           // one-launch scores: consumers' bound on the wait for the pack (microseconds)
  int one_launch = 0;    // tq_scores: keep the one-launch form for a long pass too (test control)
  int n_sets, set_div;   // rotation sets of the keys: query segment seg uses set (seg / set_div) % n_sets
};

// The bound tq_scores gives a workgroup's wait for its segment's query pack.
constexpr int PACK_WAIT_US = 200;

hipError_t launch_scores128(const ScoreArgs& a, hipStream_t stream);
hipError_t launch_scores128_prepare(const ScoreArgs& a, hipStream_t stream);    // query pack only
hipError_t launch_scores128_prepared(const ScoreArgs& a, hipStream_t stream);   // score pass only
hipError_t launch_scores128_prep(const ScoreArgs& a, int slices, hipStream_t stream);
size_t scores128_workspace(int segs, int group);
// tq_scores_noalloc's workspace: a device array of this many bytes per GPU.
constexpr size_t SCORES_SCRATCH_BYTES = 16u << 20;
// Its address on the current device (resolved once per device) and size.
hipError_t scores_scratch(void** ptr, size_t* bytes);

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
  int kv_div;            // k.segs / cache segments: 2 when each segment's heads run as two halves
  int n_sets_v, set_div_v;   // rotation sets of the values (per cache segment)
  int prepared;          // 1: ws already holds the query pack (tq_attend_prepare)
};

hipError_t launch_attend128(const AttendArgs& a, hipStream_t stream);
// The attention query pack alone (the first of launch_attend128's launches).
hipError_t launch_attend128_prepare(const AttendArgs& a, hipStream_t stream);
size_t attend128_workspace(int segs, int group, int64_t T);

// PolarQuant at d = 128 (levels 1..7).  The codebook tables travel in the
// kernel argument buffer, prepared on the host in float64 from the float32
// codebook: level-1 boundaries (compared with atan2 of the pair), the cos^2
// and sin^2 of the upper boundaries (compared with squared lengths, no
// trigonometry), and the cos and sin of every centroid (the reconstruction).
struct PolarBook {
  float b1[15];            // level-1 boundaries (radians, ascending)
  float c1[16][2];         // level-1 centroids: cos, sin
  float bc[6][15];         // levels 2..7: cos^2 of the boundaries
  float bs[6][15];         // levels 2..7: sin^2 of the boundaries
  float cu[6][16][2];      // levels 2..7 centroids: cos, sin
};

struct PolarArgs {
  // quantizer
  const float* pi;         // dense rotation [128][128], or NULL
  const float* eps;        // hadamard signs [128], or NULL
  const float* s;          // QJL matrix [128][128] when qjl
  int had, b1, b, qjl;
  PolarBook book;
  // records
  uint32_t* planes;        // [records][words]
  uint16_t* scalars;       // [records][qjl ? 2 : 1]
  int64_t records;
  // encode
  const void* x;
  int f16_in;
  int64_t n, ld_x;
  const int64_t* slot;
  // decode
  float* out;
  int64_t ld_out;
  // scores
  const float* q;          // [segs*group][128]
  int segs, group;
  int64_t seg_stride;
  const int32_t* len;
  int64_t T;
  float* scores;           // [segs*group][T]
  int wps;                 // workgroups per segment
  int64_t tpw;             // tokens per workgroup (a multiple of 256)
};

// Centroid (cos, sin) tables into the LDS: tab[0..16) level 1, tab[16 + 16 (l-2)
// + k] level l.  Every entry is read from the argument buffer at a constant
// offset (a run-time index into a kernel argument would copy the whole
// argument block to scratch memory).
__device__ __forceinline__ void polar_tables_to_lds(const PolarBook& bk, float2* tab) {
#pragma unroll
  for (int i = 0; i < 16 * 7; ++i) {
    if ((int)threadIdx.x == i % (int)blockDim.x) {
      const float* c = i < 16 ? bk.c1[i] : bk.cu[(i - 16) >> 4][(i - 16) & 15];
      tab[i] = make_float2(c[0], c[1]);
    }
  }
}

hipError_t launch_polar_encode128(const PolarArgs& a, hipStream_t stream);
hipError_t launch_polar_decode128(const PolarArgs& a, hipStream_t stream);
hipError_t launch_polar_scores128(const PolarArgs& a, hipStream_t stream);
size_t polar_scores128_lds(int b1, int qjl, int group);

}  // namespace tq
