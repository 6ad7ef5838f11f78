// Measurement and testing entry points (include/tq_testing.h): not part of
// the method.  tq_testing_stream is the attainable-bandwidth yardstick the
// score pass is compared with: a plain stream that reads and writes HBM in a
// given ratio with the same 16-byte-per-lane buffer accesses and the same
// load and store cache policies, and no arithmetic.
#include <atomic>

#include "tq_device.h"
#include "tq_internal.h"
#include "../../include/tq_testing.h"

namespace tq {
namespace {

constexpr int ST_THREADS = 256;
constexpr int ST_UNROLL = 8;      // 4 KB chunks in flight per workgroup

// Workgroup w of G owns the w-th contiguous slice of each stream, in 4 KB
// chunks (256 lanes x 16 bytes, one coalesced load or store per chunk).  It
// reads ST_UNROLL chunks at a time and, after each batch, writes as many chunks
// as keep its write slice in step with its read slice, so both streams run
// side by side for the whole kernel.  The written value depends on the loads.
template <int LOAD_CPOL>
__global__ __launch_bounds__(ST_THREADS) void stream_kernel(const uint8_t* src, uint32_t nr, uint8_t* dst,
                                                            uint32_t nw, int cpol) {
  const uint32_t G = gridDim.x, w = blockIdx.x, t = threadIdx.x;
  const uint32_t rc = (nr + ST_THREADS - 1) / ST_THREADS, wc = (nw + ST_THREADS - 1) / ST_THREADS;  // chunks
  const uint32_t r0 = (uint32_t)((uint64_t)rc * w / G), r1 = (uint32_t)((uint64_t)rc * (w + 1) / G);
  const uint32_t w0 = (uint32_t)((uint64_t)wc * w / G), w1 = (uint32_t)((uint64_t)wc * (w + 1) / G);
  const rsrc_t rs = make_rsrc(src, nr * 16u);
  const rsrc_t rd = make_rsrc(dst, nw * 16u);
  i32x4 acc = {0, 0, 0, 0};
  uint32_t wnext = w0;
  auto put = [&](uint32_t c) {
    const uint32_t item = c * ST_THREADS + t;
    const uint32_t off = item < nw ? item * 16u : OOB_OFFSET;
    if (cpol)
      __builtin_amdgcn_raw_buffer_store_b128(acc, rd, off, 0, 16);
    else
      __builtin_amdgcn_raw_buffer_store_b128(acc, rd, off, 0, 0);
  };
  for (uint32_t c0 = r0; c0 < r1; c0 += ST_UNROLL) {
    i32x4 v[ST_UNROLL];
#pragma unroll
    for (int u = 0; u < ST_UNROLL; ++u) {
      const uint32_t item = (c0 + u) * ST_THREADS + t;
      v[u] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rs, c0 + u < r1 && item < nr ? item * 16u : OOB_OFFSET, 0, LOAD_CPOL));
    }
#pragma unroll
    for (int u = 0; u < ST_UNROLL; ++u) acc ^= v[u];
    // write chunks up to the share of the read progress made so far
    const uint32_t done = c0 + ST_UNROLL < r1 ? c0 + ST_UNROLL - r0 : r1 - r0;
    const uint32_t target = w0 + (uint32_t)((uint64_t)(w1 - w0) * done / (r1 - r0));
    for (; wnext < target; ++wnext) put(wnext);
  }
  for (; wnext < w1; ++wnext) put(wnext);   // all of it when there is nothing to read
}

}  // namespace
}  // namespace tq

extern "C" tq_status tq_testing_stream(const void* src, size_t read_bytes, void* dst, size_t write_bytes,
                                       int store_policy, int workgroups, void* stream) {
  if ((read_bytes && !src) || (write_bytes && !dst)) return TQ_ERR_INVALID_ARG;
  if (read_bytes % 16 || write_bytes % 16 || ((uintptr_t)src % 16) || ((uintptr_t)dst % 16))
    return TQ_ERR_INVALID_ARG;
  if (read_bytes >= (1ull << 31) || write_bytes >= (1ull << 31)) return TQ_ERR_UNSUPPORTED;
  if (store_policy < 0 || store_policy > 3) return TQ_ERR_INVALID_ARG;
  if (read_bytes == 0 && write_bytes == 0) return TQ_OK;
  int cus = 256, dev = 0;
  if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int blocks = workgroups > 0 ? workgroups : 4 * cus;
  // with no reads every thread writes its share in the leftover loop
  if (store_policy & 2)
    hipLaunchKernelGGL(tq::stream_kernel<tq::CPOL_NT>, dim3(blocks), dim3(tq::ST_THREADS), 0, (hipStream_t)stream,
                       static_cast<const uint8_t*>(src), (uint32_t)(read_bytes / 16), static_cast<uint8_t*>(dst),
                       (uint32_t)(write_bytes / 16), store_policy & 1);
  else
    hipLaunchKernelGGL(tq::stream_kernel<0>, dim3(blocks), dim3(tq::ST_THREADS), 0, (hipStream_t)stream,
                       static_cast<const uint8_t*>(src), (uint32_t)(read_bytes / 16), static_cast<uint8_t*>(dst),
                       (uint32_t)(write_bytes / 16), store_policy & 1);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}
