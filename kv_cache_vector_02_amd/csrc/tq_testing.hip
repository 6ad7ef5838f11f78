// Measurement and testing entry points (include/tq_testing.h): not part of
// the method.  tq_testing_stream is the attainable-bandwidth yardstick the
// score pass is compared with: a plain stream that reads and writes HBM in a
// given ratio with the same 16-byte-per-lane buffer accesses and the same
// store cache policy, and no arithmetic.
#include <atomic>

#include "tq_device.h"
#include "tq_internal.h"
#include "../../include/tq_testing.h"

namespace tq {
namespace {

constexpr int ST_THREADS = 256;
constexpr int ST_UNROLL = 8;      // 16-byte loads in flight per lane

// Thread g of G reads items g, g + G, ... of the read stream, ST_UNROLL at a
// time, and after every read item adds nw to a running count, writing one
// item of the write stream (items g, g + G, ...) each time the count passes
// nr: every thread keeps the global read:write ratio, so both streams run
// side by side for the whole kernel.  The written value depends on the loads.
__global__ __launch_bounds__(ST_THREADS) void stream_kernel(const uint8_t* src, uint32_t nr, uint8_t* dst,
                                                            uint32_t nw, int cpol) {
  const uint32_t G = gridDim.x * ST_THREADS;
  const uint32_t g = blockIdx.x * ST_THREADS + threadIdx.x;
  const rsrc_t rs = make_rsrc(src, nr * 16u);
  const rsrc_t rd = make_rsrc(dst, nw * 16u);
  i32x4 acc = {0, 0, 0, 0};
  uint64_t cnt = 0;
  uint32_t w = g;
  for (uint32_t r0 = g; r0 < nr; r0 += ST_UNROLL * G) {
    i32x4 v[ST_UNROLL];
#pragma unroll
    for (int u = 0; u < ST_UNROLL; ++u) {
      const uint32_t r = r0 + u * G;
      v[u] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, r < nr ? r * 16u : OOB_OFFSET, 0, 0));
    }
#pragma unroll
    for (int u = 0; u < ST_UNROLL; ++u) {
      acc ^= v[u];
      cnt += nw;
      if (cnt >= nr) {
        cnt -= nr;
        const uint32_t off = w < nw ? w * 16u : OOB_OFFSET;
        if (cpol)
          __builtin_amdgcn_raw_buffer_store_b128(acc, rd, off, 0, 16);
        else
          __builtin_amdgcn_raw_buffer_store_b128(acc, rd, off, 0, 0);
        w += G;
      }
    }
  }
  // writes left over by rounding (at most a few per thread)
  for (; w < nw; w += G) {
    if (cpol)
      __builtin_amdgcn_raw_buffer_store_b128(acc, rd, w * 16u, 0, 16);
    else
      __builtin_amdgcn_raw_buffer_store_b128(acc, rd, w * 16u, 0, 0);
  }
}

}  // namespace
}  // namespace tq

extern "C" tq_status tq_testing_stream(const void* src, size_t read_bytes, void* dst, size_t write_bytes,
                                       int store_policy, int workgroups, void* stream) {
  if ((read_bytes && !src) || (write_bytes && !dst)) return TQ_ERR_INVALID_ARG;
  if (read_bytes % 16 || write_bytes % 16 || ((uintptr_t)src % 16) || ((uintptr_t)dst % 16))
    return TQ_ERR_INVALID_ARG;
  if (read_bytes >= (1ull << 31) || write_bytes >= (1ull << 31)) return TQ_ERR_UNSUPPORTED;
  if (store_policy != 0 && store_policy != 1) return TQ_ERR_INVALID_ARG;
  if (read_bytes == 0 && write_bytes == 0) return TQ_OK;
  int cus = 256, dev = 0;
  if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int blocks = workgroups > 0 ? workgroups : 8 * cus;
  // with no reads every thread writes its share in the leftover loop
  hipLaunchKernelGGL(tq::stream_kernel, dim3(blocks), dim3(tq::ST_THREADS), 0, (hipStream_t)stream,
                     static_cast<const uint8_t*>(src), (uint32_t)(read_bytes / 16), static_cast<uint8_t*>(dst),
                     (uint32_t)(write_bytes / 16), store_policy);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}
