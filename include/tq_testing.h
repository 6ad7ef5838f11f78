/*
 * tq_testing.h -- measurement and testing entry points of libtq.
 *
 * These are not part of the method and not needed to use it: a bandwidth
 * yardstick for the benchmark, and a form of tq_scores that forces the
 * hand-over fallback so that a test can reach it.  They follow the
 * conventions of tq.h (caller-owned device memory, work enqueued on the given
 * stream, nothing allocated, no state kept between calls).
 */
#ifndef TQ_TESTING_H
#define TQ_TESTING_H

#include <stddef.h>

#include "tq.h"

#ifdef __cplusplus
extern "C" {
#endif

/* A plain HBM stream with no arithmetic: reads read_bytes from src and writes
 * write_bytes to dst in one launch, both streams running side by side in the
 * ratio of their sizes, with the 16-byte buffer loads and stores the score
 * kernel uses.  This is the attainable-bandwidth ceiling for a kernel with the
 * same read/write mix.
 *   src, dst       device, 16-byte aligned; sizes multiples of 16, each < 2 GiB
 *   store_policy   bit 0 set: device-coherent (sc1) stores, else default
 *                  write-back stores; bit 1 set: non-temporal loads, else
 *                  default loads (the score kernel's policy is 3: sc1 stores,
 *                  non-temporal key loads)
 *   workgroups     grid size (256 threads each), or 0 for 4 per compute unit
 * The bytes written are a function of the bytes read (so no load can be
 * dropped); their values carry no meaning.
 * Returns TQ_ERR_INVALID_ARG for NULL or misaligned pointers or sizes not a
 * multiple of 16, TQ_ERR_UNSUPPORTED for a stream of 2 GiB or more. */
tq_status tq_testing_stream(const void* src, size_t read_bytes, void* dst, size_t write_bytes,
                            int store_policy, int workgroups, void* stream);

/* tq_scores with the bound on a workgroup's wait for its segment's query pack
 * given in microseconds instead of 200: 0 makes every consumer workgroup that
 * does not find the pack published at once claim it or wait for its
 * claimant, the path tq_scores takes when a producer is not yet resident.
 * It always takes the one-launch form, whatever the pass's length.
 * Results are the same bytes as tq_scores.  Other arguments and errors as for
 * tq_scores; wait_us < 0 gives TQ_ERR_INVALID_ARG. */
tq_status tq_testing_scores_wait(const tq_params* kp, const float* q, int segs, int group, tq_cache keys,
                                 const int32_t* len, int64_t T, float* scores, void* ws, size_t ws_bytes,
                                 int wait_us, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_TESTING_H */
