/*
 * libvcoll measurement helpers: not collectives.
 *
 * The collectives are HBM-streaming passes, so their natural yardsticks are
 * plain streams of 16-byte vectors: how fast this GPU reads, writes and
 * copies. The benchmark times them in the same run as the collectives (the
 * practical ceilings) and scales the collectives' hardware counter readings
 * by the copy's readings.
 */
#ifndef VCOLL_BENCH_H
#define VCOLL_BENCH_H

#include <stdint.h>

#include "vcoll.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VCOLL_BENCH_COPY = 0,        /* src -> dst, the fastest copy shape measured (one-wave workgroups,
                                  2 vectors per thread, stores that bypass the caches) */
  VCOLL_BENCH_READ = 1,        /* read src; dst is a sink of at least 4 bytes that is almost never written */
  VCOLL_BENCH_WRITE = 2,       /* write zeros to dst; src unused (may be NULL) */
  VCOLL_BENCH_COPY_PLAIN = 3   /* src -> dst, four-wave workgroups, 4 vectors per thread, streaming stores */
} vcoll_bench_kind;

/* One streaming pass of `bytes` bytes on `stream` (a hipStream_t). bytes
 * must be a multiple of 16 and the pointers it uses 16-byte aligned (dst of
 * READ: 4-byte aligned), else VCOLL_ERR_INVALID_ARG; src and dst must not
 * overlap. */
vcoll_status vcoll_bench_stream(vcoll_bench_kind kind, void* dst, const void* src, int64_t bytes, void* stream);

/* vcoll_bench_stream(VCOLL_BENCH_COPY, dst, src, bytes, stream). */
vcoll_status vcoll_bench_copy(void* dst, const void* src, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VCOLL_BENCH_H */
