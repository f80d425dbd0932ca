/*
 * libvcoll measurement helper: not a collective.
 *
 * The collectives are HBM-streaming passes, so their natural yardstick is a
 * plain streaming copy with the same access pattern (16-byte vectors,
 * non-temporal hints). The benchmark times this copy in the same run to give
 * the practical bandwidth ceiling, and uses its hardware counter readings to
 * scale the collectives' counter readings into bytes.
 */
#ifndef VCOLL_BENCH_H
#define VCOLL_BENCH_H

#include <stdint.h>

#include "vcoll.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Copy `bytes` bytes from device buffer src to device buffer dst on `stream`
 * (a hipStream_t). bytes must be a multiple of 16 and both pointers 16-byte
 * aligned, else VCOLL_ERR_INVALID_ARG; the buffers must not overlap. */
vcoll_status vcoll_bench_copy(void* dst, const void* src, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VCOLL_BENCH_H */
