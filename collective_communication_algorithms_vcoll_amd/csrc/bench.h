// Launch interface of the streaming yardsticks (bench.hip): plain read,
// write and copy kernels that the benchmark times beside the collectives.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "vcoll_bench.h"

namespace vcoll {

hipError_t launch_stream(vcoll_bench_kind kind, void* dst, const void* src, int64_t bytes, hipStream_t stream);

}  // namespace vcoll
