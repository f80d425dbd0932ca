// Launch interface of the hierarchical / 2D all-reduce kernel (hier.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"
#include "vcoll.h"

namespace vcoll {

// Hierarchical / 2D all-reduce of nodes x local ranks. Grid: x = tiles of a
// segment, y = segment u = l * nodes + j (piece j of chunk l), inside which
// the summation order is fixed.
struct HierArgs {
  RankPtrs ptr;
  int64_t n;
  int32_t nodes, local;
  int32_t vec;
  int32_t pad;
};

hipError_t launch_hierarchical(const HierArgs& a, vcoll_dtype dtype, int64_t max_segment, hipStream_t stream);

}  // namespace vcoll
