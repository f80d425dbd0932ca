// Shared by libvcoll's host code and kernels: workgroup size and the table of
// per-rank buffer pointers.
#pragma once

#include <cstdint>

#include "order.h"
#include "vcoll.h"

namespace vcoll {

constexpr int kBlock = 256;          // threads per workgroup (4 waves)

struct RankPtrs {
  const void* src[kMaxRanks];
  void* dst[kMaxRanks];
};

}  // namespace vcoll
