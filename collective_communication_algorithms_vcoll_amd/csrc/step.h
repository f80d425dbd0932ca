// Launch interface of the stepwise all-reduce kernel (step.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"
#include "vcoll.h"

namespace vcoll {

// Stepwise all-reduce: one launch applies up to kStepOps operations of one
// step to float32 working buffers (kinds as in schedule.h, plus the widening
// of bfloat16 inputs and the final bfloat16 store). src/dst point at the
// operation's first element.
constexpr int kStepOps = 64;
constexpr int kStepTile = 4096;      // elements per workgroup
enum StepLaunchKind : int32_t {
  SK_ADD = 0, SK_COPY = 1, SK_XADD = 2, SK_NARROW = 3, SK_WIDEN_BF16 = 4, SK_STORE_BF16 = 5,
  SK_COPY16 = 6              // raw copy of 16-bit elements (bf16 messages of the stepwise broadcast)
};
struct StepLaunchOp {
  const void* src;
  void* dst;
  int64_t count;
  int32_t kind;
  int32_t tile_start;
};
struct StepArgs {
  int32_t nops;
  int32_t pad;
  StepLaunchOp op[kStepOps];
};

hipError_t launch_step(const StepArgs& a, int32_t tiles, hipStream_t stream);

// Device address, on the current device, of the library's own float32 scratch
// array (VCOLL_STEP_SCRATCH_BYTES, one copy per GPU, alive until the process
// ends) for the allocation-free stepwise all-reduce. The address is looked up
// once per device and cached.
hipError_t step_scratch(void** ptr);

}  // namespace vcoll
