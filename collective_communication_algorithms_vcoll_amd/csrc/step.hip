// The stepwise (one launch per algorithm step) all-reduce kernel of libvcoll.
#include <mutex>

#include "device.h"
#include "step.h"

namespace vcoll {
namespace {

using namespace dev;

// ----------------------------------------------------------------------------
// stepwise all-reduce: the operations of one algorithm step on float32
// working buffers (one launch per step, messages moved through memory)

__device__ __forceinline__ float round_bf16(float f) { return __uint_as_float(bf16_rne(f) << 16); }

// Four consecutive elements of an operation, vector or scalar access.
__device__ __forceinline__ void step_apply4(const StepLaunchOp& o, int64_t e, bool vec) {
  float* d = static_cast<float*>(o.dst);
  const float* sf = static_cast<const float*>(o.src);
  float x[4], y[4];
  switch (o.kind) {
    case SK_ADD:
    case SK_XADD:
      if (vec) {
        const u32x4 a = ld16(o.src, e * 4), b = ld16(o.dst, e * 4);
        for (int i = 0; i < 4; ++i) { x[i] = __uint_as_float(a[i]); y[i] = __uint_as_float(b[i]); }
      } else {
        for (int i = 0; i < 4; ++i) { x[i] = sf[e + i]; y[i] = d[e + i]; }
      }
      for (int i = 0; i < 4; ++i) y[i] = y[i] + x[i];
      if (vec) {
        const u32x4 r = {__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]), __float_as_uint(y[3])};
        st16(o.dst, e * 4, r);
        if (o.kind == SK_XADD) st16(const_cast<void*>(o.src), e * 4, r);
      } else {
        for (int i = 0; i < 4; ++i) {
          d[e + i] = y[i];
          if (o.kind == SK_XADD) const_cast<float*>(sf)[e + i] = y[i];
        }
      }
      break;
    case SK_COPY:
      if (vec) st16(o.dst, e * 4, ld16(o.src, e * 4));
      else for (int i = 0; i < 4; ++i) d[e + i] = sf[e + i];
      break;
    case SK_COPY16: {
      // four 16-bit elements: one 8-byte access when both ends allow it
      if (vec) {
        static_cast<uint64_t*>(o.dst)[e / 4] = static_cast<const uint64_t*>(o.src)[e / 4];
      } else {
        for (int i = 0; i < 4; ++i) static_cast<uint16_t*>(o.dst)[e + i] = static_cast<const uint16_t*>(o.src)[e + i];
      }
      break;
    }
    case SK_NARROW:
      for (int i = 0; i < 4; ++i) d[e + i] = round_bf16(d[e + i]);
      break;
    case SK_WIDEN_BF16: {
      const uint16_t* sb = static_cast<const uint16_t*>(o.src);
      for (int i = 0; i < 4; ++i) d[e + i] = __uint_as_float(uint32_t(sb[e + i]) << 16);
      break;
    }
    default: {  // SK_STORE_BF16
      uint16_t* db = static_cast<uint16_t*>(o.dst);
      for (int i = 0; i < 4; ++i) db[e + i] = static_cast<uint16_t>(bf16_rne(sf[e + i]));
      break;
    }
  }
}

__device__ __forceinline__ void step_apply1(const StepLaunchOp& o, int64_t e) {
  float* d = static_cast<float*>(o.dst);
  const float* sf = static_cast<const float*>(o.src);
  switch (o.kind) {
    case SK_ADD: d[e] = d[e] + sf[e]; break;
    case SK_XADD: { const float v = d[e] + sf[e]; d[e] = v; const_cast<float*>(sf)[e] = v; break; }
    case SK_COPY: d[e] = sf[e]; break;
    case SK_COPY16: static_cast<uint16_t*>(o.dst)[e] = static_cast<const uint16_t*>(o.src)[e]; break;
    case SK_NARROW: d[e] = round_bf16(d[e]); break;
    case SK_WIDEN_BF16: d[e] = __uint_as_float(uint32_t(static_cast<const uint16_t*>(o.src)[e]) << 16); break;
    default: static_cast<uint16_t*>(o.dst)[e] = static_cast<uint16_t>(bf16_rne(sf[e])); break;
  }
}

__global__ __launch_bounds__(kBlock) void step_kernel(const StepArgs a) {
  const int t = blockIdx.x;
  int lo = 0, hi = a.nops - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (a.op[mid].tile_start <= t) lo = mid;
    else hi = mid - 1;
  }
  const StepLaunchOp& o = a.op[lo];
  const int64_t e0 = static_cast<int64_t>(t - o.tile_start) * kStepTile;
  const int64_t e1 = o.count < e0 + kStepTile ? o.count : e0 + kStepTile;
  // float32 sides move as 16-byte vectors when both ends are aligned, 16-bit
  // copies as 8-byte words when both ends are 8-byte aligned (e is a
  // multiple of 4 elements in every group)
  const uintptr_t ends = reinterpret_cast<uintptr_t>(o.src) | reinterpret_cast<uintptr_t>(o.dst);
  const bool vec = o.kind == SK_COPY16 ? (ends & 7u) == 0
                                       : (o.kind == SK_ADD || o.kind == SK_XADD || o.kind == SK_COPY) && (ends & 15u) == 0;
  const int64_t groups = (e1 - e0) / 4;
  for (int64_t g = threadIdx.x; g < groups; g += kBlock) step_apply4(o, e0 + 4 * g, vec);
  const int64_t tail = e0 + 4 * groups + threadIdx.x;
  if (tail < e1) step_apply1(o, tail);
}

// Float32 partial sums of the allocation-free stepwise all-reduce (bf16
// inputs): one copy per GPU, owned by the library. Host code never passes
// this name to a kernel (on the host it is only a stand-in for the symbol);
// it uses the device address that step_scratch() looks up.
static __device__ __align__(256) float scratch[VCOLL_STEP_SCRATCH_BYTES / sizeof(float)];

constexpr int kScratchDevices = 64;

}  // namespace

hipError_t launch_step(const StepArgs& a, int32_t tiles, hipStream_t stream) {
  if (tiles == 0) return hipSuccess;
  return launch(step_kernel, dim3(static_cast<unsigned>(tiles)), a, stream);
}

hipError_t step_scratch(void** ptr) {
  static std::mutex mu;
  static void* per_device[kScratchDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!per_device[dev]) {
    // each GPU holds its own copy of the array at its own address: look it
    // up with this device current, once
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!addr) return hipErrorInvalidSymbol;
    per_device[dev] = addr;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

}  // namespace vcoll
