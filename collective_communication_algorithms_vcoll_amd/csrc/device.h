// Device-side building blocks shared by libvcoll's kernels (gfx950, wave64):
// storage types, 16-byte streaming access, compile-time loops, store pacing
// and the launch helper.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "common.h"

namespace vcoll {
namespace dev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ----------------------------------------------------------------------------
// storage types: float32, or bfloat16 widened exactly and rounded once

// Round a float32 to bfloat16, nearest with ties to even, on the bit pattern:
// adding 0x7FFF plus the lowest kept bit carries exactly when the dropped half
// is above the midpoint, or at it with an odd kept part. NaN stays NaN (quiet).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int D>
struct Storage;

template <>
struct Storage<VCOLL_F32> {
  static constexpr int kVE = 4;  // elements per 16 bytes
  using elem = uint32_t;
  __device__ static __forceinline__ void widen(const u32x4 w, float* f) {
    f[0] = __uint_as_float(w.x);
    f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z);
    f[3] = __uint_as_float(w.w);
  }
  __device__ static __forceinline__ u32x4 narrow(const float* f) {
    u32x4 w;
    w.x = __float_as_uint(f[0]);
    w.y = __float_as_uint(f[1]);
    w.z = __float_as_uint(f[2]);
    w.w = __float_as_uint(f[3]);
    return w;
  }
  __device__ static __forceinline__ float widen1(elem e) { return __uint_as_float(e); }
  __device__ static __forceinline__ elem narrow1(float f) { return __float_as_uint(f); }
};

template <>
struct Storage<VCOLL_BF16> {
  static constexpr int kVE = 8;
  using elem = uint16_t;
  __device__ static __forceinline__ void widen(const u32x4 w, float* f) {
    f[0] = __uint_as_float(w.x << 16);
    f[1] = __uint_as_float(w.x & 0xffff0000u);
    f[2] = __uint_as_float(w.y << 16);
    f[3] = __uint_as_float(w.y & 0xffff0000u);
    f[4] = __uint_as_float(w.z << 16);
    f[5] = __uint_as_float(w.z & 0xffff0000u);
    f[6] = __uint_as_float(w.w << 16);
    f[7] = __uint_as_float(w.w & 0xffff0000u);
  }
  __device__ static __forceinline__ u32x4 narrow(const float* f) {
    u32x4 w;
    w.x = bf16_rne(f[0]) | (bf16_rne(f[1]) << 16);
    w.y = bf16_rne(f[2]) | (bf16_rne(f[3]) << 16);
    w.z = bf16_rne(f[4]) | (bf16_rne(f[5]) << 16);
    w.w = bf16_rne(f[6]) | (bf16_rne(f[7]) << 16);
    return w;
  }
  __device__ static __forceinline__ float widen1(elem e) { return __uint_as_float(uint32_t(e) << 16); }
  __device__ static __forceinline__ elem narrow1(float f) { return static_cast<elem>(bf16_rne(f)); }
};

// ----------------------------------------------------------------------------
// memory access: 16-byte vectors, streamed (each byte is touched once)

__device__ __forceinline__ u32x4 ld16(const void* base, int64_t byte_off) {
  return __builtin_nontemporal_load(
      reinterpret_cast<const u32x4*>(static_cast<const char*>(base) + byte_off));
}

__device__ __forceinline__ void st16(void* base, int64_t byte_off, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(static_cast<char*>(base) + byte_off));
}

// Buffer-instruction access: a resource whose base is the same for the whole
// wave (a tile start in one buffer) and whose size clips the accesses (loads
// past it return 0, stores past it are dropped); each lane adds a 32-bit
// offset. A per-lane base would make the compiler loop over the distinct
// bases, so callers keep the base uniform. Cache-policy bits of gfx950
// buffer instructions: sc0 = 1, nt = 2, sc1 = 16.
constexpr int kRawBufferFormat = 0x00020000;    // dword 3 of a raw (untyped) buffer resource
constexpr int kPolicyCached = 0;                // default: through L2, which merges partial lines
constexpr int kPolicyNT = 2;                    // non-temporal
constexpr int kPolicyThrough = 1 | 2 | 16;      // sc0 | nt | sc1: streamed past every cache level

__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, int64_t byte_off, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(static_cast<const char*>(base)) + byte_off, 0, bytes,
                                           kRawBufferFormat);
}

template <int K, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (K < N) {
    f(std::integral_constant<int, K>{});
    static_for<K + 1, N>(f);
  }
}

// Store pacing: in large grids (a.pace; the LARGE kernel variant when p is
// compiled in) a wave pauses about 64*VCOLL_STORE_SLEEP
// cycles between the p ranks it stores to. When every wave of a large grid
// bursts its p loads and then its p-way store fan-out at once, the streams
// collide in the DRAM rows; spacing the stores out raised the p = 8
// all-reduce by 3% (25 MiB per rank) to 8% (80 MiB), the p = 16 bf16 one by
// 1-3%, on MI355X. Small, latency-bound launches lose, so the host sets
// a.pace only for grids that fill the chip several times over. (The
// all-gather, one load per p stores, does not gain.)
#ifndef VCOLL_STORE_SLEEP
#define VCOLL_STORE_SLEEP 4
#endif

// Workgroups from which a launch paces its stores (see VCOLL_STORE_SLEEP).
#ifndef VCOLL_PACE_MIN_GROUPS
#define VCOLL_PACE_MIN_GROUPS 2048
#endif

template <class K, class Arg>
hipError_t launch(K kernel, dim3 grid, const Arg& arg, hipStream_t stream) {
  void* args[] = {const_cast<Arg*>(&arg)};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, dim3(kBlock), args, 0, stream);
}

template <class K, class Arg>
hipError_t launch(K kernel, dim3 grid, int block, const Arg& arg, hipStream_t stream) {
  void* args[] = {const_cast<Arg*>(&arg)};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, dim3(block), args, 0, stream);
}

}  // namespace dev
}  // namespace vcoll
