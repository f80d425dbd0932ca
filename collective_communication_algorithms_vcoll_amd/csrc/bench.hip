// Streaming yardsticks for the benchmark (not collectives): how fast this GPU
// reads, writes and copies 16-byte vectors in the shapes that measured
// fastest on MI355X (400 MiB buffers cycled out of the Infinity Cache):
//   read  -- four-wave workgroups, 4 vectors per thread, non-temporal loads;
//   write -- one-wave workgroups, 4 vectors per thread, non-temporal stores
//            that also bypass both cache levels (sc0 sc1 nt);
//   copy  -- one-wave workgroups, 2 vectors per thread, non-temporal loads,
//            sc0 sc1 nt stores;
//   plain copy -- the earlier yardstick: four-wave workgroups, 4 vectors per
//            thread, non-temporal loads and stores.
// Tiles use buffer instructions whose resource size is the tile's valid
// bytes, so the last, partial tile needs no masks.
#include "bench.h"
#include "device.h"

namespace vcoll {
namespace {

using namespace dev;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t span(const void* base, int64_t byte_off, int64_t total) {
  const int64_t left = total - byte_off;
  return raw_rsrc(base, byte_off, static_cast<int>(left < (int64_t(1) << 30) ? left : (int64_t(1) << 30)));
}

template <int V, int BS, int SPOL>
__global__ __launch_bounds__(BS) void copy_kernel(const void* src, void* dst, int64_t bytes) {
  const int64_t off = static_cast<int64_t>(blockIdx.x) * (V * BS * 16);
  const __amdgpu_buffer_rsrc_t s = span(src, off, bytes);
  const __amdgpu_buffer_rsrc_t d = span(dst, off, bytes);
  u32x4 x[V];
#pragma unroll
  for (int j = 0; j < V; ++j)
    x[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(s, threadIdx.x * 16, j * BS * 16, kPolicyNT));
#pragma unroll
  for (int j = 0; j < V; ++j)
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x[j]), d, threadIdx.x * 16, j * BS * 16, SPOL);
}

// Reads every byte once; the xor of what a thread read goes to `sink` only
// when it equals `never` (a value the host picks), so the loads cannot be
// dropped and almost never cost a store.
template <int V, int BS>
__global__ __launch_bounds__(BS) void read_kernel(const void* src, void* sink, int64_t bytes, uint32_t never) {
  const int64_t off = static_cast<int64_t>(blockIdx.x) * (V * BS * 16);
  const __amdgpu_buffer_rsrc_t s = span(src, off, bytes);
  u32x4 acc = {0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < V; ++j)
    acc ^= __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(s, threadIdx.x * 16, j * BS * 16, kPolicyNT));
  const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == never) static_cast<uint32_t*>(sink)[0] = x;
}

template <int V, int BS>
__global__ __launch_bounds__(BS) void write_kernel(void* dst, int64_t bytes) {
  const int64_t off = static_cast<int64_t>(blockIdx.x) * (V * BS * 16);
  const __amdgpu_buffer_rsrc_t d = span(dst, off, bytes);
  const u32x4 v = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < V; ++j)
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), d, threadIdx.x * 16, j * BS * 16, kPolicyThrough);
}

template <int V, int BS>
unsigned tiles_of(int64_t bytes) {
  const int64_t per = static_cast<int64_t>(V) * BS * 16;
  return static_cast<unsigned>((bytes + per - 1) / per);
}

}  // namespace

hipError_t launch_stream(vcoll_bench_kind kind, void* dst, const void* src, int64_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  switch (kind) {
    case VCOLL_BENCH_COPY: {
      void* args[] = {&src, &dst, &bytes};
      return hipLaunchKernel(reinterpret_cast<const void*>(copy_kernel<2, 64, kPolicyThrough>),
                             dim3(tiles_of<2, 64>(bytes)), dim3(64), args, 0, stream);
    }
    case VCOLL_BENCH_COPY_PLAIN: {
      void* args[] = {&src, &dst, &bytes};
      return hipLaunchKernel(reinterpret_cast<const void*>(copy_kernel<4, 256, kPolicyNT>),
                             dim3(tiles_of<4, 256>(bytes)), dim3(256), args, 0, stream);
    }
    case VCOLL_BENCH_READ: {
      uint32_t never = 0x7fc00001u;               // a NaN payload, xor of reads of finite data almost never hits it
      void* args[] = {&src, &dst, &bytes, &never};
      return hipLaunchKernel(reinterpret_cast<const void*>(read_kernel<4, 256>), dim3(tiles_of<4, 256>(bytes)),
                             dim3(256), args, 0, stream);
    }
    default: {
      void* args[] = {&dst, &bytes};
      return hipLaunchKernel(reinterpret_cast<const void*>(write_kernel<4, 64>), dim3(tiles_of<4, 64>(bytes)),
                             dim3(64), args, 0, stream);
    }
  }
}

}  // namespace vcoll
