// Device kernels of libvcoll for gfx950 (MI355X, CDNA4, wave64).
//
// The collectives of a p-rank virtual cluster run in one GPU's HBM, so the
// message hops of an algorithm are not data movement any more: an element's
// value after the collective is a fixed float32 expression over the p input
// values at that element. The reduce kernels evaluate that expression in
// registers, in the exact association the algorithm's steps produce, reading
// each input once and writing each output once -- an HBM-streaming pass with
// no reuse, so the design goals are coalesced 16-byte accesses, many bytes in
// flight per wave, and no arithmetic beyond the p-1 adds (no MFMA: nothing
// here is a contraction).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"
#include "order.h"
#include "vcoll.h"

namespace vcoll {

constexpr int kFixedMax = 16;        // largest p with a compile-time order program

// The p values with reduce kernels specialised at compile time; every other
// p runs the kernel that reads its order program at run time.
constexpr bool has_fixed_kernel(int p) { return p == 2 || p == 4 || p == 8 || p == 16; }

// Reduce (all-reduce / reduce-scatter). Grid: x = tiles of a chunk, y = chunk.
// For has_fixed_kernel(p), leaf[c * kFixedMax + k] is the buffer of the k-th input
// in chunk c's summation order (the host resolves the ring's per-chunk
// rotation and the trees' leaf order), so a workgroup fetches its p source
// pointers with one wide scalar load. For any other p, the ring has
// leaf[r] = send[r] and the kernel rotates it per chunk; the trees are given
// by the groups of their program (order_groups): leaf[q] is the buffer of
// group q's first leaf and leaf[kMaxRanks + q] that of its second (a folded
// pair) or null, for q < groups, so a kernel finds every buffer by the group
// index alone.
struct ReduceArgs {
  const void* leaf[kFixedMax * kFixedMax];
  void* dst[kMaxRanks];
  int64_t q, r;               // chunk c: off = c*q + min(c, r), count = q + (c < r)
  int32_t p;
  int32_t vec;                // every pointer 16-byte aligned: vector path allowed
  int32_t groups;             // tree programs with p not compiled in: the group count
  int32_t pace;               // space out the p-way store fan-out (large grids)
  int32_t align;              // all-reduce tiles start on this byte boundary (256 when every buffer
                              // has the same address mod 256, else 128 when mod 128, else 16)
  int32_t phase;              // that common address mod `align` (0 for align 16)
  int32_t src_align;          // 128 when every input buffer has address phase `src_phase` mod 128
  int32_t src_phase;          // (the unaligned reduce-scatter then loads whole lines), else 16 and 0
};
static_assert(sizeof(ReduceArgs) <= 4096, "kernel arguments are limited to 4 KiB");
static_assert(kFixedMax * kFixedMax >= 2 * kMaxRanks, "room for the groups' two leaves");

// grid y = chunks: p for all-reduce and reduce-scatter, 1 for a reduce to
// one root (q = n, r = 0, dst[0] = the root's buffer, scatter = true).
hipError_t launch_reduce(const ReduceArgs& a, vcoll_dtype dtype, vcoll_algo algo, bool scatter,
                         int64_t max_chunk, int chunks, hipStream_t stream);

// Ring all-reduce in two chip-wide phases, for vectors whose sums fit in the
// register files of one workgroup per compute unit: every workgroup reads
// its tile of all p ranks (chain order, the next rank's loads in flight while
// the current one is added), then writes the tile to all p outputs. Grid:
// x = tiles of a chunk, y = chunk. Requires 16-byte aligned buffers and
// chunks of a whole number of 16-byte vectors (n a multiple of p * 16 / s).
struct BurstArgs {
  const void* src[kMaxRanks];
  void* dst[kMaxRanks];
  int64_t q;                  // chunk length in elements: chunk c holds q + (c < r) of them
  int32_t r;
  int32_t p;
  int32_t tv;                 // 16-byte vectors per tile (a multiple of 8, at most burst_tile_max)
  int32_t align;              // 128: every buffer has address phase `phase` mod 128, tiles start on
  int32_t phase;              // 128-byte cache lines; 16: tiles start on any 16-byte boundary
  int32_t pad;
};

// First 16-byte vector of a burst tile in a chunk whose elements start at e0
// (VE elements per vector): the first whole vector, moved up to an `align`
// boundary of every buffer (which all have address phase `phase` mod align).
__host__ __device__ inline int64_t burst_first_vector(int64_t e0, int ve, int32_t align, int32_t phase) {
  const int64_t v = (e0 + ve - 1) / ve;
  const int64_t mis = (phase + v * 16) % align;
  return mis ? v + (align - mis) / 16 : v;
}
static_assert(sizeof(BurstArgs) <= 4096, "kernel arguments are limited to 4 KiB");

// Largest tile (16-byte vectors) one workgroup of the burst kernel holds.
int64_t burst_tile_max(vcoll_dtype dtype);

hipError_t launch_burst_ring(const BurstArgs& a, vcoll_dtype dtype, int tiles, hipStream_t stream);

}  // namespace vcoll
