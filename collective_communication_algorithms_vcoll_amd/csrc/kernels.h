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

#include "order.h"
#include "vcoll.h"

namespace vcoll {

constexpr int kBlock = 256;          // threads per workgroup (4 waves)
constexpr int kA2ABlocks = 64;       // all-to-all blocks described per launch
constexpr int kFixedMax = 16;        // largest p with a compile-time order program

// The p values with reduce kernels specialised at compile time; every other
// p runs the kernel that reads its order program at run time.
constexpr bool has_fixed_kernel(int p) { return p == 2 || p == 4 || p == 8 || p == 16; }

struct RankPtrs {
  const void* src[kMaxRanks];
  void* dst[kMaxRanks];
};

// Reduce (all-reduce / reduce-scatter). Grid: x = tiles of a chunk, y = chunk.
// For has_fixed_kernel(p), leaf[c * kFixedMax + k] is the buffer of the k-th input
// in chunk c's summation order (the host resolves the ring's per-chunk
// rotation and the trees' leaf order), so a workgroup fetches its p source
// pointers with one wide scalar load. For any other p, leaf[r] = send[r] and
// the kernel resolves the order itself.
struct ReduceArgs {
  const void* leaf[kFixedMax * kFixedMax];
  void* dst[kMaxRanks];
  int64_t q, r;               // chunk c: off = c*q + min(c, r), count = q + (c < r)
  int32_t p;
  int32_t vec;                // every pointer 16-byte aligned: vector path allowed
  int32_t final_merges;       // order program (used when p is not compiled in)
  int32_t pace;               // space out the p-way store fan-out (large grids)
  uint8_t rank[kMaxRanks];
  uint8_t merges[kMaxRanks];
};

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

// Broadcast: the root's n elements copied to q receive buffers. Grid: x = tiles.
struct BcastArgs {
  const void* src;
  void* dst[kMaxRanks];
  int64_t n;
  int32_t q;
  int32_t vec;                // every pointer 16-byte aligned
};

// All-gather. Grid: x = tiles of one block, y = source rank.
struct GatherArgs {
  RankPtrs ptr;
  int64_t m;                  // elements per rank
  int32_t p;
  int32_t vec;                // pointers aligned and m * esize a multiple of 16
};

// One (i -> j) block of an all-to-all.
struct A2ABlock {
  const char* src;            // first row (contiguous) or gather table base
  char* dst;                  // first row (contiguous) or scatter table base
  const int32_t* src_idx;     // per-row gather index, or nullptr
  const int32_t* dst_idx;     // per-row scatter index, or nullptr
  int32_t rows;
  int32_t tile_start;         // first workgroup of this block
  int32_t src_limit;          // rows of the gather table (index bound)
  int32_t dst_limit;          // rows of the scatter table (index bound)
};

// Stepwise all-reduce: one launch applies up to kStepOps operations of one
// step to float32 working buffers (kinds as in schedule.h, plus the widening
// of bfloat16 inputs and the final bfloat16 store). src/dst point at the
// operation's first element.
constexpr int kStepOps = 64;
constexpr int kStepTile = 4096;      // elements per workgroup
enum StepLaunchKind : int32_t {
  SK_ADD = 0, SK_COPY = 1, SK_XADD = 2, SK_NARROW = 3, SK_WIDEN_BF16 = 4, SK_STORE_BF16 = 5
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

struct A2AArgs {
  int64_t row_bytes;
  int32_t nblocks;
  int32_t rows_per_tile;
  int32_t vec;                // row_bytes % 16 == 0 and all bases aligned
  int32_t esize;
  A2ABlock b[kA2ABlocks];
};

// FP8 dispatch: per (block, row tile) workgroup as the all-to-all, each row
// gathered from a bfloat16 token table and quantised on the way.
struct Fp8Args {
  int64_t hidden;             // elements per row, a multiple of 128
  int64_t out_row_bytes;      // hidden + hidden / 32
  int32_t nblocks;
  int32_t rows_per_tile;
  A2ABlock b[kA2ABlocks];     // src = token table, src_idx = gather map, dst = first row of the block
};

// Launchers (return hipError_t of the launch).
// grid y = chunks: p for all-reduce and reduce-scatter, 1 for a reduce to
// one root (q = n, r = 0, dst[0] = the root's buffer, scatter = true).
hipError_t launch_reduce(const ReduceArgs& a, vcoll_dtype dtype, vcoll_algo algo, bool scatter,
                         int64_t max_chunk, int chunks, hipStream_t stream);
hipError_t launch_broadcast(const BcastArgs& a, vcoll_dtype dtype, hipStream_t stream);
hipError_t launch_dispatch_fp8(const Fp8Args& a, int32_t tiles, hipStream_t stream);
hipError_t launch_all_gather(const GatherArgs& a, vcoll_dtype dtype, hipStream_t stream);
hipError_t launch_all_to_all(const A2AArgs& a, int32_t tiles, hipStream_t stream);
hipError_t launch_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream);
hipError_t launch_step(const StepArgs& a, int32_t tiles, hipStream_t stream);
hipError_t launch_hierarchical(const HierArgs& a, vcoll_dtype dtype, int64_t max_segment, hipStream_t stream);

}  // namespace vcoll
