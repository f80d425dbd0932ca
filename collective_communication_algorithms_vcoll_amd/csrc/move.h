// Launch interface of the data-movement kernels (move.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"
#include "vcoll.h"

namespace vcoll {

constexpr int kA2ABlocks = 64;       // all-to-all blocks described per launch

// All-gather. Grid: x = tiles of one block, y = source rank.
struct GatherArgs {
  RankPtrs ptr;
  int64_t m;                  // elements per rank
  int32_t p;
  int32_t vec;                // pointers aligned and m * esize a multiple of 16
  int32_t lines;              // every output on a 128-byte line and m * esize a multiple of 128
  int32_t pad;
};

// Broadcast: the root's n elements copied to q receive buffers. Grid: x = tiles.
struct BcastArgs {
  const void* src;
  void* dst[kMaxRanks];
  int64_t n;
  int32_t q;
  int32_t vec;                // every pointer 16-byte aligned
  int32_t lines;              // every receive buffer on a 128-byte line
  int32_t pad;
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
  int32_t vec_out;            // receive rows 16-byte aligned: 16-byte code stores
  int32_t pad;
  A2ABlock b[kA2ABlocks];     // src = token table, src_idx = gather map, dst = first row of the block
};

// Token-major MoE dispatch. Grid: x = tiles of tokens, y = sending rank i:
// token t of rank i goes to row slots[i][2(t*topk+k)+1] of rank
// slots[i][2(t*topk+k)] for every slot k.
struct PushArgs {
  const void* table[kMaxRanks];      // each rank's token rows
  const int32_t* slots[kMaxRanks];   // each rank's [tokens * topk][2] (destination rank, row)
  void* recv[kMaxRanks];
  int32_t recv_rows[kMaxRanks];
  int64_t tokens;
  int64_t row_bytes;          // bytes of a token row
  int64_t out_row_bytes;      // bytes of a received row (row_bytes, or hidden + hidden/32 for FP8)
  int64_t hidden;             // elements per row (FP8: a multiple of 128)
  int32_t topk, p;
  int32_t vec;                // rows and bases 16-byte aligned (copy path)
  int32_t tokens_per_tile;
  int32_t vec_out;            // FP8: receive rows 16-byte aligned (16-byte code stores)
  int32_t segments;           // workgroups per tile, each one segment of every row (push_segments)
};
static_assert(sizeof(PushArgs) <= 4096, "kernel arguments are limited to 4 KiB");

// Token-major MoE combine: rank i's row t*topk + k is pulled from row r of
// expert-output buffer j, (j, r) = slots[i][t*topk + k] (the dispatch's slot).
struct CombineArgs {
  const void* src[kMaxRanks];        // each rank's expert-output rows (dispatch receive layout)
  void* out[kMaxRanks];              // each rank's [tokens * topk] combined rows
  const int32_t* slots[kMaxRanks];   // each rank's [tokens * topk][2] (source rank, row)
  int32_t src_rows[kMaxRanks];
  int64_t tokens;
  int64_t row_bytes;
  int32_t topk, p;
  int32_t vec;                       // rows and bases 16-byte aligned
  int32_t tokens_per_tile;
  int32_t segments;                  // workgroups per tile, each one segment of every row (pull_segments)
  int32_t pad;
};
static_assert(sizeof(CombineArgs) <= 4096, "kernel arguments are limited to 4 KiB");

hipError_t launch_all_gather(const GatherArgs& a, vcoll_dtype dtype, hipStream_t stream);
hipError_t launch_broadcast(const BcastArgs& a, vcoll_dtype dtype, hipStream_t stream);
hipError_t launch_all_to_all(const A2AArgs& a, int32_t tiles, hipStream_t stream);
hipError_t launch_dispatch_fp8(const Fp8Args& a, int32_t tiles, hipStream_t stream);
// Workgroups that share one tile of token rows, each copying one segment of
// every row (1 when rows are short, FP8 or not 16-byte aligned).
int32_t push_segments(int64_t row_bytes, bool fp8, bool vec);
int32_t pull_segments(int64_t row_bytes, bool vec);
hipError_t launch_dispatch_push(const PushArgs& a, bool fp8, hipStream_t stream);
hipError_t launch_combine_pull(const CombineArgs& a, hipStream_t stream);

}  // namespace vcoll
