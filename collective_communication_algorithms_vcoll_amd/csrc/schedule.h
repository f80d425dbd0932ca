// Host-side schedules of the virtual-cluster collectives: chunk partition,
// summation-order programs, message ledger, MoE plan. No HIP dependency.
#pragma once

#include <cstdint>
#include <vector>

#include "order.h"
#include "vcoll.h"

namespace vcoll {

// Balanced partition of n elements into p chunks (first n mod p chunks one longer).
struct Chunks {
  int64_t q = 0, r = 0;
  int p = 1;
  Chunks(int64_t n, int p_) : q(n / p_), r(n % p_), p(p_) {}
  int64_t off(int c) const { return c * q + (c < r ? c : r); }
  int64_t count(int c) const { return q + (c < r ? 1 : 0); }
};

// Checks (op, algo, p) and returns VCOLL_OK or VCOLL_ERR_UNSUPPORTED.
vcoll_status check_combination(vcoll_op op, vcoll_algo algo, int p);

// Messages of op/algo, sorted by (step, src, dst, src_off); sets *n_steps.
vcoll_status build_ledger(vcoll_op op, vcoll_algo algo, int p, int64_t n, int64_t elem_bytes,
                          const int64_t* splits, int64_t row_elems,
                          std::vector<vcoll_msg>& out, int32_t* n_steps);

// Row offsets of block (i -> j): in the sender's buffer and in the receiver's.
void block_offsets(int p, const int64_t* splits, std::vector<int64_t>& send_off,
                   std::vector<int64_t>& recv_off);

// Hierarchical / 2D all-reduce of nodes x local ranks (rank = g*local + l):
// ring reduce-scatter inside each group over `local` chunks, ring all-reduce
// of chunk l across the same-index ranks (chunk l cut into `nodes` pieces),
// ring all-gather inside each group; all rings of a phase in lockstep.
vcoll_status build_ledger_hierarchical(int nodes, int local, int64_t n, int64_t elem_bytes,
                                       std::vector<vcoll_msg>& out, int32_t* n_steps);

// Broadcast (op VCOLL_OP_BROADCAST; algo BINARY_TREE, NAIVE,
// SCATTER_ALLGATHER or PIPELINED_CHAIN with `blocks` blocks) or binomial
// reduce (VCOLL_OP_REDUCE, BINARY_TREE) rooted at `root`; ranks are taken
// relative to the root, v = (r - root) mod p.
vcoll_status build_ledger_rooted(vcoll_op op, vcoll_algo algo, int p, int64_t n, int64_t elem_bytes, int root,
                                 int64_t blocks, std::vector<vcoll_msg>& out, int32_t* n_steps);

// One operation of a step of the stepwise (unfused) all-reduce, on float32
// working buffers W[r] of n elements, over elements [off, off + count):
//   ADD    W[dst] += W[src]          (the receiver adds what arrives)
//   COPY   W[dst]  = W[src]
//   XADD   W[src] = W[dst] = W[src] + W[dst]   (both partners of an exchange)
//   NARROW W[dst] = W[dst] rounded to bfloat16 (a finished result, once)
// Operations of one step never read what another operation of the same step
// writes, so a step may run as any number of launches in sequence.
// With bfloat16 storage, the NARROW operations form one step of their own,
// right after the last adding step.
enum StepKind : int32_t { STEP_ADD = 0, STEP_COPY = 1, STEP_XADD = 2, STEP_NARROW = 3 };

struct StepOp {
  int32_t kind, src, dst;
  int64_t off, count;
};

// Steps of `algo`'s all-reduce; message steps follow build_ledger exactly.
// Returns the number of message steps (steps.size() is one more when
// `narrow` adds the rounding step).
int build_step_program(vcoll_algo algo, int p, int64_t n, bool narrow,
                       std::vector<std::vector<StepOp>>& steps);

vcoll_status moe_plan(int p, int64_t tokens, int topk, int experts_per_rank,
                      const int32_t* topk_ids, int64_t* splits, int32_t* src_rows,
                      int32_t* dst_rows);

// Deduplicated dispatch plan (one row per (token, destination rank)) and the
// expansion map back to the plain layout of moe_plan; see vcoll.h.
vcoll_status moe_plan_dedup(int p, int64_t tokens, int topk, int experts_per_rank,
                            const int32_t* topk_ids, int64_t* splits_unique, int32_t* src_unique,
                            int32_t* expand, int64_t* expand_count);

// Token-major view of a moe_plan: slots[i][2(t*topk+k)] = destination rank,
// [.. + 1] = row in that rank's receive buffer, of rank i's pair (t, k).
vcoll_status moe_slots(int p, int64_t tokens, int topk, const int64_t* splits, const int32_t* dst_rows,
                       int32_t* slots);

// Token-major form of one rank's deduplicated-dispatch expansion: for each
// unique row u, the plain rows x with expand[x] == u as (0, x) pairs in
// ascending x, padded with (-1, -1) to topk; see vcoll.h.
vcoll_status moe_expand_slots(int64_t unique_rows, int topk, const int32_t* expand, int64_t expand_count,
                              int32_t* slots);

// Token-major form of a deduplicated dispatch plan: for rank i's token t,
// the (destination rank, row of its deduplicated receive buffer) of each
// copy, in ascending destination order, padded with (-1, -1) to `width`;
// see vcoll.h.
vcoll_status moe_dedup_slots(int p, int64_t tokens, int width, const int64_t* splits_unique,
                             const int32_t* src_unique, int32_t* slots);

}  // namespace vcoll
