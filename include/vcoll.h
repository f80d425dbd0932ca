/*
 * libvcoll -- collectives of a single-GPU "virtual cluster" on MI355X (gfx950).
 *
 * p logical ranks each own one buffer in the same GPU's memory. The library
 * computes what the collective leaves in every rank's buffer, reproducing
 * each algorithm's summation order exactly, in one streaming pass over the
 * buffers; the step-by-step message traffic the algorithm would put on a
 * network is reported separately by vcoll_ledger().
 *
 * Sources, by page title:
 *   [NCC] "Networks and Collective Communication" (semidirectx, cs349e
 *         prerequisite lecture 5): semantics section 4.1, identities 4.2,
 *         per-device bytes 4.3, ring 5.1, recursive doubling / Rabenseifner /
 *         binary tree 5.2, MoE all-to-all 7.4.
 *   [HPC] "11-1. Distributed training" (HPC101 notes): "Collective
 *         Communication Primitives", "Ring Algorithm".
 *   [LDT] "LLM Distributed Training Collectives": "Ring AllReduce".
 *
 * Common conventions
 *   - Every function returns a vcoll_status; nothing throws across the ABI.
 *   - All arguments are validated before anything is enqueued: a return
 *     other than VCOLL_ERR_HIP means no work was launched. (Calls that
 *     enqueue several launches -- the stepwise all-reduce, all-to-alls and
 *     FP8 dispatches of more than 64 non-empty blocks -- may have enqueued
 *     earlier launches when a later one returns VCOLL_ERR_HIP.)
 *   - Sizes: element counts (n, m, row_elems, tokens, hidden) above 2^48,
 *     and any buffer the arguments describe above 2^56 bytes, are refused
 *     with VCOLL_ERR_INVALID_ARG, so every byte offset fits in int64.
 *   - Device work is enqueued on `stream` (a hipStream_t; NULL is the null
 *     stream) and the call returns before it completes. The library never
 *     synchronizes and never allocates device memory at run time. Its only
 *     state is two per-device caches filled on first use and kept until the
 *     process ends (the device's compute-unit count, which sizes the
 *     two-phase all-reduce, and the address of the static scratch array of
 *     vcoll_allreduce_stepwise_static), plus that array itself. A failed
 *     launch returns VCOLL_ERR_HIP; faults of running kernels surface at
 *     the caller's next synchronization.
 *   - `send` / `recv` are host arrays of p device pointers, read only during
 *     the call. The caller owns every device buffer.
 *   - Rank buffers are contiguous arrays of the storage type. When every
 *     pointer of a call is 16-byte aligned the kernels move 16-byte vectors;
 *     otherwise they fall back to element-wise access (slower, same result).
 *     Buffers that also share their address mod 128 (or 256) get tiles on
 *     whole cache lines, which the all-reduces need for full speed.
 *   - Arithmetic: float32 adds, round to nearest even, no fused
 *     multiply-add, denormals kept. bfloat16 inputs widen exactly to
 *     float32, all p-1 adds of an element happen in float32, and the result
 *     is rounded to bfloat16 (nearest, ties to even) once.
 *   - Chunks: an n-element vector is cut into p chunks, chunk c covering
 *     [off(c), off(c) + count(c)) with off(c) = c*floor(n/p) + min(c, n mod p)
 *     (the first n mod p chunks hold one extra element).
 */
#ifndef VCOLL_H
#define VCOLL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VCOLL_ABI_VERSION 1
#define VCOLL_MAX_RANKS 128
/* Size of the library's own scratch array (one per GPU) behind
 * vcoll_allreduce_stepwise_static: 64 MiB of float32 partial sums. */
#define VCOLL_STEP_SCRATCH_BYTES (64 * 1024 * 1024)

typedef enum {
  VCOLL_OK = 0,
  VCOLL_ERR_INVALID_ARG = 1,     /* out-of-range p, n, dtype, algo, NULL pointer, bad split */
  VCOLL_ERR_UNSUPPORTED = 2,     /* the (operation, algorithm, p) combination does not exist */
  VCOLL_ERR_BUFFER_TOO_SMALL = 3,/* ledger capacity below the number of messages */
  VCOLL_ERR_HIP = 4,             /* the HIP runtime refused a launch */
  VCOLL_ERR_SCRATCH_LIMIT = 5    /* the call needs more than the library's static scratch array */
} vcoll_status;

typedef enum {
  VCOLL_RING = 0,                /* [NCC] 5.1, [HPC] "Ring Algorithm", [LDT] */
  VCOLL_RECURSIVE_DOUBLING = 1,  /* [NCC] 5.2 */
  VCOLL_RABENSEIFNER = 2,        /* [NCC] 5.2 */
  VCOLL_BINARY_TREE = 3,         /* [NCC] 5.2 (binomial reduce + broadcast) */
  VCOLL_NAIVE = 4,               /* [NCC] 5.5 broadcast: the root sends to one rank per step */
  VCOLL_SCATTER_ALLGATHER = 5,   /* [NCC] 4.2 broadcast: scatter, then ring all-gather */
  VCOLL_PIPELINED_CHAIN = 6      /* [NCC] 5.5 broadcast: k blocks down a chain of ranks */
} vcoll_algo;

typedef enum {
  VCOLL_F32 = 0,
  VCOLL_BF16 = 1,
  VCOLL_U8 = 2                   /* raw bytes: vcoll_all_to_all and its ledger only */
} vcoll_dtype;

typedef enum {
  VCOLL_OP_ALLREDUCE = 0,
  VCOLL_OP_REDUCE_SCATTER = 1,
  VCOLL_OP_ALL_GATHER = 2,
  VCOLL_OP_ALL_TO_ALL = 3,
  VCOLL_OP_BROADCAST = 4,        /* ledger through vcoll_ledger_rooted only */
  VCOLL_OP_REDUCE = 5            /* ledger through vcoll_ledger_rooted only */
} vcoll_op;

/* One message of an algorithm's schedule. Offsets and count are in elements
 * of the storage type; bytes = count * element size. */
typedef struct {
  int32_t step, src, dst, reserved;
  int64_t src_off, dst_off, count, bytes;
} vcoll_msg;

/* Library version of this header's ABI (VCOLL_ABI_VERSION). */
int vcoll_abi_version(void);

/* Static text for a status code (never NULL). */
const char* vcoll_status_str(vcoll_status status);

/* Text of the HIP error behind the most recent VCOLL_ERR_HIP returned to the
 * calling thread ("" if none); static storage, never NULL. */
const char* vcoll_last_hip_error(void);

/* Bounds of chunk c (0 <= c < p) of an n-element vector, as defined above.
 * Host only. */
vcoll_status vcoll_chunk(int p, int64_t n, int c, int64_t* off, int64_t* count);

/*
 * All-reduce: afterwards every recv[r] holds the elementwise sum of the p
 * send[r] vectors of n elements, summed in the order the algorithm's steps
 * produce ([NCC] 4.1 semantics; orders from 5.1 / 5.2):
 *   RING: chunk c is summed along the ring starting after its owner,
 *     (((x[c+1] + x[c+2]) + ...) + x[c-1]) + x[c], ranks mod p; the ring runs
 *     rank i -> i+1 and rank c finishes chunk c. Any p.
 *   RECURSIVE_DOUBLING: partners i, i xor 2^k add full vectors, k = 0, 1, ..:
 *     a balanced tree pairing neighbouring ranks first. If p is not a power
 *     of two, with p2 the largest power of two below p and r = p - p2, rank
 *     pairs (2j, 2j+1), j < r, are added first and stand as one leaf.
 *   RABENSEIFNER: recursive halving at distance p2/2, p2/4, .., 1 then
 *     recursive doubling: a balanced tree pairing ranks p2/2 apart first;
 *     same pre-addition of rank pairs when p is not a power of two.
 *   BINARY_TREE: binomial reduce to rank 0 (masks 1, 2, 4, ..) then binomial
 *     broadcast: for p = 2^k the same tree as recursive doubling; otherwise
 *     the power-of-two-aligned subtrees of 0..p-1 added right to left.
 * Every rank receives bitwise the same vector. recv[r] == send[r] (in place)
 * is allowed; other overlaps are not. 1 <= p <= VCOLL_MAX_RANKS, n >= 0
 * (0 is a no-op).
 */
vcoll_status vcoll_allreduce(vcoll_algo algo, int p, int64_t n, vcoll_dtype dtype,
                             const void* const* send, void* const* recv, void* stream);

/*
 * Stepwise all-reduce: the same result as vcoll_allreduce, bit for bit, but
 * executed the way the algorithm runs on a network ([NCC] code note: a
 * virtual cluster with real data, message by message): one launch per step
 * of the schedule vcoll_ledger lists, each moving that step's messages
 * through memory (receivers add or copy what arrives; recursive-doubling
 * partners exchange). It costs the memory round trips and per-step launch
 * latency that the fused vcoll_allreduce avoids, which is what it measures.
 * float32: works in recv (in place allowed); workspace unused (may be NULL).
 * bfloat16: partial sums stay float32 in `workspace`, at least p*n*4 bytes
 * (VCOLL_ERR_BUFFER_TOO_SMALL otherwise), rounded once as in vcoll_allreduce.
 * *n_launches (may be NULL) receives the number of kernel launches enqueued.
 */
vcoll_status vcoll_allreduce_stepwise(vcoll_algo algo, int p, int64_t n, vcoll_dtype dtype,
                                      const void* const* send, void* const* recv, void* workspace,
                                      int64_t workspace_bytes, int32_t* n_launches, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation as vcoll_allreduce_stepwise, bit for bit and launch for launch,
 * with the bfloat16 float32 partial sums in a scratch array the library
 * owns instead of a caller workspace. The array is a file-scope device
 * variable of VCOLL_STEP_SCRATCH_BYTES: every GPU the library runs on holds
 * its own copy until the process ends, and the call uses the copy of the
 * current device (the stream must belong to it). The call allocates no
 * device memory. Its first use on a device looks the array's address up once
 * (a HIP symbol query, before anything is enqueued; a failure returns
 * VCOLL_ERR_HIP).
 * bfloat16 needs p*n*4 <= VCOLL_STEP_SCRATCH_BYTES, else
 * VCOLL_ERR_SCRATCH_LIMIT (nothing enqueued); float32 works in recv and uses
 * no scratch, at any size. Nothing in the array has to start at zero: every
 * call first writes the partial sums it later reads. All calls on one GPU
 * share the array, so calls that overlap on one GPU (different streams
 * without ordering between them) race and give undefined results; calls
 * ordered on one stream are safe.
 */
vcoll_status vcoll_allreduce_stepwise_static(vcoll_algo algo, int p, int64_t n, vcoll_dtype dtype,
                                             const void* const* send, void* const* recv,
                                             int32_t* n_launches, void* stream);

/*
 * Broadcast ([NCC] 4.1): every rank's buffer receives the root's n elements,
 * bit for bit. All broadcast algorithms ([NCC] 4.2 scatter + all-gather,
 * 5.5 naive, binomial tree, pipelined chain) leave the same bytes; they
 * differ only in their messages (vcoll_ledger_rooted), so one pass reads
 * `send` (the root's buffer) once and writes every recv[r]. recv holds p
 * device pointers; recv[root] may be NULL or equal to send (then nothing is
 * written there). Receive buffers must not overlap send or each other.
 * 0 <= root < p.
 */
vcoll_status vcoll_broadcast(int p, int64_t n, vcoll_dtype dtype, int root, const void* send, void* const* recv,
                             void* stream);

/*
 * Stepwise broadcast: the same bytes as vcoll_broadcast, but executed the way
 * the algorithm runs on a network, one launch per step of the schedule
 * vcoll_ledger_rooted lists for (algo, root, blocks), each copying that
 * step's messages between the rank buffers -- [NCC] 5.5 naive (p-1 steps),
 * binomial tree (ceil(log2 p)), 4.2 scatter + all-gather (1 + (p-1)),
 * pipelined chain of `blocks` blocks (p-2+blocks; 1 <= blocks <= 65536).
 * It measures what the one-pass broadcast hides: per-step launch latency and
 * the bytes each step moves. The root's messages are read from `send`;
 * recv[root], when it is neither NULL nor `send`, first gets a local copy
 * (one extra launch) and receives whatever the schedule sends to the root;
 * `send` is never written. Steps whose messages are all empty launch
 * nothing. *n_launches (may be NULL) receives the launches enqueued.
 */
vcoll_status vcoll_broadcast_stepwise(vcoll_algo algo, int p, int64_t n, vcoll_dtype dtype, int root, int64_t blocks,
                                      const void* send, void* const* recv, int32_t* n_launches, void* stream);

/*
 * Reduce to a root ([NCC] 4.1: elementwise sum, result on the root only) by
 * the binomial tree of [NCC] 5.2 on ranks relative to the root,
 * v = (r - root) mod p: masks 1, 2, 4, ..; the relative rank whose lowest
 * set bit is the mask adds its partial sum into v - mask. `recv` is the
 * root's output buffer (n elements; may equal send[root]); no other buffer
 * is written. algo must be VCOLL_BINARY_TREE (others: VCOLL_ERR_UNSUPPORTED).
 */
vcoll_status vcoll_reduce(vcoll_algo algo, int p, int64_t n, vcoll_dtype dtype, int root,
                          const void* const* send, void* recv, void* stream);

/*
 * Message ledger of a rooted collective, conventions as vcoll_ledger. op
 * VCOLL_OP_BROADCAST with algo VCOLL_NAIVE (p-1 steps, the root sends the
 * whole vector to relative rank s+1 in step s), VCOLL_BINARY_TREE
 * (ceil(log2 p) steps, masks descending: relative rank v, a multiple of 2m,
 * sends to v+m), VCOLL_SCATTER_ALLGATHER (step 0: the root sends chunk v to
 * every relative rank v != 0; then ring all-gather step s, in ledger step
 * 1+s, has v forward chunk (v-s) mod p to v+1) or
 * VCOLL_PIPELINED_CHAIN (`blocks` >= 1 balanced blocks; in step t relative
 * rank v passes block t-v to v+1; p-2+blocks steps); op VCOLL_OP_REDUCE with
 * VCOLL_BINARY_TREE. `blocks` is read only by the chain. Host only.
 */
vcoll_status vcoll_ledger_rooted(vcoll_op op, vcoll_algo algo, int p, int64_t n, vcoll_dtype dtype, int root,
                                 int64_t blocks, vcoll_msg* msgs, int64_t cap, int64_t* n_msgs,
                                 int64_t* sent_bytes, int64_t* recv_bytes, int32_t* n_steps);

/*
 * Token-major form of a vcoll_moe_plan ([NCC] 7.4), for vcoll_moe_dispatch.
 * Host only. From splits [p*p] and dst_rows [p][tokens*topk] of
 * vcoll_moe_plan it fills slots [p][tokens*topk][2] int32: for rank i's
 * pair (t, k), the destination rank j and the row of recv[j] that the
 * plain dispatch (vcoll_all_to_all with src_rows) writes it to. splits
 * within the limits of vcoll_all_to_all, at most tokens*topk rows sent per
 * rank and every dst_rows entry in [0, tokens*topk), else
 * VCOLL_ERR_INVALID_ARG (slots may then be partly written).
 */
vcoll_status vcoll_moe_slots(int p, int64_t tokens, int topk, const int64_t* splits, const int32_t* dst_rows,
                             int32_t* slots);

/*
 * MoE dispatch, token-major ([NCC] 7.4): every token row of every rank is
 * read once and written to each of its topk slots (slots[i] on the device,
 * as filled by vcoll_moe_slots), so the token tables are read once instead
 * of once per (token, expert) pair. fp8 = 0 copies rows of `hidden`
 * elements of dtype (F32 or BF16); the receive buffers then equal those of
 * the plain dispatch bit for bit. fp8 != 0 (dtype BF16, hidden a multiple
 * of 128) stores each row as the FP8 payload of vcoll_moe_dispatch_fp8,
 * quantised once per token. recv_rows[j] bounds recv[j]; a slot outside
 * [0, p) x [0, recv_rows[j]) is skipped. Token tables 16-byte aligned for
 * FP8; receive buffers 4-byte aligned for FP8.
 */
vcoll_status vcoll_moe_dispatch(int p, int64_t tokens, int topk, int64_t hidden, vcoll_dtype dtype, int fp8,
                                const void* const* token_tables, const int32_t* const* slots,
                                void* const* recv, const int64_t* recv_rows, void* stream);

/*
 * Token-major form of a deduplicated dispatch plan ([NCC] 7.4 and exercise
 * 10), for vcoll_moe_dispatch. Host only. From splits_unique [p*p] and
 * src_unique [p][tokens*topk] of vcoll_moe_plan_dedup it fills slots
 * [p][tokens*topk][2] int32: for rank i's token t, the destination ranks it
 * is sent to, ascending, each with the row of that rank's deduplicated
 * receive buffer it lands in, then (-1, -1). vcoll_moe_dispatch with these
 * slots (recv_rows[j] = sum_i splits_unique[i][j]) reads each token once
 * and writes the receive buffers of the deduplicated all-to-all
 * (vcoll_all_to_all(splits_unique, src_rows = src_unique)) bit for bit, or,
 * with fp8, those of vcoll_moe_dispatch_fp8 over the same plan. A token id
 * outside [0, tokens), or more than topk copies of one token, is
 * VCOLL_ERR_INVALID_ARG.
 */
vcoll_status vcoll_moe_dedup_slots(int p, int64_t tokens, int topk, const int64_t* splits_unique,
                                   const int32_t* src_unique, int32_t* slots);

/*
 * Token-major form of one rank's deduplicated-dispatch expansion ([NCC] 7.4
 * and exercise 10: a token arrives once per rank and is then copied to
 * every (token, expert) row of that rank that needs it), for
 * vcoll_moe_dispatch with p = 1. Host only. expand (expand_count entries)
 * is rank j's expansion map from vcoll_moe_plan_dedup (plain row x copies
 * unique row expand[x]); unique_rows is the number of rows rank j received
 * in the deduplicated all-to-all. Fills slots [unique_rows*topk][2] int32:
 * for unique row u, the plain rows copying it as (0, x) pairs in ascending
 * x, then (-1, -1). vcoll_moe_dispatch(1, unique_rows, topk, ...) with the
 * received unique rows as the token table and recv_rows = expand_count then
 * writes the plain layout, reading each unique row once; the result equals
 * the gathering expansion (vcoll_all_to_all with src_rows = expand) bit for
 * bit. An expand entry outside [0, unique_rows), or a unique row copied
 * more than topk times, is VCOLL_ERR_INVALID_ARG.
 */
vcoll_status vcoll_moe_expand_slots(int64_t unique_rows, int topk, const int32_t* expand, int64_t expand_count,
                                    int32_t* slots);

/*
 * Token-major MoE combine ([NCC] 7.4: combine is the all-to-all that returns
 * every expert output to the rank and position of its token; 4.2: applied
 * after the dispatch it restores the original layout). For every rank i,
 * token t < tokens and slot k < topk:
 *   out[i][t*topk + k] = expert_out[j][r],  (j, r) = slots[i][t*topk + k],
 * rows of hidden elements of dtype. slots are the dispatch's, from
 * vcoll_moe_slots ([tokens*topk][2] int32 per rank), and expert_out[j] holds
 * rank j's expert outputs in its dispatch receive order (expert_rows[j]
 * rows). The result equals the reverse vcoll_all_to_all (splits transposed)
 * scattered by dst_rows, bit for bit; here each output row pulls its source
 * row, so each rank's output is written in order. A slot outside
 * [0, p) x [0, expert_rows[j]) leaves its output row untouched. out[i]
 * holds tokens*topk rows; buffers must not overlap. Rows move as 16-byte
 * vectors when every buffer is 16-byte aligned and a row is a multiple of
 * 16 bytes, else as 2-byte words.
 */
vcoll_status vcoll_moe_combine(int p, int64_t tokens, int topk, int64_t hidden, vcoll_dtype dtype,
                               const void* const* expert_out, const int64_t* expert_rows,
                               const int32_t* const* slots, void* const* out, void* stream);

/*
 * Deduplicated MoE dispatch plan ([NCC] 7.4 and exercise 10: a token goes
 * once to each place that needs it and is then copied locally). Host only,
 * integers only; topk_ids and expert placement as vcoll_moe_plan. Rank i
 * sends each token once to every rank j holding at least one of its chosen
 * experts, rows ordered by (j, token): splits_unique [p*p] int64 rows i -> j,
 * src_unique [p][tokens*topk] int32 the token of each sent row (the first
 * sum_j splits_unique[i][j] entries are used). Rank j's deduplicated
 * receive buffer holds the blocks of ranks 0..p-1 in order; expand
 * [p][p*tokens*topk] int32 gives, for each row of the plain dispatch layout
 * of vcoll_moe_plan at rank j (expand_count[j] = sum_i splits[i][j] rows),
 * the deduplicated row it copies. Dispatch is vcoll_all_to_all(
 * splits_unique, src_rows = src_unique) followed by the local expansion
 * vcoll_all_to_all with diagonal splits expand_count and src_rows = expand;
 * the result equals the plain dispatch bit for bit.
 */
vcoll_status vcoll_moe_plan_dedup(int p, int64_t tokens, int topk, int experts_per_rank, const int32_t* topk_ids,
                                  int64_t* splits_unique, int32_t* src_unique, int32_t* expand,
                                  int64_t* expand_count);

/*
 * MoE dispatch with an FP8 payload ([NCC] 7.4: DeepSeek-V3 dispatches in
 * FP8, combines in BF16). Rank i's k-th sent row is token src_rows[i][k] of
 * its bfloat16 table tokens[i] ([token_rows[i]][hidden]); it is quantised
 * at the sender and lands, in the all-to-all layout of vcoll_all_to_all, in
 * recv[j] as a row of hidden + hidden/32 bytes: hidden E4M3 codes (OCP FP8
 * E4M3, no infinities, largest 448, round to nearest even), then one
 * float32 scale per group of 128 elements. A group's scale is 2^k, k the
 * smallest integer with amax <= 448 * 2^k (amax the largest finite |x| of
 * the group; k clamped to [-126, 126]; k = 0 for an all-zero group), and
 * element x is stored as E4M3(x * 2^-k); non-finite elements store 0x7F.
 * hidden must be a positive multiple of 128; token tables 16-byte aligned
 * and receive buffers 4-byte aligned; an index outside [0, token_rows[i])
 * skips its row.
 */
vcoll_status vcoll_moe_dispatch_fp8(int p, int64_t hidden, const int64_t* splits, const void* const* tokens,
                                    const int64_t* token_rows, const int32_t* const* src_rows,
                                    void* const* recv, void* stream);

/*
 * Hierarchical all-reduce ([NCC] 6.3; [LDT] 16 ranks as 2 nodes x 8): p =
 * nodes*local ranks, rank = g*local + l. (1) Inside every group of `local`
 * ranks a ring reduce-scatter over `local` chunks; (2) for every index l, the
 * `nodes` ranks g*local + l run a ring all-reduce of chunk l, cut into
 * `nodes` pieces; (3) inside every group a ring all-gather. The 2D torus
 * all-reduce of an a x b grid ([NCC] 6.1: rows, then columns, then back) is
 * the same with nodes = a and local = b. In piece j of chunk l the sum is an
 * outer chain over the groups starting after group j, of inner chains over
 * each group's ranks starting after rank l. Chunks and pieces are balanced
 * as above. Every rank receives the same vector; in place allowed.
 * 1 <= nodes*local <= VCOLL_MAX_RANKS.
 */
vcoll_status vcoll_allreduce_hierarchical(int nodes, int local, int64_t n, vcoll_dtype dtype,
                                          const void* const* send, void* const* recv, void* stream);

/* Message ledger of vcoll_allreduce_hierarchical, conventions as vcoll_ledger:
 * steps 0..local-2 in-group reduce-scatter, then nodes-1 cross-group
 * reduce-scatter and nodes-1 cross-group all-gather steps, then local-1
 * in-group all-gather steps. Host only. */
vcoll_status vcoll_ledger_hierarchical(int nodes, int local, int64_t n, vcoll_dtype dtype, vcoll_msg* msgs,
                                       int64_t cap, int64_t* n_msgs, int64_t* sent_bytes,
                                       int64_t* recv_bytes, int32_t* n_steps);

/*
 * Reduce-scatter ([HPC] "Collective Communication Primitives": process k gets
 * the k-th piece of the sum; [NCC] 4.1): recv[c] (count(c) elements) receives
 * chunk c of the sum, in the same order as the all-reduce of the same
 * algorithm. RING for any p; RABENSEIFNER (recursive halving) for p a power
 * of two. Other algorithms: VCOLL_ERR_UNSUPPORTED. Buffers must not overlap.
 */
vcoll_status vcoll_reduce_scatter(vcoll_algo algo, int p, int64_t n, vcoll_dtype dtype,
                                  const void* const* send, void* const* recv, void* stream);

/*
 * All-gather ([HPC] primitives; [NCC] 4.1): every recv[r] (p*m elements)
 * receives send[0] .. send[p-1] (m elements each) concatenated in rank
 * order, as raw storage words. RING for any p; RECURSIVE_DOUBLING for p a
 * power of two (the result is the same, only the ledger differs). Buffers
 * must not overlap.
 */
vcoll_status vcoll_all_gather(vcoll_algo algo, int p, int64_t m, vcoll_dtype dtype,
                              const void* const* send, void* const* recv, void* stream);

/*
 * Variable-split all-to-all ([NCC] 4.1: block j of device i goes to device j,
 * the transpose of the device-by-block matrix; 7.4: MoE dispatch/combine).
 * Rows have row_elems elements. `splits` is a host array [p*p]; splits[i*p+j]
 * >= 0 rows go from rank i to rank j; the rows each rank sends, and those it
 * receives, total at most INT32_MAX (else VCOLL_ERR_INVALID_ARG). send[i]
 * holds its blocks j = 0..p-1 in order; recv[j] receives the blocks
 * i = 0..p-1 in order. Rows are moved as raw storage words.
 *   src_rows (optional, host array of p device int32 pointers, entries may be
 *   NULL): when src_rows[i] is set, the k-th row rank i sends (block order)
 *   is row src_rows[i][k] of send[i], a table of src_table_rows[i] rows --
 *   a fused gather (MoE dispatch from the token buffer).
 *   dst_rows (optional, likewise): when dst_rows[j] is set, the k-th row rank
 *   j receives (block order) is written to row dst_rows[j][k] of recv[j], a
 *   table of dst_table_rows[j] rows -- a fused scatter (MoE combine).
 *   A gather or scatter index outside its table is skipped by the kernel
 *   (that row is neither read nor written).
 * Buffers must not overlap.
 */
vcoll_status vcoll_all_to_all(int p, int64_t row_elems, vcoll_dtype dtype, const int64_t* splits,
                              const void* const* send, void* const* recv,
                              const int32_t* const* src_rows, const int64_t* src_table_rows,
                              const int32_t* const* dst_rows, const int64_t* dst_table_rows,
                              void* stream);

/*
 * Message ledger ([NCC] code note: a virtual cluster accounts every message;
 * 4.3 per-device bytes). Host only, no device work. Enumerates the messages
 * of `op` run with `algo` on p ranks of n elements (all-gather: m elements
 * per rank; all-to-all: `splits` and `row_elems` within the limits of
 * vcoll_all_to_all, algo ignored, direct
 * schedule where step s-1 sends block i -> (i+s) mod p, s = 1..p-1, the
 * diagonal block being local). Each step is synchronous; recursive doubling
 * and Rabenseifner with p not a power of two add a pre-step (2j -> 2j+1) and
 * a post-step (2j+1 -> 2j), j < r. Records are sorted by (step, src, dst,
 * src_off). Two-call use: with msgs == NULL only *n_msgs is set; with
 * cap < *n_msgs the call returns VCOLL_ERR_BUFFER_TOO_SMALL and sets *n_msgs.
 * sent_bytes / recv_bytes (p entries) and n_steps may be NULL.
 */
vcoll_status vcoll_ledger(vcoll_op op, vcoll_algo algo, int p, int64_t n, vcoll_dtype dtype,
                          const int64_t* splits, int64_t row_elems,
                          vcoll_msg* msgs, int64_t cap, int64_t* n_msgs,
                          int64_t* sent_bytes, int64_t* recv_bytes, int32_t* n_steps);

/*
 * MoE dispatch plan ([NCC] 7.4: every (token, chosen expert) pair is one row
 * sent to the rank holding that expert). Host only, integers only.
 * topk_ids: host int32 [p][tokens][topk], expert ids in
 * [0, p*experts_per_rank); expert e lives on rank e / experts_per_rank.
 * Rank i sends its rows ordered by (destination rank, expert, token).
 * Outputs (host): splits [p*p] int64 rows i -> j; src_rows [p][tokens*topk]
 * int32, the token each sent row copies; dst_rows [p][tokens*topk] int32,
 * the (token, slot) position token*topk + slot each returning row lands on
 * at combine. Dispatch is vcoll_all_to_all(splits, src_rows = src_rows);
 * combine is vcoll_all_to_all(splits transposed, dst_rows = dst_rows).
 */
vcoll_status vcoll_moe_plan(int p, int64_t tokens, int topk, int experts_per_rank,
                            const int32_t* topk_ids, int64_t* splits,
                            int32_t* src_rows, int32_t* dst_rows);

/*
 * Alpha-beta cost model ([NCC] 2.1: a message of b bytes costs alpha + b/beta,
 * alpha in seconds, beta in bytes per second). Host only.
 *
 * vcoll_model_formula: closed-form all-reduce time for `bytes` per rank
 * ([NCC] 5.1 and exercise 2: ring 2(p-1)(alpha + bytes/(p beta)); 5.2:
 * recursive doubling log2 p (alpha + bytes/beta), Rabenseifner
 * 2 log2 p alpha + 2(p-1)/p bytes/beta, binary tree
 * 2 ceil(log2 p)(alpha + bytes/beta)). For p not a power of two, recursive
 * doubling and Rabenseifner run on p2 = 2^floor(log2 p) ranks plus two
 * full-vector fold steps. 1 <= p <= 2^20 (host arithmetic only).
 *
 * vcoll_model_ledger_time: a simulated clock over vcoll_ledger's messages of
 * the same arguments: each step costs alpha plus the largest byte count any
 * rank sends or receives in that step, divided by beta (full-duplex ports).
 * For p dividing n it equals the closed form.
 * Errors: VCOLL_ERR_INVALID_ARG for alpha < 0, beta <= 0, NULL outputs, or
 * what vcoll_ledger rejects.
 */
vcoll_status vcoll_model_formula(vcoll_algo algo, int p, double bytes, double alpha, double beta,
                                 double* seconds);
vcoll_status vcoll_model_ledger_time(vcoll_op op, vcoll_algo algo, int p, int64_t n, vcoll_dtype dtype,
                                     const int64_t* splits, int64_t row_elems, double alpha, double beta,
                                     double* seconds, int32_t* n_steps);

/*
 * Alpha-beta clock on a two-level network ([NCC] 2.3 scale-up / scale-out;
 * 6.3 and exercise 6): ranks r and s share a node when r/local == s/local;
 * a message inside a node costs (alpha_in, beta_in), across nodes
 * (alpha_out, beta_out). Each step lasts as long as its slowest port: the
 * largest of alpha + bytes/beta over every rank's sending and receiving
 * port of each class that carries bytes in the step. hierarchical != 0
 * clocks vcoll_ledger_hierarchical(nodes, local, ...) (algo ignored);
 * otherwise vcoll_ledger's all-reduce with `algo` on nodes*local ranks.
 */
vcoll_status vcoll_model_ledger_time_nodes(int hierarchical, vcoll_algo algo, int nodes, int local, int64_t n,
                                           vcoll_dtype dtype, double alpha_in, double beta_in,
                                           double alpha_out, double beta_out, double* seconds,
                                           int32_t* n_steps);

/*
 * Closed-form broadcast times of nbytes ([NCC] 4.2, 5.5): NAIVE
 * (p-1)(alpha + n/beta); BINARY_TREE ceil(log2 p)(alpha + n/beta);
 * PIPELINED_CHAIN (p-2+blocks)(alpha + n/(blocks beta)); SCATTER_ALLGATHER
 * (alpha + (p-1)/p n/beta) + (p-1)(alpha + n/(p beta)). p = 1 gives 0.
 */
vcoll_status vcoll_model_broadcast_formula(vcoll_algo algo, int p, double nbytes, int64_t blocks, double alpha,
                                           double beta, double* seconds);

/* The chain's optimum ([NCC] 5.5, exercise 9): blocks* = sqrt((p-2) n /
 * (alpha beta)) (real, before rounding) and T* = (sqrt((p-2) alpha) +
 * sqrt(n/beta))^2. Needs p >= 3. */
vcoll_status vcoll_model_chain_optimum(int p, double nbytes, double alpha, double beta, double* blocks,
                                       double* seconds);

/* The simulated clock of vcoll_model_ledger_time_nodes over any ledger the
 * caller holds (n_msgs records on p ranks; local = p gives the one-class
 * clock of vcoll_model_ledger_time). Host only. */
vcoll_status vcoll_model_clock(const vcoll_msg* msgs, int64_t n_msgs, int p, int local, double alpha_in,
                               double beta_in, double alpha_out, double beta_out, double* seconds);

#ifdef __cplusplus
}
#endif

#endif /* VCOLL_H */
