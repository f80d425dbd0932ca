// C ABI of libvcoll: argument validation, launch descriptors, dispatch.
// Every check happens before the first launch, so an error return means that
// nothing was enqueued.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "bench.h"
#include "hier.h"
#include "move.h"
#include "reduce.h"
#include "step.h"
#include "schedule.h"
#include "vcoll.h"
#include "vcoll_bench.h"

using namespace vcoll;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

thread_local const char* g_last_hip_error = "";

vcoll_status from_hip(hipError_t e) {
  if (e == hipSuccess) return VCOLL_OK;
  g_last_hip_error = hipGetErrorString(e);
  return VCOLL_ERR_HIP;
}

int64_t elem_bytes(vcoll_dtype d) { return d == VCOLL_F32 ? 4 : (d == VCOLL_BF16 ? 2 : 1); }

bool valid_dtype(int d) { return d == VCOLL_F32 || d == VCOLL_BF16; }

// the all-to-all only moves rows, so it also takes raw bytes
bool valid_a2a_dtype(int d) { return valid_dtype(d) || d == VCOLL_U8; }

bool valid_algo(int a) { return a >= VCOLL_RING && a <= VCOLL_BINARY_TREE; }

bool valid_p(int p) { return p >= 1 && p <= kMaxRanks; }

// nodes x local ranks: each factor is bounded before the product is formed,
// so the product cannot overflow int
bool valid_grid(int nodes, int local) {
  return nodes >= 1 && local >= 1 && nodes <= kMaxRanks && local <= kMaxRanks && valid_p(nodes * local);
}

// rows x topk within int32 (the row indices of the MoE maps), tested by
// division so that the product is only formed once it is known to fit
bool pairs_fit(int64_t rows, int topk) { return topk >= 1 && rows >= 0 && rows <= INT32_MAX / topk; }

// Element counts up to 2^48: far beyond any buffer, and small enough that
// every byte offset (count x 4 bytes x up to 128 ranks) fits in int64.
constexpr int64_t kMaxCount = int64_t(1) << 48;

bool valid_count(int64_t n) { return n >= 0 && n <= kMaxCount; }

// A buffer of `rows` rows of `row_bytes` bytes stays within 2^56 bytes.
bool fits(int64_t rows, int64_t row_bytes) {
  return row_bytes <= 0 || rows <= (int64_t(1) << 56) / row_bytes;
}

// Row counts of an all-to-all: every entry >= 0 and each rank's sent and
// received totals within INT32_MAX rows (row indices are int32) and within
// the byte bound of fits(); the per-rank totals go to `sent` and `got`.
bool valid_splits(int p, const int64_t* splits, int64_t row_bytes, std::vector<int64_t>& sent,
                  std::vector<int64_t>& got) {
  sent.assign(p, 0);
  got.assign(p, 0);
  for (int i = 0; i < p; ++i)
    for (int j = 0; j < p; ++j) {
      const int64_t s = splits[i * p + j];
      if (s < 0 || s > INT32_MAX) return false;
      sent[i] += s;
      got[j] += s;
      if (sent[i] > INT32_MAX || got[j] > INT32_MAX) return false;
    }
  for (int i = 0; i < p; ++i)
    if (!fits(sent[i], row_bytes) || !fits(got[i], row_bytes)) return false;
  return true;
}

bool all_set(int p, const void* const* ptrs) {
  if (!ptrs) return false;
  for (int r = 0; r < p; ++r)
    if (!ptrs[r]) return false;
  return true;
}

bool all_aligned(int p, const void* const* ptrs) {
  for (int r = 0; r < p; ++r)
    if (!aligned16(ptrs[r])) return false;
  return true;
}

// The address of every send (and, when given, receive) buffer mod `m` (a
// power of two), or -1 when they differ.
int32_t common_phase(int p, const void* const* send, void* const* recv, uintptr_t m) {
  const uintptr_t ph = reinterpret_cast<uintptr_t>(send[0]) & (m - 1);
  for (int r = 0; r < p; ++r)
    if ((reinterpret_cast<uintptr_t>(send[r]) & (m - 1)) != ph ||
        (recv && (reinterpret_cast<uintptr_t>(recv[r]) & (m - 1)) != ph))
      return -1;
  return static_cast<int32_t>(ph);
}

// Compute units of the current device, read once per device (0 when no
// device can be queried, which turns the burst kernel off).
int device_cus() {
  static std::mutex mu;
  static int cus[64] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus[dev] = v;
  }
  return cus[dev];
}

// Smallest tile (16-byte vectors) for which the two-phase ring kernel beats
// the one-pass kernel: 16 vectors per thread (16 MiB of float32 per rank at
// p = 8) gained 9 %, 4 vectors (4 MiB) lost 2.3x, on MI355X.
constexpr int64_t kBurstMinTile = 3072;

// Tiles per chunk for the two-phase ring all-reduce, or 0 when the one-pass
// kernel is the better choice: the whole vector must fit in one generation
// of workgroups (one per compute unit) at between kBurstMinTile and
// burst_tile_max vectors each. A chunk's tiles cover the 16-byte vectors
// wholly inside it (the kernel sums the few elements around its ends one by
// one), so the largest such count over the chunks sets the tile.
int burst_tiles(int p, const Chunks& ch, vcoll_dtype dtype, int32_t align, int32_t phase, int64_t* tv) {
  const int ve = 16 / static_cast<int>(elem_bytes(dtype));
  const int per_chunk = device_cus() / p;
  if (per_chunk < 1) return 0;
  int64_t cv = 0;
  for (int c = 0; c < p; ++c) {
    const int64_t e0 = ch.off(c), e1 = e0 + ch.count(c);
    const int64_t whole = e1 / ve - burst_first_vector(e0, ve, align, phase);
    if (whole > cv) cv = whole;
  }
  const int64_t t = ((cv + per_chunk - 1) / per_chunk + 7) / 8 * 8;   // whole 128-byte cache lines
  if (t < kBurstMinTile || t > burst_tile_max(dtype)) return 0;
  *tv = t;
  return static_cast<int>((cv + t - 1) / t);
}

// Leaf buffers of a tree program for the kernels with a run-time p: group q
// of the program (order_groups) in leaf[q] and, for a folded pair, its
// second leaf in leaf[kMaxRanks + q]; `input(k)` is the buffer of program
// leaf k.
template <class Input>
void set_tree_groups(ReduceArgs& a, vcoll_algo algo, int p, const Input& input) {
  int first[kMaxRanks + 1] = {};
  a.groups = order_groups(algo, p, first);
  for (int q = 0; q < a.groups; ++q) {
    a.leaf[q] = input(first[q]);
    a.leaf[kMaxRanks + q] = first[q + 1] - first[q] == 2 ? input(first[q] + 1) : nullptr;
  }
}

vcoll_status reduce_common(vcoll_algo algo, int p, int64_t n, vcoll_dtype dtype,
                           const void* const* send, void* const* recv, void* stream, bool scatter) {
  if (!valid_p(p) || !valid_count(n) || !valid_dtype(dtype) || !valid_algo(algo)) return VCOLL_ERR_INVALID_ARG;
  const vcoll_status combo =
      check_combination(scatter ? VCOLL_OP_REDUCE_SCATTER : VCOLL_OP_ALLREDUCE, algo, p);
  if (combo != VCOLL_OK) return combo;
  if (n == 0) return VCOLL_OK;
  if (!all_set(p, send) || !all_set(p, const_cast<const void* const*>(recv))) return VCOLL_ERR_INVALID_ARG;

  ReduceArgs a;
  std::memset(&a, 0, sizeof(a));
  for (int r = 0; r < p; ++r) a.dst[r] = recv[r];
  const Chunks ch(n, p);
  a.q = ch.q;
  a.r = ch.r;
  a.p = p;
  a.vec = all_aligned(p, send) && all_aligned(p, const_cast<const void* const*>(recv));
  // a common address phase mod 256 (else mod 128) lets the tiles start on
  // whole cache lines of every buffer; rows that share only the phase mod
  // 128 (a [p, n] tensor with n = 32 mod 64, float32) ran the one-pass
  // all-reduces 9-20 % faster on MI355X with 128-byte than with 16-byte
  // tiles (p = 16 x 16 MiB trees 144 -> 117 us, p = 8 x 64 MiB 204 -> 181)
  const int32_t ph256 = common_phase(p, send, recv, 256), ph128 = common_phase(p, send, recv, 128);
  a.align = ph256 >= 0 ? 256 : (ph128 >= 0 ? 128 : 16);
  a.phase = ph256 >= 0 ? ph256 : (ph128 >= 0 ? ph128 : 0);
  const int32_t src128 = common_phase(p, send, nullptr, 128);
  a.src_align = src128 >= 0 ? 128 : 16;
  a.src_phase = src128 >= 0 ? src128 : 0;
  const int32_t burst_align = ph128 >= 0 ? 128 : 16, burst_phase = ph128 >= 0 ? ph128 : 0;
  int64_t tv = 0;
  const int tiles = (!scatter && algo == VCOLL_RING && a.vec)
                        ? burst_tiles(p, ch, dtype, burst_align, burst_phase, &tv) : 0;
  if (tiles > 0) {
    BurstArgs b;
    std::memset(&b, 0, sizeof(b));
    for (int r = 0; r < p; ++r) {
      b.src[r] = send[r];
      b.dst[r] = recv[r];
    }
    b.q = ch.q;
    b.r = static_cast<int32_t>(ch.r);
    b.p = p;
    b.tv = static_cast<int32_t>(tv);
    b.align = burst_align;
    b.phase = burst_phase;
    return from_hip(launch_burst_ring(b, dtype, tiles, static_cast<hipStream_t>(stream)));
  }
  const OrderProgram prog = order_program(algo, p);
  if (has_fixed_kernel(p)) {
    // leaf pointers in summation order: ring rotated per chunk (chunk c's
    // chain starts at rank c+1), trees the same for every chunk
    const int rows = algo == VCOLL_RING ? p : 1;
    for (int c = 0; c < rows; ++c)
      for (int k = 0; k < p; ++k)
        a.leaf[c * kFixedMax + k] = send[algo == VCOLL_RING ? (c + 1 + k) % p : prog.rank[k]];
  } else if (algo == VCOLL_RING) {
    for (int k = 0; k < p; ++k) a.leaf[k] = send[k];
  } else {
    set_tree_groups(a, algo, p, [&](int k) { return send[prog.rank[k]]; });
  }
  return from_hip(launch_reduce(a, dtype, algo, scatter, ch.count(0), p, static_cast<hipStream_t>(stream)));
}

// Workgroup tiles of each launch of at most kA2ABlocks blocks; false when a
// launch would need more than INT32_MAX of them (checked before any launch,
// so that an error return still means nothing was enqueued).
bool block_launch_tiles(const std::vector<A2ABlock>& blocks, int32_t rows_per_tile) {
  for (size_t b0 = 0; b0 < blocks.size(); b0 += kA2ABlocks) {
    int64_t tiles = 0;
    for (size_t k = b0; k < std::min<size_t>(blocks.size(), b0 + kA2ABlocks); ++k)
      tiles += (blocks[k].rows + rows_per_tile - 1) / rows_per_tile;
    if (tiles > INT32_MAX) return false;
  }
  return true;
}

// Two-call ledger convention shared by every ledger entry point.
vcoll_status emit_ledger(const std::vector<vcoll_msg>& out, int32_t steps, int p, vcoll_msg* msgs, int64_t cap,
                         int64_t* n_msgs, int64_t* sent_bytes, int64_t* recv_bytes, int32_t* n_steps) {
  *n_msgs = static_cast<int64_t>(out.size());
  if (msgs) {
    if (cap < static_cast<int64_t>(out.size())) return VCOLL_ERR_BUFFER_TOO_SMALL;
    std::copy(out.begin(), out.end(), msgs);
  }
  if (sent_bytes) std::fill(sent_bytes, sent_bytes + p, 0);
  if (recv_bytes) std::fill(recv_bytes, recv_bytes + p, 0);
  for (const vcoll_msg& m : out) {
    if (sent_bytes) sent_bytes[m.src] += m.bytes;
    if (recv_bytes) recv_bytes[m.dst] += m.bytes;
  }
  if (n_steps) *n_steps = steps;
  return VCOLL_OK;
}

}  // namespace

extern "C" {

int vcoll_abi_version(void) { return VCOLL_ABI_VERSION; }

const char* vcoll_last_hip_error(void) { return g_last_hip_error; }

const char* vcoll_status_str(vcoll_status status) {
  switch (status) {
    case VCOLL_OK: return "ok";
    case VCOLL_ERR_INVALID_ARG: return "invalid argument";
    case VCOLL_ERR_UNSUPPORTED: return "unsupported operation/algorithm/p combination";
    case VCOLL_ERR_BUFFER_TOO_SMALL: return "ledger buffer too small";
    case VCOLL_ERR_HIP: return "HIP launch failed";
    case VCOLL_ERR_SCRATCH_LIMIT: return "size exceeds the library's static scratch array (VCOLL_STEP_SCRATCH_BYTES)";
  }
  return "unknown status";
}

vcoll_status vcoll_chunk(int p, int64_t n, int c, int64_t* off, int64_t* count) {
  if (!valid_p(p) || !valid_count(n) || c < 0 || c >= p || !off || !count) return VCOLL_ERR_INVALID_ARG;
  const Chunks ch(n, p);
  *off = ch.off(c);
  *count = ch.count(c);
  return VCOLL_OK;
}

vcoll_status vcoll_allreduce(vcoll_algo algo, int p, int64_t n, vcoll_dtype dtype,
                             const void* const* send, void* const* recv, void* stream) {
  return reduce_common(algo, p, n, dtype, send, recv, stream, false);
}

vcoll_status vcoll_reduce_scatter(vcoll_algo algo, int p, int64_t n, vcoll_dtype dtype,
                                  const void* const* send, void* const* recv, void* stream) {
  return reduce_common(algo, p, n, dtype, send, recv, stream, true);
}

vcoll_status vcoll_all_gather(vcoll_algo algo, int p, int64_t m, vcoll_dtype dtype,
                              const void* const* send, void* const* recv, void* stream) {
  if (!valid_p(p) || !valid_count(m) || !valid_dtype(dtype) || !valid_algo(algo)) return VCOLL_ERR_INVALID_ARG;
  const vcoll_status combo = check_combination(VCOLL_OP_ALL_GATHER, algo, p);
  if (combo != VCOLL_OK) return combo;
  if (m == 0) return VCOLL_OK;
  if (!all_set(p, send) || !all_set(p, const_cast<const void* const*>(recv))) return VCOLL_ERR_INVALID_ARG;
  GatherArgs a;
  std::memset(&a, 0, sizeof(a));
  for (int r = 0; r < p; ++r) {
    a.ptr.src[r] = send[r];
    a.ptr.dst[r] = recv[r];
  }
  a.m = m;
  a.p = p;
  a.vec = all_aligned(p, send) && all_aligned(p, const_cast<const void* const*>(recv)) &&
          (m * elem_bytes(dtype)) % 16 == 0;
  a.lines = common_phase(p, const_cast<const void* const*>(recv), nullptr, 128) == 0 &&
            (m * elem_bytes(dtype)) % 128 == 0;
  return from_hip(launch_all_gather(a, dtype, static_cast<hipStream_t>(stream)));
}

vcoll_status vcoll_all_to_all(int p, int64_t row_elems, vcoll_dtype dtype, const int64_t* splits,
                              const void* const* send, void* const* recv,
                              const int32_t* const* src_rows, const int64_t* src_table_rows,
                              const int32_t* const* dst_rows, const int64_t* dst_table_rows,
                              void* stream) {
  if (!valid_p(p) || !valid_count(row_elems) || !valid_a2a_dtype(dtype) || !splits) return VCOLL_ERR_INVALID_ARG;
  const int64_t rb = row_elems * elem_bytes(dtype);
  std::vector<int64_t> sent, got;
  if (!valid_splits(p, splits, rb, sent, got)) return VCOLL_ERR_INVALID_ARG;
  auto gathers = [&](int i) { return src_rows && src_rows[i]; };
  auto scatters = [&](int j) { return dst_rows && dst_rows[j]; };
  for (int i = 0; i < p; ++i) {
    if (sent[i] > 0 && rb > 0 && (!send || !send[i])) return VCOLL_ERR_INVALID_ARG;
    if (got[i] > 0 && rb > 0 && (!recv || !recv[i])) return VCOLL_ERR_INVALID_ARG;
    if (gathers(i) && (!src_table_rows || src_table_rows[i] < 0 || src_table_rows[i] > INT32_MAX ||
                       !fits(src_table_rows[i], rb)))
      return VCOLL_ERR_INVALID_ARG;
    if (scatters(i) && (!dst_table_rows || dst_table_rows[i] < 0 || dst_table_rows[i] > INT32_MAX ||
                        !fits(dst_table_rows[i], rb)))
      return VCOLL_ERR_INVALID_ARG;
  }
  if (rb == 0) return VCOLL_OK;
  std::vector<int64_t> so, ro;
  block_offsets(p, splits, so, ro);

  // one descriptor per non-empty block; launches of up to kA2ABlocks blocks
  const int32_t rows_per_tile = static_cast<int32_t>(std::max<int64_t>(1, std::min<int64_t>(64, 32768 / rb)));
  std::vector<A2ABlock> blocks;
  std::vector<bool> block_vec;
  for (int i = 0; i < p; ++i)
    for (int j = 0; j < p; ++j) {
      const int64_t rows = splits[i * p + j];
      if (rows == 0) continue;
      A2ABlock b{};
      const bool g = gathers(i), s = scatters(j);
      b.src = static_cast<const char*>(send[i]) + (g ? 0 : so[i * p + j] * rb);
      b.dst = static_cast<char*>(recv[j]) + (s ? 0 : ro[i * p + j] * rb);
      b.src_idx = g ? src_rows[i] + so[i * p + j] : nullptr;
      b.dst_idx = s ? dst_rows[j] + ro[i * p + j] : nullptr;
      b.rows = static_cast<int32_t>(rows);
      b.src_limit = static_cast<int32_t>(g ? src_table_rows[i] : rows);
      b.dst_limit = static_cast<int32_t>(s ? dst_table_rows[j] : rows);
      blocks.push_back(b);
      block_vec.push_back(aligned16(b.src) && aligned16(b.dst));
    }
  if (!block_launch_tiles(blocks, rows_per_tile)) return VCOLL_ERR_UNSUPPORTED;
  for (size_t b0 = 0; b0 < blocks.size(); b0 += kA2ABlocks) {
    A2AArgs a;
    std::memset(&a, 0, sizeof(a));
    a.row_bytes = rb;
    a.rows_per_tile = rows_per_tile;
    a.esize = static_cast<int32_t>(elem_bytes(dtype));
    a.vec = (rb % 16) == 0;
    int64_t tiles = 0;
    const size_t nb = std::min<size_t>(kA2ABlocks, blocks.size() - b0);
    for (size_t k = 0; k < nb; ++k) {
      a.b[k] = blocks[b0 + k];
      a.b[k].tile_start = static_cast<int32_t>(tiles);
      tiles += (a.b[k].rows + rows_per_tile - 1) / rows_per_tile;
      if (!block_vec[b0 + k]) a.vec = 0;
    }
    a.nblocks = static_cast<int32_t>(nb);
    const vcoll_status st =
        from_hip(launch_all_to_all(a, static_cast<int32_t>(tiles), static_cast<hipStream_t>(stream)));
    if (st != VCOLL_OK) return st;
  }
  return VCOLL_OK;
}

vcoll_status vcoll_ledger(vcoll_op op, vcoll_algo algo, int p, int64_t n, vcoll_dtype dtype,
                          const int64_t* splits, int64_t row_elems, vcoll_msg* msgs, int64_t cap,
                          int64_t* n_msgs, int64_t* sent_bytes, int64_t* recv_bytes, int32_t* n_steps) {
  if (!valid_p(p) || !n_msgs) return VCOLL_ERR_INVALID_ARG;
  if (op < VCOLL_OP_ALLREDUCE || op > VCOLL_OP_ALL_TO_ALL) return VCOLL_ERR_INVALID_ARG;
  if (!(op == VCOLL_OP_ALL_TO_ALL ? valid_a2a_dtype(dtype) : valid_dtype(dtype))) return VCOLL_ERR_INVALID_ARG;
  if (op == VCOLL_OP_ALL_TO_ALL) {
    std::vector<int64_t> sent, got;
    if (!splits || !valid_count(row_elems) ||
        !valid_splits(p, splits, row_elems * elem_bytes(dtype), sent, got))
      return VCOLL_ERR_INVALID_ARG;
  } else {
    if (!valid_count(n) || !valid_algo(algo)) return VCOLL_ERR_INVALID_ARG;
    const vcoll_status combo = check_combination(op, algo, p);
    if (combo != VCOLL_OK) return combo;
  }
  std::vector<vcoll_msg> out;
  int32_t steps = 0;
  build_ledger(op, algo, p, n, elem_bytes(dtype), splits, row_elems, out, &steps);
  return emit_ledger(out, steps, p, msgs, cap, n_msgs, sent_bytes, recv_bytes, n_steps);
}

vcoll_status vcoll_ledger_rooted(vcoll_op op, vcoll_algo algo, int p, int64_t n, vcoll_dtype dtype, int root,
                                 int64_t blocks, vcoll_msg* msgs, int64_t cap, int64_t* n_msgs,
                                 int64_t* sent_bytes, int64_t* recv_bytes, int32_t* n_steps) {
  if (!valid_p(p) || !valid_count(n) || !valid_dtype(dtype) || !n_msgs || root < 0 || root >= p)
    return VCOLL_ERR_INVALID_ARG;
  if (op != VCOLL_OP_BROADCAST && op != VCOLL_OP_REDUCE) return VCOLL_ERR_INVALID_ARG;
  std::vector<vcoll_msg> out;
  int32_t steps = 0;
  const vcoll_status st = build_ledger_rooted(op, algo, p, n, elem_bytes(dtype), root, blocks, out, &steps);
  if (st != VCOLL_OK) return st;
  return emit_ledger(out, steps, p, msgs, cap, n_msgs, sent_bytes, recv_bytes, n_steps);
}

vcoll_status vcoll_broadcast(int p, int64_t n, vcoll_dtype dtype, int root, const void* send, void* const* recv,
                             void* stream) {
  if (!valid_p(p) || !valid_count(n) || !valid_dtype(dtype) || root < 0 || root >= p) return VCOLL_ERR_INVALID_ARG;
  if (n == 0) return VCOLL_OK;
  if (!send || !recv) return VCOLL_ERR_INVALID_ARG;
  BcastArgs a;
  std::memset(&a, 0, sizeof(a));
  a.src = send;
  a.n = n;
  a.vec = aligned16(send);
  a.lines = 1;
  for (int r = 0; r < p; ++r) {
    if (r == root && (recv[r] == nullptr || recv[r] == send)) continue;
    if (!recv[r]) return VCOLL_ERR_INVALID_ARG;
    a.dst[a.q++] = recv[r];
    a.vec = a.vec && aligned16(recv[r]);
    a.lines = a.lines && (reinterpret_cast<uintptr_t>(recv[r]) & 127u) == 0;
  }
  return from_hip(launch_broadcast(a, dtype, static_cast<hipStream_t>(stream)));
}

vcoll_status vcoll_reduce(vcoll_algo algo, int p, int64_t n, vcoll_dtype dtype, int root,
                          const void* const* send, void* recv, void* stream) {
  if (!valid_p(p) || !valid_count(n) || !valid_dtype(dtype) || root < 0 || root >= p) return VCOLL_ERR_INVALID_ARG;
  if (algo != VCOLL_BINARY_TREE)
    return (algo >= VCOLL_RING && algo <= VCOLL_PIPELINED_CHAIN) ? VCOLL_ERR_UNSUPPORTED : VCOLL_ERR_INVALID_ARG;
  if (n == 0) return VCOLL_OK;
  if (!all_set(p, send) || !recv) return VCOLL_ERR_INVALID_ARG;
  ReduceArgs a;
  std::memset(&a, 0, sizeof(a));
  a.dst[0] = recv;                  // the whole vector is one chunk, written to the root only
  a.q = n;
  a.r = 0;
  a.p = p;
  a.vec = all_aligned(p, send) && aligned16(recv);
  a.align = 16;                     // one chunk starting at element 0: no tile realignment
  a.src_align = 16;
  // the tree runs on ranks relative to the root: leaf v is rank (v + root) mod p
  const OrderProgram prog = order_program(VCOLL_BINARY_TREE, p);
  auto input = [&](int k) { return send[(prog.rank[k] + root) % p]; };
  if (has_fixed_kernel(p)) {
    for (int k = 0; k < p; ++k) a.leaf[k] = input(k);                         // leaves in program order
  } else {
    set_tree_groups(a, VCOLL_BINARY_TREE, p, input);
  }
  return from_hip(launch_reduce(a, dtype, VCOLL_BINARY_TREE, true, n, 1, static_cast<hipStream_t>(stream)));
}

vcoll_status vcoll_moe_plan(int p, int64_t tokens, int topk, int experts_per_rank,
                            const int32_t* topk_ids, int64_t* splits, int32_t* src_rows,
                            int32_t* dst_rows) {
  if (!valid_p(p) || !valid_count(tokens) || topk < 1 || experts_per_rank < 1) return VCOLL_ERR_INVALID_ARG;
  if (!pairs_fit(tokens, topk)) return VCOLL_ERR_INVALID_ARG;
  if (!splits || (tokens > 0 && (!topk_ids || !src_rows || !dst_rows))) return VCOLL_ERR_INVALID_ARG;
  return moe_plan(p, tokens, topk, experts_per_rank, topk_ids, splits, src_rows, dst_rows);
}

namespace {

// Enqueue a list of step operations as launches of at most kStepOps each.
vcoll_status run_step_ops(const std::vector<StepLaunchOp>& ops, hipStream_t stream, int32_t* launches) {
  for (size_t b0 = 0; b0 < ops.size(); b0 += kStepOps) {
    StepArgs a;
    std::memset(&a, 0, sizeof(a));
    int64_t tiles = 0;
    const size_t nb = std::min<size_t>(kStepOps, ops.size() - b0);
    for (size_t k = 0; k < nb; ++k) {
      a.op[k] = ops[b0 + k];
      a.op[k].tile_start = static_cast<int32_t>(tiles);
      tiles += (a.op[k].count + kStepTile - 1) / kStepTile;
    }
    a.nops = static_cast<int32_t>(nb);
    if (tiles > INT32_MAX) return VCOLL_ERR_INVALID_ARG;
    const vcoll_status st = from_hip(launch_step(a, static_cast<int32_t>(tiles), stream));
    if (st != VCOLL_OK) return st;
    if (launches) ++*launches;
  }
  return VCOLL_OK;
}

}  // namespace

namespace {

// Arguments of a stepwise all-reduce, before any workspace question.
vcoll_status stepwise_args(vcoll_algo algo, int p, int64_t n, vcoll_dtype dtype, const void* const* send,
                           void* const* recv) {
  if (!valid_p(p) || !valid_count(n) || !valid_dtype(dtype) || !valid_algo(algo)) return VCOLL_ERR_INVALID_ARG;
  if (n == 0) return VCOLL_OK;
  if (!all_set(p, send) || !all_set(p, const_cast<const void* const*>(recv))) return VCOLL_ERR_INVALID_ARG;
  return VCOLL_OK;
}

// The stepwise all-reduce on validated arguments; for bf16, `workspace`
// holds at least p*n float32.
vcoll_status stepwise_run(vcoll_algo algo, int p, int64_t n, vcoll_dtype dtype, const void* const* send,
                          void* const* recv, void* workspace, int32_t* n_launches, void* stream) {
  const bool bf16 = dtype == VCOLL_BF16;
  // working buffers: recv itself for float32, the float32 workspace for bf16
  std::vector<float*> W(p);
  for (int r = 0; r < p; ++r)
    W[r] = bf16 ? static_cast<float*>(workspace) + static_cast<int64_t>(r) * n : static_cast<float*>(recv[r]);
  std::vector<std::vector<StepOp>> steps;
  build_step_program(algo, p, n, bf16, steps);
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto op = [](int32_t kind, const void* src, void* dst, int64_t count) {
    StepLaunchOp o{};
    o.src = src;
    o.dst = dst;
    o.count = count;
    o.kind = kind;
    return o;
  };
  // load the inputs into the working buffers
  std::vector<StepLaunchOp> ops;
  for (int r = 0; r < p; ++r) {
    if (bf16) ops.push_back(op(SK_WIDEN_BF16, send[r], W[r], n));
    else if (send[r] != recv[r]) ops.push_back(op(SK_COPY, send[r], W[r], n));
  }
  vcoll_status st = run_step_ops(ops, s, n_launches);
  if (st != VCOLL_OK) return st;
  // one launch (or more, for many operations) per algorithm step
  for (const std::vector<StepOp>& step : steps) {
    ops.clear();
    for (const StepOp& o : step) {
      if (o.count == 0) continue;
      ops.push_back(op(o.kind, W[o.src] + o.off, W[o.dst] + o.off, o.count));
    }
    st = run_step_ops(ops, s, n_launches);
    if (st != VCOLL_OK) return st;
  }
  if (bf16) {
    ops.clear();
    for (int r = 0; r < p; ++r) ops.push_back(op(SK_STORE_BF16, W[r], recv[r], n));
    st = run_step_ops(ops, s, n_launches);
  }
  return st;
}

}  // namespace

vcoll_status vcoll_allreduce_stepwise(vcoll_algo algo, int p, int64_t n, vcoll_dtype dtype,
                                      const void* const* send, void* const* recv, void* workspace,
                                      int64_t workspace_bytes, int32_t* n_launches, void* stream) {
  if (n_launches) *n_launches = 0;
  const vcoll_status st = stepwise_args(algo, p, n, dtype, send, recv);
  if (st != VCOLL_OK || n == 0) return st;
  if (dtype == VCOLL_BF16) {
    if (!workspace) return VCOLL_ERR_INVALID_ARG;
    if (workspace_bytes < static_cast<int64_t>(p) * n * 4) return VCOLL_ERR_BUFFER_TOO_SMALL;
  }
  return stepwise_run(algo, p, n, dtype, send, recv, workspace, n_launches, stream);
}

vcoll_status vcoll_allreduce_stepwise_static(vcoll_algo algo, int p, int64_t n, vcoll_dtype dtype,
                                             const void* const* send, void* const* recv,
                                             int32_t* n_launches, void* stream) {
  if (n_launches) *n_launches = 0;
  const vcoll_status st = stepwise_args(algo, p, n, dtype, send, recv);
  if (st != VCOLL_OK || n == 0) return st;
  void* workspace = nullptr;
  if (dtype == VCOLL_BF16) {
    // p <= 128 and n <= 2^48, so the product fits in int64
    if (static_cast<int64_t>(p) * n * 4 > VCOLL_STEP_SCRATCH_BYTES) return VCOLL_ERR_SCRATCH_LIMIT;
    const hipError_t e = step_scratch(&workspace);
    if (e != hipSuccess) return from_hip(e);
  }
  return stepwise_run(algo, p, n, dtype, send, recv, workspace, n_launches, stream);
}

// Blocks of a stepwise pipelined chain: each block adds one launch.
constexpr int64_t kMaxChainBlocks = 65536;

vcoll_status vcoll_broadcast_stepwise(vcoll_algo algo, int p, int64_t n, vcoll_dtype dtype, int root, int64_t blocks,
                                      const void* send, void* const* recv, int32_t* n_launches, void* stream) {
  if (n_launches) *n_launches = 0;
  if (!valid_p(p) || !valid_count(n) || !valid_dtype(dtype) || root < 0 || root >= p) return VCOLL_ERR_INVALID_ARG;
  if (algo == VCOLL_PIPELINED_CHAIN && blocks > kMaxChainBlocks) return VCOLL_ERR_INVALID_ARG;
  std::vector<vcoll_msg> msgs;
  int32_t n_steps = 0;
  const vcoll_status led = build_ledger_rooted(VCOLL_OP_BROADCAST, algo, p, n, elem_bytes(dtype), root,
                                               blocks, msgs, &n_steps);
  if (led != VCOLL_OK) return led;
  if (n == 0) return VCOLL_OK;
  if (!send || !recv) return VCOLL_ERR_INVALID_ARG;
  for (int r = 0; r < p; ++r)
    if (r != root && !recv[r]) return VCOLL_ERR_INVALID_ARG;
  // the root's messages leave from `send`; its own receive buffer (if any,
  // and not `send` itself) gets a local copy first, which is no message, and
  // receives the messages addressed to the root (the scatter + all-gather
  // ring sends the root chunks it already holds; with no separate buffer
  // they are dropped, `send` is never written)
  const int64_t es = elem_bytes(dtype);
  const int32_t kind = dtype == VCOLL_F32 ? SK_COPY : SK_COPY16;
  char* const root_out = (recv[root] && recv[root] != send) ? static_cast<char*>(recv[root]) : nullptr;
  auto src_buf = [&](int r) -> const char* {
    return static_cast<const char*>(r == root ? send : recv[r]);
  };
  auto dst_buf = [&](int r) -> char* { return r == root ? root_out : static_cast<char*>(recv[r]); };
  auto op = [&](const void* src, void* dst, int64_t count) {
    StepLaunchOp o{};
    o.src = src;
    o.dst = dst;
    o.count = count;
    o.kind = kind;
    return o;
  };
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::vector<StepLaunchOp> ops;
  if (root_out) {
    ops.push_back(op(send, root_out, n));
    const vcoll_status st = run_step_ops(ops, s, n_launches);
    if (st != VCOLL_OK) return st;
  }
  size_t k = 0;
  for (int32_t step = 0; step < n_steps; ++step) {
    ops.clear();
    for (; k < msgs.size() && msgs[k].step == step; ++k) {
      const vcoll_msg& m = msgs[k];
      if (m.count > 0 && dst_buf(m.dst))
        ops.push_back(op(src_buf(m.src) + m.src_off * es, dst_buf(m.dst) + m.dst_off * es, m.count));
    }
    const vcoll_status st = run_step_ops(ops, s, n_launches);
    if (st != VCOLL_OK) return st;
  }
  return VCOLL_OK;
}

vcoll_status vcoll_allreduce_hierarchical(int nodes, int local, int64_t n, vcoll_dtype dtype,
                                          const void* const* send, void* const* recv, void* stream) {
  if (!valid_grid(nodes, local) || !valid_count(n) || !valid_dtype(dtype))
    return VCOLL_ERR_INVALID_ARG;
  if (n == 0) return VCOLL_OK;
  const int p = nodes * local;
  if (!all_set(p, send) || !all_set(p, const_cast<const void* const*>(recv))) return VCOLL_ERR_INVALID_ARG;
  HierArgs a;
  std::memset(&a, 0, sizeof(a));
  for (int r = 0; r < p; ++r) {
    a.ptr.src[r] = send[r];
    a.ptr.dst[r] = recv[r];
  }
  a.n = n;
  a.nodes = nodes;
  a.local = local;
  a.vec = all_aligned(p, send) && all_aligned(p, const_cast<const void* const*>(recv));
  const Chunks ch(n, local);
  const int64_t max_segment = (ch.count(0) + nodes - 1) / nodes;
  return from_hip(launch_hierarchical(a, dtype, max_segment, static_cast<hipStream_t>(stream)));
}

vcoll_status vcoll_ledger_hierarchical(int nodes, int local, int64_t n, vcoll_dtype dtype, vcoll_msg* msgs,
                                       int64_t cap, int64_t* n_msgs, int64_t* sent_bytes,
                                       int64_t* recv_bytes, int32_t* n_steps) {
  if (!valid_grid(nodes, local) || !valid_count(n) || !valid_dtype(dtype) || !n_msgs)
    return VCOLL_ERR_INVALID_ARG;
  const int p = nodes * local;
  std::vector<vcoll_msg> out;
  int32_t steps = 0;
  build_ledger_hierarchical(nodes, local, n, elem_bytes(dtype), out, &steps);
  return emit_ledger(out, steps, p, msgs, cap, n_msgs, sent_bytes, recv_bytes, n_steps);
}

vcoll_status vcoll_moe_slots(int p, int64_t tokens, int topk, const int64_t* splits, const int32_t* dst_rows,
                             int32_t* slots) {
  if (!valid_p(p) || !valid_count(tokens) || topk < 1 || !splits || (tokens > 0 && (!dst_rows || !slots)))
    return VCOLL_ERR_INVALID_ARG;
  if (!pairs_fit(tokens, topk)) return VCOLL_ERR_INVALID_ARG;
  std::vector<int64_t> sent, got;                                // receive rows are int32 in the slots
  if (!valid_splits(p, splits, 0, sent, got)) return VCOLL_ERR_INVALID_ARG;
  return moe_slots(p, tokens, topk, splits, dst_rows, slots);
}

vcoll_status vcoll_moe_dedup_slots(int p, int64_t tokens, int topk, const int64_t* splits_unique,
                                   const int32_t* src_unique, int32_t* slots) {
  if (!valid_p(p) || !valid_count(tokens) || topk < 1 || !splits_unique) return VCOLL_ERR_INVALID_ARG;
  if (!pairs_fit(tokens, topk)) return VCOLL_ERR_INVALID_ARG;
  if (tokens > 0 && (!src_unique || !slots)) return VCOLL_ERR_INVALID_ARG;
  std::vector<int64_t> sent, got;                                // receive rows are int32 in the slots
  if (!valid_splits(p, splits_unique, 0, sent, got)) return VCOLL_ERR_INVALID_ARG;
  for (int i = 0; i < p; ++i)
    if (sent[i] > tokens * topk) return VCOLL_ERR_INVALID_ARG;  // src_unique holds tokens*topk entries per rank
  return moe_dedup_slots(p, tokens, topk, splits_unique, src_unique, slots);
}

vcoll_status vcoll_moe_expand_slots(int64_t unique_rows, int topk, const int32_t* expand, int64_t expand_count,
                                    int32_t* slots) {
  if (!valid_count(unique_rows) || topk < 1 || !valid_count(expand_count)) return VCOLL_ERR_INVALID_ARG;
  if (!pairs_fit(unique_rows, topk) || expand_count > INT32_MAX) return VCOLL_ERR_INVALID_ARG;
  if ((expand_count > 0 && !expand) || (unique_rows > 0 && !slots)) return VCOLL_ERR_INVALID_ARG;
  return moe_expand_slots(unique_rows, topk, expand, expand_count, slots);
}

vcoll_status vcoll_moe_dispatch(int p, int64_t tokens, int topk, int64_t hidden, vcoll_dtype dtype, int fp8,
                                const void* const* token_tables, const int32_t* const* slots,
                                void* const* recv, const int64_t* recv_rows, void* stream) {
  if (!valid_p(p) || !valid_count(tokens) || topk < 1 || !valid_count(hidden) || !valid_dtype(dtype) || !recv_rows)
    return VCOLL_ERR_INVALID_ARG;
  if (fp8 && (dtype != VCOLL_BF16 || hidden % 128 != 0)) return VCOLL_ERR_INVALID_ARG;
  if (!pairs_fit(tokens, topk) || hidden > INT32_MAX / 4) return VCOLL_ERR_INVALID_ARG;
  if (tokens == 0 || hidden == 0) return VCOLL_OK;
  if (!token_tables || !slots || !recv) return VCOLL_ERR_INVALID_ARG;
  const int64_t rb = hidden * elem_bytes(dtype);
  const int64_t orb = fp8 ? hidden + hidden / 32 : rb;
  if (!fits(tokens, rb)) return VCOLL_ERR_INVALID_ARG;
  bool vec = rb % 16 == 0;
  for (int j = 0; j < p; ++j) {
    if (recv_rows[j] < 0 || recv_rows[j] > INT32_MAX || !fits(recv_rows[j], orb)) return VCOLL_ERR_INVALID_ARG;
    if (recv_rows[j] > 0 && !recv[j]) return VCOLL_ERR_INVALID_ARG;
    if (recv_rows[j] > 0 && fp8 && (reinterpret_cast<uintptr_t>(recv[j]) & 3u) != 0) return VCOLL_ERR_INVALID_ARG;
    if (recv_rows[j] > 0) vec = vec && aligned16(recv[j]);
  }
  for (int i = 0; i < p; ++i) {
    if (!token_tables[i] || !slots[i]) return VCOLL_ERR_INVALID_ARG;
    if (fp8 && !aligned16(token_tables[i])) return VCOLL_ERR_INVALID_ARG;
    vec = vec && aligned16(token_tables[i]);
  }
  PushArgs a;
  std::memset(&a, 0, sizeof(a));
  for (int j = 0; j < p; ++j) {
    a.recv[j] = recv[j];
    a.recv_rows[j] = static_cast<int32_t>(recv_rows[j]);
  }
  a.tokens = tokens;
  a.row_bytes = rb;
  a.out_row_bytes = orb;
  a.hidden = hidden;
  a.topk = topk;
  a.p = p;
  a.vec = vec;
  a.vec_out = orb % 16 == 0;
  for (int j = 0; j < p; ++j)
    if (recv_rows[j] > 0) a.vec_out = a.vec_out && aligned16(recv[j]);
  // up to 16 KiB of token rows per workgroup (one 7168-element bf16 token)
  a.tokens_per_tile = static_cast<int32_t>(std::max<int64_t>(1, std::min<int64_t>(64, 16384 / rb)));
  a.segments = push_segments(rb, fp8 != 0, vec);
  for (int i = 0; i < p; ++i) {
    a.table[i] = token_tables[i];
    a.slots[i] = slots[i];
  }
  // the grid (tiles x segments workgroups of up to 512 threads) must stay within 2^32 threads
  if ((a.tokens + a.tokens_per_tile - 1) / a.tokens_per_tile * a.segments > (int64_t(UINT32_MAX) >> 9))
    return VCOLL_ERR_UNSUPPORTED;
  return from_hip(launch_dispatch_push(a, fp8 != 0, static_cast<hipStream_t>(stream)));
}

vcoll_status vcoll_moe_combine(int p, int64_t tokens, int topk, int64_t hidden, vcoll_dtype dtype,
                               const void* const* expert_out, const int64_t* expert_rows,
                               const int32_t* const* slots, void* const* out, void* stream) {
  if (!valid_p(p) || !valid_count(tokens) || topk < 1 || !valid_count(hidden) || !valid_dtype(dtype) ||
      !expert_rows)
    return VCOLL_ERR_INVALID_ARG;
  if (!pairs_fit(tokens, topk) || hidden > INT32_MAX / 4) return VCOLL_ERR_INVALID_ARG;
  const int64_t rb = hidden * elem_bytes(dtype);
  if (!fits(tokens * topk, rb)) return VCOLL_ERR_INVALID_ARG;
  if (tokens == 0 || hidden == 0) return VCOLL_OK;
  if (!expert_out || !slots || !out) return VCOLL_ERR_INVALID_ARG;
  bool vec = rb % 16 == 0;
  for (int j = 0; j < p; ++j) {
    if (expert_rows[j] < 0 || expert_rows[j] > INT32_MAX || !fits(expert_rows[j], rb)) return VCOLL_ERR_INVALID_ARG;
    if (expert_rows[j] > 0 && !expert_out[j]) return VCOLL_ERR_INVALID_ARG;
    if (expert_rows[j] > 0) vec = vec && aligned16(expert_out[j]);
  }
  for (int i = 0; i < p; ++i) {
    if (!slots[i] || !out[i]) return VCOLL_ERR_INVALID_ARG;
    vec = vec && aligned16(out[i]);
  }
  CombineArgs a;
  std::memset(&a, 0, sizeof(a));
  for (int r = 0; r < p; ++r) {
    a.src[r] = expert_out[r];
    a.src_rows[r] = static_cast<int32_t>(expert_rows[r]);
    a.out[r] = out[r];
    a.slots[r] = slots[r];
  }
  a.tokens = tokens;
  a.row_bytes = rb;
  a.topk = topk;
  a.p = p;
  a.vec = vec;
  // up to 128 KiB of output rows per workgroup (one token's 8 rows of 7168 bf16)
  a.tokens_per_tile = static_cast<int32_t>(std::max<int64_t>(1, std::min<int64_t>(64, 131072 / (topk * rb))));
  a.segments = pull_segments(rb, vec);
  // the grid (tiles x segments workgroups of up to 512 threads) must stay within 2^32 threads
  if ((a.tokens + a.tokens_per_tile - 1) / a.tokens_per_tile * a.segments > (int64_t(UINT32_MAX) >> 9))
    return VCOLL_ERR_UNSUPPORTED;
  return from_hip(launch_combine_pull(a, static_cast<hipStream_t>(stream)));
}

vcoll_status vcoll_moe_plan_dedup(int p, int64_t tokens, int topk, int experts_per_rank, const int32_t* topk_ids,
                                  int64_t* splits_unique, int32_t* src_unique, int32_t* expand,
                                  int64_t* expand_count) {
  if (!valid_p(p) || !valid_count(tokens) || topk < 1 || experts_per_rank < 1 || !topk_ids || !splits_unique ||
      !src_unique || !expand || !expand_count)
    return VCOLL_ERR_INVALID_ARG;
  if (!pairs_fit(tokens, topk) || static_cast<int64_t>(p) * tokens * topk > INT32_MAX) return VCOLL_ERR_INVALID_ARG;
  return moe_plan_dedup(p, tokens, topk, experts_per_rank, topk_ids, splits_unique, src_unique, expand,
                        expand_count);
}

vcoll_status vcoll_moe_dispatch_fp8(int p, int64_t hidden, const int64_t* splits, const void* const* tokens,
                                    const int64_t* token_rows, const int32_t* const* src_rows,
                                    void* const* recv, void* stream) {
  if (!valid_p(p) || hidden <= 0 || hidden % 128 != 0 || hidden > INT32_MAX / 2 || !splits || !token_rows ||
      !src_rows)
    return VCOLL_ERR_INVALID_ARG;
  const int64_t orb = hidden + hidden / 32;
  std::vector<int64_t> sent, got;
  if (!valid_splits(p, splits, orb, sent, got)) return VCOLL_ERR_INVALID_ARG;
  for (int i = 0; i < p; ++i) {
    if (sent[i] > 0 && (!tokens || !tokens[i] || !aligned16(tokens[i]) || !src_rows[i] ||
                        token_rows[i] < 0 || token_rows[i] > INT32_MAX))
      return VCOLL_ERR_INVALID_ARG;
    if (got[i] > 0 && (!recv || !recv[i] || (reinterpret_cast<uintptr_t>(recv[i]) & 3u) != 0))
      return VCOLL_ERR_INVALID_ARG;
  }
  std::vector<int64_t> so, ro;
  block_offsets(p, splits, so, ro);
  const int32_t rows_per_tile = static_cast<int32_t>(std::max<int64_t>(1, std::min<int64_t>(64, 32768 / (2 * hidden))));
  bool vec_out = orb % 16 == 0;                 // 16-byte code stores when every receive row is aligned
  for (int j = 0; j < p; ++j)
    if (got[j] > 0) vec_out = vec_out && aligned16(recv[j]);
  std::vector<A2ABlock> blocks;
  for (int i = 0; i < p; ++i)
    for (int j = 0; j < p; ++j) {
      const int64_t rows = splits[i * p + j];
      if (rows == 0) continue;
      A2ABlock b{};
      b.src = static_cast<const char*>(tokens[i]);
      b.dst = static_cast<char*>(recv[j]) + ro[i * p + j] * orb;
      b.src_idx = src_rows[i] + so[i * p + j];
      b.dst_idx = nullptr;
      b.rows = static_cast<int32_t>(rows);
      b.src_limit = static_cast<int32_t>(token_rows[i]);
      b.dst_limit = static_cast<int32_t>(rows);
      blocks.push_back(b);
    }
  if (!block_launch_tiles(blocks, rows_per_tile)) return VCOLL_ERR_UNSUPPORTED;
  for (size_t b0 = 0; b0 < blocks.size(); b0 += kA2ABlocks) {
    Fp8Args a;
    std::memset(&a, 0, sizeof(a));
    a.hidden = hidden;
    a.out_row_bytes = orb;
    a.rows_per_tile = rows_per_tile;
    a.vec_out = vec_out;
    int64_t tiles = 0;
    const size_t nb = std::min<size_t>(kA2ABlocks, blocks.size() - b0);
    for (size_t k = 0; k < nb; ++k) {
      a.b[k] = blocks[b0 + k];
      a.b[k].tile_start = static_cast<int32_t>(tiles);
      tiles += (a.b[k].rows + rows_per_tile - 1) / rows_per_tile;
    }
    a.nblocks = static_cast<int32_t>(nb);
    const vcoll_status st =
        from_hip(launch_dispatch_fp8(a, static_cast<int32_t>(tiles), static_cast<hipStream_t>(stream)));
    if (st != VCOLL_OK) return st;
  }
  return VCOLL_OK;
}

vcoll_status vcoll_bench_stream(vcoll_bench_kind kind, void* dst, const void* src, int64_t bytes, void* stream) {
  if (kind < VCOLL_BENCH_COPY || kind > VCOLL_BENCH_COPY_PLAIN) return VCOLL_ERR_INVALID_ARG;
  if (bytes < 0 || (bytes % 16) != 0) return VCOLL_ERR_INVALID_ARG;
  if (bytes == 0) return VCOLL_OK;
  const bool uses_src = kind != VCOLL_BENCH_WRITE;
  if (!dst || (uses_src && (!src || !aligned16(src)))) return VCOLL_ERR_INVALID_ARG;
  if (kind == VCOLL_BENCH_READ ? (reinterpret_cast<uintptr_t>(dst) & 3u) != 0 : !aligned16(dst))
    return VCOLL_ERR_INVALID_ARG;
  return from_hip(launch_stream(kind, dst, src, bytes, static_cast<hipStream_t>(stream)));
}

vcoll_status vcoll_bench_copy(void* dst, const void* src, int64_t bytes, void* stream) {
  return vcoll_bench_stream(VCOLL_BENCH_COPY, dst, src, bytes, stream);
}

}  // extern "C"
