// The host half of libvcoll under AddressSanitizer and UndefinedBehavior-
// Sanitizer: argument validation, schedules, ledgers, the alpha-beta model
// and the MoE plans, with the kernel launchers replaced by stubs that record
// each launch and return success (fake, never dereferenced device
// addresses). Built with g++ and run by tests/test_host_sanitize.py; exits
// non-zero on the first failed check (the sanitizers abort on their own).
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <vector>

#include "bench.h"
#include "hier.h"
#include "move.h"
#include "reduce.h"
#include "schedule.h"
#include "step.h"
#include "vcoll.h"

static long g_launches = 0;
using vcoll::kMaxRanks;
using vcoll::kA2ABlocks;

extern "C" const char* hipGetErrorString(hipError_t) { return "stub"; }
// a 256-compute-unit device 0, so that the size-selected kernels are exercised
extern "C" hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
extern "C" hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) { *v = 256; return hipSuccess; }

namespace vcoll {
hipError_t launch_reduce(const ReduceArgs& a, vcoll_dtype, vcoll_algo algo, bool, int64_t max_chunk, int chunks,
                         hipStream_t) {
  if (a.p < 1 || a.p > kMaxRanks || chunks < 1 || max_chunk < 0) std::abort();
  // the input phase the unaligned reduce-scatter aligns its waves to: 128
  // only when every input shares it
  if (!(a.src_align == 16 || a.src_align == 128) || a.src_phase < 0 || a.src_phase >= a.src_align ||
      a.src_phase % 16 != 0)
    std::abort();
  // the tree programs' groups (the kernels with a run-time p read them): a
  // first leaf for every group, a second one exactly for the folded pairs
  if (algo != VCOLL_RING && !has_fixed_kernel(a.p)) {
    int first[kMaxRanks + 1] = {};
    const int g = order_groups(algo, a.p, first);
    if (a.groups != g) std::abort();
    for (int q = 0; q < g; ++q)
      if (!a.leaf[q] || (a.leaf[kMaxRanks + q] != nullptr) != (first[q + 1] - first[q] == 2)) std::abort();
  }
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_hierarchical(const HierArgs&, vcoll_dtype, int64_t, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_all_gather(const GatherArgs& a, vcoll_dtype dtype, hipStream_t) {
  if (a.p < 1 || a.m < 0) std::abort();
  // whole-line tiles: every output on a 128-byte line and blocks a whole number of lines
  bool lines = a.m * (dtype == VCOLL_F32 ? 4 : 2) % 128 == 0;
  for (int r = 0; r < a.p; ++r) lines = lines && reinterpret_cast<uintptr_t>(a.ptr.dst[r]) % 128 == 0;
  if ((a.lines != 0) != lines) std::abort();
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_broadcast(const BcastArgs& a, vcoll_dtype, hipStream_t) {
  if (a.q < 0 || a.q > kMaxRanks) std::abort();
  bool lines = true;
  for (int r = 0; r < a.q; ++r) lines = lines && reinterpret_cast<uintptr_t>(a.dst[r]) % 128 == 0;
  if ((a.lines != 0) != lines) std::abort();
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_all_to_all(const A2AArgs& a, int32_t tiles, hipStream_t) {
  if (a.nblocks < 1 || a.nblocks > kA2ABlocks || tiles < 1) std::abort();
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_dispatch_fp8(const Fp8Args&, int32_t, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_dispatch_push(const PushArgs&, bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_combine_pull(const CombineArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
int32_t push_segments(int64_t row_bytes, bool fp8, bool vec) { return fp8 || !vec ? 1 : int32_t((row_bytes / 16 + 127) / 128); }
int32_t pull_segments(int64_t row_bytes, bool vec) { return vec ? int32_t((row_bytes / 16 + 63) / 64) : 1; }
hipError_t launch_stream(vcoll_bench_kind, void*, const void*, int64_t, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_step(const StepArgs&, int32_t, hipStream_t) { ++g_launches; return hipSuccess; }
int64_t burst_tile_max(vcoll_dtype dtype) { return dtype == VCOLL_F32 ? 25 * 256 : 16 * 256; }
}  // namespace vcoll
static long g_burst = 0;
namespace vcoll {
hipError_t launch_burst_ring(const BurstArgs& a, vcoll_dtype dtype, int tiles, hipStream_t) {
  // the tiles cover the whole vectors of the largest chunk, and every tile
  // starts inside it
  const int64_t ve = dtype == VCOLL_F32 ? 4 : 8;
  int64_t cv = 0;
  for (int c = 0; c < a.p; ++c) {
    const int64_t e0 = c * a.q + (c < a.r ? c : a.r), e1 = e0 + a.q + (c < a.r ? 1 : 0);
    const int64_t whole = e1 / ve - burst_first_vector(e0, static_cast<int>(ve), a.align, a.phase);
    cv = whole > cv ? whole : cv;
  }
  if (!(a.tv >= 1 && a.tv <= burst_tile_max(dtype) && a.tv % 8 == 0 && int64_t(tiles - 1) * a.tv < cv &&
        int64_t(tiles) * a.tv >= cv && a.r >= 0 && a.r < a.p && (a.align == 16 || a.align == 128) &&
        a.phase >= 0 && a.phase < a.align && a.phase % 16 == 0)) {
    std::fprintf(stderr, "burst tiling does not cover the chunk\n");
    std::abort();
  }
  ++g_launches;
  ++g_burst;
  return hipSuccess;
}
// the scratch lookup of the allocation-free stepwise mode: a host stand-in
// address (the stubbed launches never dereference it)
hipError_t step_scratch(void** ptr) {
  static float stand_in[4];
  *ptr = stand_in;
  return hipSuccess;
}
}  // namespace vcoll

#define CHECK(cond)                                                             \
  do {                                                                          \
    if (!(cond)) {                                                              \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      std::exit(1);                                                             \
    }                                                                           \
  } while (0)

static void* fake(int r) { return reinterpret_cast<void*>(uintptr_t(0x10000000) + uintptr_t(r) * 0x1000000); }

static void ledgers(std::mt19937_64& rng) {
  const int ps[] = {1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 15, 16, 17, 24, 31, 32, 33, 64, 72, 100, 127, 128};
  const vcoll_algo algos[] = {VCOLL_RING, VCOLL_RECURSIVE_DOUBLING, VCOLL_RABENSEIFNER, VCOLL_BINARY_TREE};
  for (int p : ps) {
    const int64_t ns[] = {0, 1, p - 1 > 0 ? p - 1 : 1, p, p + 1, 1000, int64_t(1) << 20};
    for (int64_t n : ns)
      for (vcoll_op op : {VCOLL_OP_ALLREDUCE, VCOLL_OP_REDUCE_SCATTER, VCOLL_OP_ALL_GATHER})
        for (vcoll_algo algo : algos) {
          int64_t count = -1;
          vcoll_status st = vcoll_ledger(op, algo, p, n, VCOLL_F32, nullptr, 0, nullptr, 0, &count, nullptr, nullptr,
                                         nullptr);
          if (st == VCOLL_ERR_UNSUPPORTED) continue;
          CHECK(st == VCOLL_OK && count >= 0);
          std::vector<vcoll_msg> msgs(count + 1);
          std::vector<int64_t> sent(p), got(p);
          int32_t steps = -1;
          if (count > 0) {
            CHECK(vcoll_ledger(op, algo, p, n, VCOLL_F32, nullptr, 0, msgs.data(), count - 1, &count, nullptr,
                               nullptr, nullptr) == VCOLL_ERR_BUFFER_TOO_SMALL);
          }
          CHECK(vcoll_ledger(op, algo, p, n, VCOLL_BF16, nullptr, 0, msgs.data(), count, &count, sent.data(),
                             got.data(), &steps) == VCOLL_OK);
          int64_t s = 0, g = 0;
          for (int r = 0; r < p; ++r) {
            s += sent[r];
            g += got[r];
          }
          CHECK(s == g && steps >= 0);
          if (op == VCOLL_OP_ALLREDUCE && (algo == VCOLL_RING || algo == VCOLL_RABENSEIFNER) && n % p == 0 &&
              (p & (p - 1)) == 0)
            for (int r = 0; r < p; ++r) CHECK(sent[r] == 2 * (p - 1) * (n / p) * 2);
        }
    // all-to-all with random splits
    std::vector<int64_t> splits(size_t(p) * p);
    for (auto& v : splits) v = int64_t(rng() % 5);
    int64_t count = 0;
    CHECK(vcoll_ledger(VCOLL_OP_ALL_TO_ALL, VCOLL_RING, p, 0, VCOLL_BF16, splits.data(), 33, nullptr, 0, &count,
                       nullptr, nullptr, nullptr) == VCOLL_OK);
    std::vector<vcoll_msg> msgs(count + 1);
    CHECK(vcoll_ledger(VCOLL_OP_ALL_TO_ALL, VCOLL_RING, p, 0, VCOLL_BF16, splits.data(), 33, msgs.data(), count,
                       &count, nullptr, nullptr, nullptr) == VCOLL_OK);
  }
  // hierarchical and rooted ledgers
  const int shapes[][2] = {{1, 1}, {2, 4}, {4, 2}, {2, 8}, {4, 4}, {3, 5}, {8, 8}, {16, 8}};
  for (const auto& sh : shapes)
    for (int64_t n : {int64_t(0), int64_t(7), int64_t(4096), int64_t(1000003)}) {
      int64_t count = 0;
      int32_t steps = 0;
      CHECK(vcoll_ledger_hierarchical(sh[0], sh[1], n, VCOLL_F32, nullptr, 0, &count, nullptr, nullptr, &steps) ==
            VCOLL_OK);
      std::vector<vcoll_msg> msgs(count + 1);
      CHECK(vcoll_ledger_hierarchical(sh[0], sh[1], n, VCOLL_BF16, msgs.data(), count, &count, nullptr, nullptr,
                                      &steps) == VCOLL_OK);
    }
  for (int p : {1, 2, 3, 8, 13, 72, 128})
    for (int root : {0, p / 2, p - 1})
      for (vcoll_algo algo : {VCOLL_BINARY_TREE, VCOLL_NAIVE, VCOLL_SCATTER_ALLGATHER, VCOLL_PIPELINED_CHAIN})
        for (int64_t blocks : {int64_t(1), int64_t(3), int64_t(64)}) {
          int64_t count = 0;
          const vcoll_status st = vcoll_ledger_rooted(VCOLL_OP_BROADCAST, algo, p, 100003, VCOLL_F32, root, blocks,
                                                      nullptr, 0, &count, nullptr, nullptr, nullptr);
          if (st != VCOLL_OK) continue;
          std::vector<vcoll_msg> msgs(count + 1);
          std::vector<int64_t> sent(p), got(p);
          CHECK(vcoll_ledger_rooted(VCOLL_OP_BROADCAST, algo, p, 100003, VCOLL_F32, root, blocks, msgs.data(), count,
                                    &count, sent.data(), got.data(), nullptr) == VCOLL_OK);
          double t = 0;
          CHECK(vcoll_model_clock(msgs.data(), count, p, p, 2e-6, 450e9, 2e-6, 450e9, &t) == VCOLL_OK && t >= 0);
        }
}

static void model() {
  for (vcoll_algo algo : {VCOLL_RING, VCOLL_RECURSIVE_DOUBLING, VCOLL_RABENSEIFNER, VCOLL_BINARY_TREE})
    for (int p : {1, 2, 5, 8, 16, 72, 128}) {
      double t = -1;
      CHECK(vcoll_model_formula(algo, p, 1e6, 2e-6, 450e9, &t) == VCOLL_OK && t >= 0);
      int32_t steps = 0;
      CHECK(vcoll_model_ledger_time(VCOLL_OP_ALLREDUCE, algo, p, 4096, VCOLL_F32, nullptr, 0, 2e-6, 450e9, &t,
                                    &steps) == VCOLL_OK);
    }
  double blocks = 0, t = 0;
  CHECK(vcoll_model_chain_optimum(8, 1e8, 2e-6, 450e9, &blocks, &t) == VCOLL_OK && blocks >= 1);
}

static void moe(std::mt19937_64& rng) {
  const int p = 8, tokens = 512, topk = 8, epr = 32;
  std::vector<int32_t> ids(size_t(p) * tokens * topk);
  for (int i = 0; i < p; ++i)
    for (int t = 0; t < tokens; ++t) {
      std::vector<int> chosen;
      while (int(chosen.size()) < topk) {
        const int e = int(rng() % (p * epr));
        bool dup = false;
        for (int c : chosen) dup = dup || c == e;
        if (!dup) chosen.push_back(e);
      }
      for (int k = 0; k < topk; ++k) ids[(size_t(i) * tokens + t) * topk + k] = chosen[k];
    }
  std::vector<int64_t> splits(p * p);
  std::vector<int32_t> src(size_t(p) * tokens * topk), dst(size_t(p) * tokens * topk);
  CHECK(vcoll_moe_plan(p, tokens, topk, epr, ids.data(), splits.data(), src.data(), dst.data()) == VCOLL_OK);
  int64_t total = 0;
  for (auto v : splits) total += v;
  CHECK(total == int64_t(p) * tokens * topk);
  std::vector<int32_t> slots(size_t(p) * tokens * topk * 2);
  CHECK(vcoll_moe_slots(p, tokens, topk, splits.data(), dst.data(), slots.data()) == VCOLL_OK);
  std::vector<int64_t> su(p * p);
  std::vector<int32_t> srcu(size_t(p) * tokens * topk), expand(size_t(p) * p * tokens * topk);   // [p][p*tokens*topk]
  std::vector<int64_t> expand_count(p);
  CHECK(vcoll_moe_plan_dedup(p, tokens, topk, epr, ids.data(), su.data(), srcu.data(), expand.data(),
                             expand_count.data()) == VCOLL_OK);
  // token-major forms of the deduplicated plan: send slots and per-rank expansion slots
  std::vector<int32_t> dslots(size_t(p) * tokens * topk * 2);
  CHECK(vcoll_moe_dedup_slots(p, tokens, topk, su.data(), srcu.data(), dslots.data()) == VCOLL_OK);
  const int64_t cap = int64_t(p) * tokens * topk;
  for (int j = 0; j < p; ++j) {
    int64_t unique_rows = 0;
    for (int i = 0; i < p; ++i) unique_rows += su[size_t(i) * p + j];
    std::vector<int32_t> xs(size_t(unique_rows) * topk * 2 + 2);
    CHECK(vcoll_moe_expand_slots(unique_rows, topk, expand.data() + j * cap, expand_count[j], xs.data()) == VCOLL_OK);
    if (unique_rows > 0)                                    // one unique row too few: an entry out of range
      CHECK(vcoll_moe_expand_slots(unique_rows - 1, topk, expand.data() + j * cap, expand_count[j], xs.data()) ==
            VCOLL_ERR_INVALID_ARG || expand_count[j] == 0);
  }
  ids[5] = p * epr;                                         // an expert id out of range is refused
  CHECK(vcoll_moe_plan(p, tokens, topk, epr, ids.data(), splits.data(), src.data(), dst.data()) ==
        VCOLL_ERR_INVALID_ARG);
}

static void launches(std::mt19937_64& rng) {
  void* send[kMaxRanks];
  void* recv[kMaxRanks];
  for (int r = 0; r < kMaxRanks; ++r) {
    send[r] = fake(r);
    recv[r] = fake(r + kMaxRanks);
  }
  const vcoll_algo algos[] = {VCOLL_RING, VCOLL_RECURSIVE_DOUBLING, VCOLL_RABENSEIFNER, VCOLL_BINARY_TREE};
  for (int p : {1, 2, 3, 8, 16, 24, 72, 128})
    for (int64_t n : {int64_t(1), int64_t(1000), int64_t(6553600)})
      for (vcoll_algo algo : algos) {
        CHECK(vcoll_allreduce(algo, p, n, VCOLL_F32, send, recv, nullptr) == VCOLL_OK);
        const vcoll_status rs = vcoll_reduce_scatter(algo, p, n, VCOLL_BF16, send, recv, nullptr);
        CHECK(rs == VCOLL_OK || rs == VCOLL_ERR_UNSUPPORTED);
        const vcoll_status ag = vcoll_all_gather(algo, p, n, VCOLL_F32, send, recv, nullptr);
        CHECK(ag == VCOLL_OK || ag == VCOLL_ERR_UNSUPPORTED);
      }
  for (int p : {1, 4, 72, 128}) {
    CHECK(vcoll_broadcast(p, 12345, VCOLL_F32, p - 1, send[0], recv, nullptr) == VCOLL_OK);
    CHECK(vcoll_reduce(VCOLL_BINARY_TREE, p, 12345, VCOLL_BF16, p / 2, send, recv[0], nullptr) == VCOLL_OK);
    std::vector<int64_t> splits(size_t(p) * p);
    for (auto& v : splits) v = int64_t(rng() % 7);
    CHECK(vcoll_all_to_all(p, 7168, VCOLL_BF16, splits.data(), send, recv, nullptr, nullptr, nullptr, nullptr,
                           nullptr) == VCOLL_OK);
  }
  for (int nodes : {2, 4})
    CHECK(vcoll_allreduce_hierarchical(nodes, 4, 100000, VCOLL_F32, send, recv, nullptr) == VCOLL_OK);
  // the allocation-free stepwise mode: same launches as with a workspace
  for (int p : {2, 8, 72}) {
    int32_t with_ws = 0, without = 0;
    std::vector<float> ws(size_t(p) * 1000);
    CHECK(vcoll_allreduce_stepwise(VCOLL_RABENSEIFNER, p, 1000, VCOLL_BF16, send, recv, ws.data(),
                                   int64_t(ws.size()) * 4, &with_ws, nullptr) == VCOLL_OK);
    CHECK(vcoll_allreduce_stepwise_static(VCOLL_RABENSEIFNER, p, 1000, VCOLL_BF16, send, recv, &without,
                                          nullptr) == VCOLL_OK);
    CHECK(with_ws == without && without > 0);
  }
  // the stepwise broadcast: every algorithm, roots, launch counts from the ledger
  for (int p : {1, 2, 7, 64, 65, 128}) {
    for (vcoll_algo algo : {VCOLL_NAIVE, VCOLL_BINARY_TREE, VCOLL_SCATTER_ALLGATHER, VCOLL_PIPELINED_CHAIN}) {
      int32_t launched = 0;
      const long at = g_launches;
      CHECK(vcoll_broadcast_stepwise(algo, p, 10007, VCOLL_BF16, p / 3, 5, send[p / 3], recv, &launched, nullptr) ==
            VCOLL_OK);
      CHECK(launched == g_launches - at);
    }
  }
  // error paths: nothing is launched
  const long before = g_launches;
  {
    int32_t launched = -1;
    // 8 x 2^21 float32 partial sums = 64 MiB fits; one more element does not
    CHECK(vcoll_allreduce_stepwise_static(VCOLL_RING, 8, (int64_t(1) << 21) + 1, VCOLL_BF16, send, recv, &launched,
                                          nullptr) == VCOLL_ERR_SCRATCH_LIMIT);
    CHECK(launched == 0);
    CHECK(vcoll_allreduce_stepwise_static(VCOLL_RING, 8, int64_t(1) << 48, VCOLL_BF16, send, recv, &launched,
                                          nullptr) == VCOLL_ERR_SCRATCH_LIMIT);
    CHECK(vcoll_allreduce_stepwise_static(VCOLL_RING, 0, 10, VCOLL_BF16, send, recv, &launched, nullptr) ==
          VCOLL_ERR_INVALID_ARG);
  }
  CHECK(vcoll_allreduce(VCOLL_RING, 0, 10, VCOLL_F32, send, recv, nullptr) == VCOLL_ERR_INVALID_ARG);
  CHECK(vcoll_allreduce(VCOLL_RING, 129, 10, VCOLL_F32, send, recv, nullptr) == VCOLL_ERR_INVALID_ARG);
  CHECK(vcoll_allreduce(VCOLL_RING, 4, -1, VCOLL_F32, send, recv, nullptr) == VCOLL_ERR_INVALID_ARG);
  CHECK(vcoll_allreduce(VCOLL_RING, 4, 10, VCOLL_F32, nullptr, recv, nullptr) == VCOLL_ERR_INVALID_ARG);
  CHECK(vcoll_allreduce(VCOLL_RING, 4, int64_t(1) << 50, VCOLL_F32, send, recv, nullptr) == VCOLL_ERR_INVALID_ARG);
  // rank grids whose product wraps around int, and token x topk products
  // beyond int64, are refused before the product is formed (UBSan would flag it)
  {
    int64_t cnt = 0;
    double secs = 0;
    const int grids[3][2] = {{4, (1 << 30) + 1}, {65536, 65536}, {(1 << 30) + 1, 4}};
    for (const auto& g : grids) {
      CHECK(vcoll_allreduce_hierarchical(g[0], g[1], 64, VCOLL_F32, send, recv, nullptr) == VCOLL_ERR_INVALID_ARG);
      CHECK(vcoll_ledger_hierarchical(g[0], g[1], 64, VCOLL_F32, nullptr, 0, &cnt, nullptr, nullptr, nullptr) ==
            VCOLL_ERR_INVALID_ARG);
      CHECK(vcoll_model_ledger_time_nodes(1, VCOLL_RING, g[0], g[1], 64, VCOLL_F32, 1e-6, 1e9, 1e-6, 1e9, &secs,
                                          nullptr) == VCOLL_ERR_INVALID_ARG);
    }
    int32_t ids[8] = {};
    int64_t sp[4] = {};
    int32_t rows[8] = {};
    CHECK(vcoll_moe_plan(2, int64_t(1) << 48, INT32_MAX, 4, ids, sp, rows, rows) == VCOLL_ERR_INVALID_ARG);
    CHECK(vcoll_moe_slots(2, int64_t(1) << 48, INT32_MAX, sp, rows, rows) == VCOLL_ERR_INVALID_ARG);
    CHECK(vcoll_moe_expand_slots(int64_t(1) << 48, INT32_MAX, rows, 1, rows) == VCOLL_ERR_INVALID_ARG);
  }
  CHECK(vcoll_reduce_scatter(VCOLL_RECURSIVE_DOUBLING, 4, 10, VCOLL_F32, send, recv, nullptr) ==
        VCOLL_ERR_UNSUPPORTED);
  CHECK(vcoll_reduce_scatter(VCOLL_RABENSEIFNER, 6, 10, VCOLL_F32, send, recv, nullptr) == VCOLL_ERR_UNSUPPORTED);
  std::vector<int64_t> bad = {1, -1, 0, 2};
  CHECK(vcoll_all_to_all(2, 16, VCOLL_F32, bad.data(), send, recv, nullptr, nullptr, nullptr, nullptr, nullptr) ==
        VCOLL_ERR_INVALID_ARG);
  CHECK(g_launches == before);
}

// Every tree program (push / add stack machine of order_program) equals the
// binary counter over its groups (order_groups), operand for operand: leaves
// are written as their rank, a sum as (older+newer).
static void group_programs() {
  for (int algo : {VCOLL_RECURSIVE_DOUBLING, VCOLL_RABENSEIFNER, VCOLL_BINARY_TREE})
    for (int p = 1; p <= kMaxRanks; ++p) {
      const vcoll::OrderProgram prog = vcoll::order_program(algo, p);
      std::vector<std::string> st;
      auto merge = [&]() {
        const std::string b = st.back();
        st.pop_back();
        st.back() = "(" + st.back() + "+" + b + ")";
      };
      for (int k = 0; k < p; ++k) {
        st.push_back(std::to_string(prog.rank[k]));
        for (int m = 0; m < prog.merges[k]; ++m) merge();
      }
      for (int m = 0; m < prog.final_merges; ++m) merge();
      CHECK(st.size() == 1);
      int first[kMaxRanks + 1] = {};
      const int groups = vcoll::order_groups(algo, p, first);
      CHECK(groups >= 1 && groups <= kMaxRanks && first[0] == 0 && first[groups] == p);
      std::string lvl[8];
      for (int q = 0; q < groups; ++q) {
        const int k = first[q], n = first[q + 1] - k;
        CHECK(n == 1 || n == 2);
        std::string v = std::to_string(prog.rank[k]);
        if (n == 2) v = "(" + v + "+" + std::to_string(prog.rank[k + 1]) + ")";
        const int closes = vcoll::ctz_int(q + 1);
        for (int l = 0; l < closes; ++l) v = "(" + lvl[l] + "+" + v + ")";
        lvl[closes] = v;
      }
      std::string total;
      for (int l = 0; l < 8; ++l)
        if ((groups >> l) & 1) total = total.empty() ? lvl[l] : "(" + lvl[l] + "+" + total + ")";
      if (total != st[0]) {
        std::fprintf(stderr, "algo %d p %d: counter %s, program %s\n", algo, p, total.c_str(), st[0].c_str());
        std::abort();
      }
    }
}

int main() {
  std::mt19937_64 rng(7);
  group_programs();
  ledgers(rng);
  model();
  moe(rng);
  launches(rng);
  CHECK(g_launches > 0);
  {
    // the DDP bucket (p = 8 x 6,553,600 float32) takes the two-phase ring kernel
    void* send[8];
    void* recv[8];
    for (int r = 0; r < 8; ++r) {
      send[r] = reinterpret_cast<void*>(uintptr_t(0x100000) * (r + 1));
      recv[r] = reinterpret_cast<void*>(uintptr_t(0x100000) * (r + 9));
    }
    const long before = g_burst;
    CHECK(vcoll_allreduce(VCOLL_RING, 8, 6553600, VCOLL_F32, send, recv, nullptr) == VCOLL_OK);
    CHECK(g_burst == before + 1);
    CHECK(vcoll_allreduce(VCOLL_RABENSEIFNER, 8, 6553600, VCOLL_F32, send, recv, nullptr) == VCOLL_OK);
    CHECK(vcoll_allreduce(VCOLL_RING, 8, 1 << 20, VCOLL_F32, send, recv, nullptr) == VCOLL_OK);
    CHECK(vcoll_allreduce(VCOLL_RING, 8, 2 * 6553600, VCOLL_F32, send, recv, nullptr) == VCOLL_OK);
    CHECK(g_burst == before + 1);
    // chunks that are not whole vectors (n mod p*VE != 0) take it too
    CHECK(vcoll_allreduce(VCOLL_RING, 8, 6553600 + 5, VCOLL_F32, send, recv, nullptr) == VCOLL_OK);
    CHECK(g_burst == before + 2);
    CHECK(vcoll_allreduce(VCOLL_RING, 8, 6553600 - 3, VCOLL_BF16, send, recv, nullptr) == VCOLL_OK);
    CHECK(g_burst == before + 3);
  }
  {
    // p = 72 x 16 MiB float32: 58,254 or 58,255 elements per chunk
    void* send[72];
    void* recv[72];
    for (int r = 0; r < 72; ++r) {
      send[r] = reinterpret_cast<void*>(uintptr_t(0x100000) * (r + 1));
      recv[r] = reinterpret_cast<void*>(uintptr_t(0x100000) * (r + 73));
    }
    const long before = g_burst;
    CHECK(vcoll_allreduce(VCOLL_RING, 72, 1 << 22, VCOLL_F32, send, recv, nullptr) == VCOLL_OK);
    CHECK(g_burst == before + 1);
  }
  std::printf("OK %ld launches recorded\n", g_launches);
  return 0;
}
