// The fused reduce kernels of libvcoll for gfx950: all-reduce, reduce-scatter
// and reduce to a root, each evaluating its algorithm's summation order in
// registers in one streaming pass.
//
// Summation orders come from "Networks and Collective Communication" (cs349e
// prerequisite lecture 5), sections 5.1 (ring) and 5.2 (recursive doubling,
// Rabenseifner, binomial tree); order.h writes each as a push / add program.
#include "device.h"
#include "reduce.h"

namespace vcoll {
namespace {

using namespace dev;

// ----------------------------------------------------------------------------
// order programs unfolded at compile time (p fixed)

template <int ALGO, int P>
struct Prog {
  static constexpr OrderProgram value = order_program(ALGO, P);
  static constexpr int depth = value.max_depth > 0 ? value.max_depth : 1;
};

// Replace the top two of DEPTH live stack entries by their sum, M times.
template <int DEPTH, int M, int SD, int N>
__device__ __forceinline__ void merge_top(float (&st)[SD][N]) {
  if constexpr (M > 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) st[DEPTH - 2][i] = st[DEPTH - 2][i] + st[DEPTH - 1][i];
    merge_top<DEPTH - 1, M - 1>(st);
  }
}

// Push leaf K (widened by `leaf`) and apply its merges; recurse to K + 1.
template <int ALGO, int P, int K, int DEPTH, int SD, int N, class Leaf>
__device__ __forceinline__ void run_program(float (&st)[SD][N], const Leaf& leaf) {
  if constexpr (K < P) {
    leaf(std::integral_constant<int, K>{}, st[DEPTH]);
    constexpr int M = Prog<ALGO, P>::value.merges[K];
    merge_top<DEPTH + 1, M>(st);
    run_program<ALGO, P, K + 1, DEPTH + 1 - M>(st, leaf);
  } else {
    merge_top<DEPTH, Prog<ALGO, P>::value.final_merges>(st);
  }
}

// Stack entries alive before leaf K is pushed.
template <int ALGO, int P>
constexpr int depth_before(int K) {
  int d = 0;
  for (int j = 0; j < K; ++j) d += 1 - Prog<ALGO, P>::value.merges[j];
  return d;
}

// Push leaf K (already widened) and apply its merges; after the last leaf,
// the final collapse.
template <int ALGO, int P, int K, int SD, int N>
__device__ __forceinline__ void push_leaf(float (&st)[SD][N], const float (&v)[N]) {
  constexpr int D = depth_before<ALGO, P>(K);
  constexpr int M = Prog<ALGO, P>::value.merges[K];
#pragma unroll
  for (int i = 0; i < N; ++i) st[D][i] = v[i];
  merge_top<D + 1, M>(st);
  if constexpr (K == P - 1) merge_top<D + 1 - M, Prog<ALGO, P>::value.final_merges>(st);
}

// The program leaf that stands for rank r (p compiled in).
template <int ALGO, int P>
constexpr int leaf_of_rank(int r) {
  for (int j = 0; j < P; ++j)
    if (Prog<ALGO, P>::value.rank[j] == r) return j;
  return r;
}

// Ranks whose loads a wave keeps in flight ahead of the one it is adding.
// Large grids (which also pace their stores) issue all p ranks up front;
// small, latency-bound grids run a pipeline of a few ranks, which measured
// 10% faster at 1 MiB per rank. Build-time override of the small-grid
// depth: -DVCOLL_LAG=<n>.
#ifndef VCOLL_LAG
#define VCOLL_LAG 4
#endif
template <int P, bool LARGE>
constexpr int load_lag() { return LARGE ? P : (VCOLL_LAG < P ? VCOLL_LAG : P); }

// Row of leaf pointers of chunk c (p compiled in): the ring's order rotates
// with the chunk, the trees' order is the same for every chunk (row 0).
template <int ALGO>
__device__ __forceinline__ const void* const* leaf_row(const ReduceArgs& a, int c) {
  return &a.leaf[(ALGO == VCOLL_RING ? c : 0) * kFixedMax];
}

// ----------------------------------------------------------------------------
// tree orders with p known only at run time: the binary counter of
// order_groups. Group q closes ctz(q + 1) subtrees; the groups run in
// batches whose position in the batch is a compile-time index (see
// counter_push), so every close adds fixed registers (no stack to shift, no
// per-leaf merge count to read); the host lays out each group's leaf
// buffers. Against a shift-register stack driven by the program's merge
// counts, on MI355X: p = 72 tree all-reduces of 1 MiB per rank 58 -> 41-49
// us, 4 MiB 130 -> 119-123 us, 64 MiB within 1 %.

constexpr int kLevels = 8;         // open subtrees of a counter over up to 128 groups

// Add group Q's value v (destroyed) to the counter.
template <int Q, int N>
__device__ __forceinline__ void counter_add(float (&lvl)[kLevels][N], float (&v)[N]) {
  constexpr int closes = ctz_int(Q + 1);
  static_assert(closes < kLevels, "at most 128 groups");
#pragma unroll
  for (int l = 0; l < closes; ++l)
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = lvl[l][i] + v[i];
#pragma unroll
  for (int i = 0; i < N; ++i) lvl[closes][i] = v[i];
}

// The sum over all `groups` groups: the open subtrees (one per set bit of
// the count) from the smallest up, each older one added to the running sum.
template <int N>
__device__ __forceinline__ void counter_total(const float (&lvl)[kLevels][N], int groups, float (&out)[N]) {
  bool first = true;
#pragma unroll
  for (int l = 0; l < kLevels; ++l) {
    if ((groups >> l) & 1) {
#pragma unroll
      for (int i = 0; i < N; ++i) out[i] = first ? lvl[l][i] : lvl[l][i] + out[i];
      first = false;
    }
  }
}

// Groups of a run-time tree program whose loads a thread keeps in flight
// together (a folded pair loads two leaves) on the per-thread paths. 8
// against 4 on MI355X: p = 24 x 256 KiB per rank 9.9 against 11.0 us, p = 72
// x 1 MiB 41 against 45 us (the latency-bound sizes, where fewer batches
// mean fewer waits); 4 was 3 % faster for the binomial tree at p = 24 x 16
// MiB. Build-time override: -DVCOLL_TREE_BATCH=<power of two>.
#ifndef VCOLL_TREE_BATCH
#define VCOLL_TREE_BATCH 8
#endif
constexpr int kTreeBatch = VCOLL_TREE_BATCH;

// Add group q0 + b of a batch of B groups (B a power of two, q0 a multiple
// of B) to the counter. Group q0 + b closes ctz(b + 1) subtrees for b < B -
// 1, a compile-time count, and the batch's last group log2(B) + ctz(q0 / B +
// 1): its levels past log2(B) are predicated on that count, so every
// register index stays fixed while the batches run in a loop. (Unrolling
// all 128 groups instead gives the argument block so many uses that the
// compiler copies it to scratch memory.)
template <int B, int b, int N>
__device__ __forceinline__ void counter_push(float (&lvl)[kLevels][N], float (&v)[N], int q0) {
  static_assert(B >= 2 && (B & (B - 1)) == 0 && kMaxRanks % B == 0 && b < B, "batches of a power of two");
  if constexpr (b < B - 1) {
    counter_add<b>(lvl, v);
  } else {
    constexpr int LB = ctz_int(B);
    // selects, not branches: a conditional store per level is merged by the
    // compiler into one store through a chosen pointer, which moves the
    // counter to scratch memory
    const int extra = __builtin_ctz(static_cast<unsigned>(q0 / B + 1));
#pragma unroll
    for (int l = 0; l < LB; ++l)
#pragma unroll
      for (int i = 0; i < N; ++i) v[i] = lvl[l][i] + v[i];
#pragma unroll
    for (int l = LB; l < kLevels - 1; ++l) {
      const bool close = l - LB < extra;
#pragma unroll
      for (int i = 0; i < N; ++i) v[i] = close ? lvl[l][i] + v[i] : v[i];
    }
#pragma unroll
    for (int l = LB; l < kLevels; ++l) {
      const bool keep = l - LB == extra;
#pragma unroll
      for (int i = 0; i < N; ++i) lvl[l][i] = keep ? v[i] : lvl[l][i];
    }
  }
}

// Run a tree program (groups in a.leaf, see ReduceArgs) B groups at a time:
// issue(s0, s1, pair, b) starts the loads of group q0 + b's first leaf
// (buffer s0) and, for a folded pair, its second (s1) into slot b of the
// caller's registers, every load of a batch before the first value is
// taken; take(b, pair, v) widens slot b into v, the pair's two leaves added.
// Every buffer is found by the group index alone, so the loads of a batch
// wait on nothing.
template <int ALGO, int B, int N, class Issue, class Take>
__device__ __forceinline__ void run_groups(const ReduceArgs& a, float (&out)[N], const Issue& issue,
                                           const Take& take) {
  constexpr bool kPairs = ALGO != VCOLL_BINARY_TREE;             // the binomial tree folds nothing
  const int groups = a.groups;
  float lvl[kLevels][N];
#pragma unroll 1
  for (int q0 = 0; q0 < groups; q0 += B) {
    bool pair[B];
    static_for<0, B>([&](auto bb) {
      constexpr int b = decltype(bb)::value;
      const int q = q0 + b;
      if (q < groups) {
        const void* s1 = kPairs ? a.leaf[kMaxRanks + q] : nullptr;
        pair[b] = s1 != nullptr;
        issue(a.leaf[q], s1, pair[b], bb);
      }
    });
    static_for<0, B>([&](auto bb) {
      constexpr int b = decltype(bb)::value;
      if (q0 + b < groups) {
        float v[N];
        take(bb, pair[b], v);
        counter_push<B, b>(lvl, v, q0);
      }
    });
  }
  counter_total(lvl, groups, out);
}

// ----------------------------------------------------------------------------
// one element (chunk heads and tails, unaligned buffers)

template <int D, int ALGO, int P, bool RS>
__device__ __forceinline__ void reduce_one(const ReduceArgs& a, int c, int p, int rot, int64_t e,
                                           int64_t off) {
  using S = Storage<D>;
  using E = typename S::elem;
  float result;
  if constexpr (P > 0) {
    const void* const* L = leaf_row<ALGO>(a, c);
    E raw[P];
    static_for<0, P>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      raw[k] = static_cast<const E*>(L[k])[e];
    });
    float st[Prog<ALGO, P>::depth][1];
    run_program<ALGO, P, 0, 0>(st, [&](auto kc, float(&d)[1]) {
      d[0] = S::widen1(raw[decltype(kc)::value]);
    });
    result = st[0][0];
  } else {
    // loads go out kOneBatch ranks (groups) at a time, so a long program (p
    // up to 128) waits for memory p / kOneBatch times rather than p times
    constexpr int kOneBatch = 16;
    if constexpr (ALGO == VCOLL_RING) {
      result = 0.0f;
      for (int k0 = 0; k0 < p; k0 += kOneBatch) {
        E raw[kOneBatch];
#pragma unroll
        for (int b = 0; b < kOneBatch; ++b)
          if (k0 + b < p) raw[b] = static_cast<const E*>(a.leaf[(rot + k0 + b) % p])[e];
#pragma unroll
        for (int b = 0; b < kOneBatch; ++b)
          if (k0 + b < p) result = k0 + b == 0 ? S::widen1(raw[b]) : result + S::widen1(raw[b]);
      }
    } else {
      E raw[kOneBatch], raw2[kOneBatch];
      float res[1];
      run_groups<ALGO, kOneBatch, 1>(
          a, res,
          [&](const void* s0, const void* s1, bool pair, auto bc) {
            constexpr int b = decltype(bc)::value;
            raw[b] = static_cast<const E*>(s0)[e];
            if (pair) raw2[b] = static_cast<const E*>(s1)[e];
          },
          [&](auto bc, bool pair, float(&v)[1]) {
            constexpr int b = decltype(bc)::value;
            v[0] = S::widen1(raw[b]);
            if (pair) v[0] = v[0] + S::widen1(raw2[b]);
          });
      result = res[0];
    }
  }
  const E out = S::narrow1(result);
  if constexpr (RS) {
    static_cast<E*>(a.dst[c])[e - off] = out;
  } else {
    for (int r = 0; r < p; ++r) static_cast<E*>(a.dst[r])[e] = out;
  }
}

// kElemBatch elements e0 + u*stride at once (those below `limit`): the loads
// of all of them go out together, so a thread waits on memory once per batch
// of ranks rather than once per element (the path of buffers that are not
// 16-byte aligned, where every element is reduced this way).
constexpr int kElemBatch = 4;

template <int D, int ALGO, int P, bool RS>
__device__ __forceinline__ void reduce_elems(const ReduceArgs& a, int c, int p, int rot, int64_t e0,
                                             int64_t stride, int64_t limit, int64_t off) {
  using S = Storage<D>;
  using E = typename S::elem;
  constexpr int U = kElemBatch;
  int64_t e[U];
  bool ok[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    e[u] = e0 + u * stride;
    ok[u] = e[u] < limit;
  }
  float res[U];
  if constexpr (P > 0) {
    const void* const* L = leaf_row<ALGO>(a, c);
    E raw[P][U];
    static_for<0, P>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
#pragma unroll
      for (int u = 0; u < U; ++u) raw[k][u] = ok[u] ? static_cast<const E*>(L[k])[e[u]] : E(0);
    });
    float st[Prog<ALGO, P>::depth][U];
    run_program<ALGO, P, 0, 0>(st, [&](auto kc, float(&d)[U]) {
#pragma unroll
      for (int u = 0; u < U; ++u) d[u] = S::widen1(raw[decltype(kc)::value][u]);
    });
#pragma unroll
    for (int u = 0; u < U; ++u) res[u] = st[0][u];
  } else {
    // ranks whose loads are in flight together: 8 keeps the kernel's register
    // count (set by its vector path) where it was; 16 took the run-time
    // trees from 5 to 4 waves per SIMD and p = 72 tree all-reduces of 4 and
    // 16 MiB per rank 2-9 % slower, for 6 % on unaligned buffers
    constexpr int B = 8;
    if constexpr (ALGO == VCOLL_RING) {
#pragma unroll
      for (int u = 0; u < U; ++u) res[u] = 0.0f;
      for (int k0 = 0; k0 < p; k0 += B) {
        E raw[B][U];
#pragma unroll
        for (int b = 0; b < B; ++b)
          if (k0 + b < p) {
            const void* src = a.leaf[(rot + k0 + b) % p];
#pragma unroll
            for (int u = 0; u < U; ++u) raw[b][u] = ok[u] ? static_cast<const E*>(src)[e[u]] : E(0);
          }
#pragma unroll
        for (int b = 0; b < B; ++b)
          if (k0 + b < p) {
#pragma unroll
            for (int u = 0; u < U; ++u) res[u] = k0 + b == 0 ? S::widen1(raw[b][u]) : res[u] + S::widen1(raw[b][u]);
          }
      }
    } else {
      E raw[kTreeBatch][U], raw2[kTreeBatch][U];
      run_groups<ALGO, kTreeBatch, U>(
          a, res,
          [&](const void* s0, const void* s1, bool pair, auto bc) {
            constexpr int b = decltype(bc)::value;
#pragma unroll
            for (int u = 0; u < U; ++u) raw[b][u] = ok[u] ? static_cast<const E*>(s0)[e[u]] : E(0);
            if (pair) {
#pragma unroll
              for (int u = 0; u < U; ++u) raw2[b][u] = ok[u] ? static_cast<const E*>(s1)[e[u]] : E(0);
            }
          },
          [&](auto bc, bool pair, float(&v)[U]) {
            constexpr int b = decltype(bc)::value;
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = S::widen1(raw[b][u]);
            if (pair) {
#pragma unroll
              for (int u = 0; u < U; ++u) v[u] = v[u] + S::widen1(raw2[b][u]);
            }
          });
    }
  }
  E out[U];
#pragma unroll
  for (int u = 0; u < U; ++u) out[u] = S::narrow1(res[u]);
  if constexpr (RS) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (ok[u]) static_cast<E*>(a.dst[c])[e[u] - off] = out[u];
  } else {
    for (int r = 0; r < p; ++r)
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (ok[u]) static_cast<E*>(a.dst[r])[e[u]] = out[u];
  }
}

// ----------------------------------------------------------------------------
// V 16-byte vectors per thread, fixed p: all p*V loads are issued before the
// first add, the order program runs in registers, then p*V (or V) stores.

template <int D, int ALGO, int P, int V, bool RS, bool LARGE, bool FULL>
__device__ __forceinline__ void reduce_vectors_fixed(const ReduceArgs& a, int c,
                                                     const int64_t (&boff)[V],
                                                     const bool (&valid)[V], int64_t out_shift) {
  using S = Storage<D>;
  constexpr int VE = S::kVE;
  constexpr int LAG = load_lag<P, LARGE>();
  const void* const* L = leaf_row<ALGO>(a, c);
  u32x4 raw[P][V];
  float st[Prog<ALGO, P>::depth][V * VE];

  // software pipeline in summation order: the loads of leaf k go out, then
  // leaf k - LAG (whose loads went out LAG steps earlier) is added
  static_for<0, P + LAG>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    if constexpr (k < P) {
      // the leaf whose loads go out at step k: the program's k-th, or, when
      // every load goes out before the first add, the one of the k-th rank
      // (Rabenseifner's program takes the ranks bit-reversed; issued in that
      // order its p = 16 x 4 MiB all-reduce took 27-28 us against 23.5 for
      // the other algorithms on MI355X, in rank order 23.6-24.0)
      constexpr int kl = LAG == P ? leaf_of_rank<ALGO, P>(k) : k;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        if constexpr (FULL) {
          raw[kl][j] = ld16(L[kl], boff[j]);
        } else {
          raw[kl][j] = valid[j] ? ld16(L[kl], boff[j]) : u32x4{0, 0, 0, 0};
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (k >= LAG) {
      constexpr int q = k - LAG;
      float v[V * VE];
#pragma unroll
      for (int j = 0; j < V; ++j) S::widen(raw[q][j], &v[j * VE]);
      push_leaf<ALGO, P, q>(st, v);
    }
    __builtin_amdgcn_sched_barrier(0);
  });
  u32x4 out[V];
#pragma unroll
  for (int j = 0; j < V; ++j) out[j] = S::narrow(&st[0][j * VE]);
  if constexpr (RS) {
#pragma unroll
    for (int j = 0; j < V; ++j)
      if (FULL || valid[j]) st16(a.dst[c], boff[j] - out_shift, out[j]);
  } else {
    static_for<0, P>([&](auto rc) {
      void* dst = a.dst[decltype(rc)::value];
#pragma unroll
      for (int j = 0; j < V; ++j)
        if (FULL || valid[j]) st16(dst, boff[j], out[j]);
      if constexpr (LARGE) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_sleep(VCOLL_STORE_SLEEP);
        __builtin_amdgcn_sched_barrier(0);
      }
    });
  }
}

// Same for a p known only at run time (one vector per thread; loads go out
// eight ranks at a time).
template <int D, int ALGO, bool RS>
__device__ __forceinline__ void reduce_vector_runtime(const ReduceArgs& a, int c, int p, int rot,
                                                      int64_t boff, bool valid, int64_t out_shift) {
  using S = Storage<D>;
  constexpr int VE = S::kVE;
  constexpr int B = 8;               // ranks whose loads are in flight together (ring)
  float acc[VE];
  if constexpr (ALGO == VCOLL_RING) {
    for (int k0 = 0; k0 < p; k0 += B) {
      u32x4 raw[B];
#pragma unroll
      for (int b = 0; b < B; ++b)
        if (k0 + b < p) raw[b] = valid ? ld16(a.leaf[(rot + k0 + b) % p], boff) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int b = 0; b < B; ++b) {
        if (k0 + b < p) {
          float v[VE];
          S::widen(raw[b], v);
#pragma unroll
          for (int i = 0; i < VE; ++i) acc[i] = k0 + b == 0 ? v[i] : acc[i] + v[i];
        }
      }
    }
  } else {
    u32x4 raw[kTreeBatch], raw2[kTreeBatch];
    run_groups<ALGO, kTreeBatch, VE>(
        a, acc,
        [&](const void* s0, const void* s1, bool pair, auto bc) {
          constexpr int b = decltype(bc)::value;
          raw[b] = valid ? ld16(s0, boff) : u32x4{0, 0, 0, 0};
          if (pair) raw2[b] = valid ? ld16(s1, boff) : u32x4{0, 0, 0, 0};
        },
        [&](auto bc, bool pair, float(&v)[VE]) {
          constexpr int b = decltype(bc)::value;
          S::widen(raw[b], v);
          if (pair) {
            float w[VE];
            S::widen(raw2[b], w);
#pragma unroll
            for (int i = 0; i < VE; ++i) v[i] = v[i] + w[i];
          }
        });
  }
  if (!valid) return;
  const u32x4 out = S::narrow(acc);
  if constexpr (RS) {
    st16(a.dst[c], boff - out_shift, out);
  } else {
    for (int r = 0; r < p; ++r) {
      st16(a.dst[r], boff, out);
      if (a.pace) __builtin_amdgcn_s_sleep(VCOLL_STORE_SLEEP);
    }
  }
}

// ----------------------------------------------------------------------------
// the reduce kernel: workgroup (x, y) handles tile x of chunk y

template <int D, int ALGO, int P, int V, bool RS, bool LARGE, int BS>
__global__ __launch_bounds__(BS) void reduce_kernel(const ReduceArgs a) {
  using S = Storage<D>;
  constexpr int VE = S::kVE;
  constexpr int ES = 16 / VE;
  const int c = blockIdx.y;
  const int p = P > 0 ? P : a.p;
  const int64_t off = c * a.q + (c < a.r ? c : a.r);
  const int64_t cnt = a.q + (c < a.r ? 1 : 0);
  const int rot = (ALGO == VCOLL_RING) ? (c + 1) % p : 0;
  const int tid = threadIdx.x;
  // a reduce-scatter writes element e of chunk c to recv[c][e - off]: both
  // sides must be vector aligned, so the chunk start must be (the ring with a
  // run-time p has its own kernel for unaligned chunk starts)
  const bool vec = a.vec != 0 && (!RS || (off % VE) == 0);

  if (vec) {
    // the vector tiles of an all-reduce start on a 256-byte boundary of every
    // buffer when the buffers allow it (whole cache lines per wave: chunk
    // starts that are only 16-byte aligned cost p = 72 5 % extra HBM
    // traffic), those of a reduce-scatter on a 128-byte line of every input
    // (p = 72 x 16 MiB per rank, f32, 16-byte aligned chunks: 222.7 -> 200.4
    // us on MI355X); the elements before it and the ragged end take the
    // element path
    const int64_t align = RS ? a.src_align : a.align;
    const int64_t mis = ((RS ? a.src_phase : a.phase) + off * ES) % align;
    const int64_t head_e = mis ? (align - mis) / ES : 0;
    const int64_t head = head_e < cnt ? head_e : cnt;
    const int64_t nvec = (cnt - head) / VE;
    const int64_t e_base = off + head;
    const int64_t v0 = static_cast<int64_t>(blockIdx.x) * (V * BS) + tid;
    if (static_cast<int64_t>(blockIdx.x) * (V * BS) < nvec) {
      if constexpr (P > 0) {
        int64_t boff[V];
        bool valid[V];
#pragma unroll
        for (int j = 0; j < V; ++j) {
          const int64_t v = v0 + j * BS;
          valid[j] = v < nvec;
          boff[j] = (e_base + v * VE) * ES;
        }
        if ((static_cast<int64_t>(blockIdx.x) + 1) * (V * BS) <= nvec) {
          reduce_vectors_fixed<D, ALGO, P, V, RS, LARGE, true>(a, c, boff, valid, off * ES);
        } else {
          reduce_vectors_fixed<D, ALGO, P, V, RS, LARGE, false>(a, c, boff, valid, off * ES);
        }
      } else {
#pragma unroll 1
        for (int j = 0; j < V; ++j) {
          const int64_t v = v0 + j * BS;
          reduce_vector_runtime<D, ALGO, RS>(a, c, p, rot, (e_base + v * VE) * ES, v < nvec,
                                             off * ES);
        }
      }
    }
    if (blockIdx.x == 0) {
      const int64_t tail = cnt - head - nvec * VE;
      for (int64_t i = tid; i < head + tail; i += BS)
        reduce_one<D, ALGO, P, RS>(a, c, p, rot, i < head ? off + i : e_base + nvec * VE + (i - head), off);
    }
  } else {
    static_assert((V * VE) % kElemBatch == 0, "whole element batches per thread");
    const int64_t e0 = static_cast<int64_t>(blockIdx.x) * (V * BS * VE);
#pragma unroll 1
    for (int j = 0; j < V * VE; j += kElemBatch)
      reduce_elems<D, ALGO, P, RS>(a, c, p, rot, off + e0 + j * BS + tid, BS, off + cnt, off);
  }
}

// ----------------------------------------------------------------------------
// ring reduce-scatter with a run-time p and chunk starts that are not 16-byte
// aligned. The output recv[c] is aligned, the inputs are not: element j of
// chunk c is input element off + j. Each lane sums the ring chain over one
// ALIGNED input vector; output vector j then takes the last VE - shift sums
// of input vector j and the first `shift` sums of input vector j + 1, which
// the next lane holds (one wave shuffle per output vector, not per rank).
// Two wave shapes:
//  * LINES = false: a wave loads 64 consecutive input vectors and stores the
//    63 outputs whose both vectors it holds (waves overlap by one vector);
//  * LINES = true: a wave's 64 input vectors start on a 128-byte line of
//    every input (when the inputs share an address phase mod 128), so its
//    loads are whole lines, and it stores all 64 outputs that start in
//    them; the vector after the wave, which the last output needs, is
//    summed by the wave's last lane as well (one extra 16-byte load per
//    rank, from a line the next wave loads).
// The chunk's last output vectors, whose neighbour would reach past the
// chunk, and its ragged end take the element path. Measured on MI355X with
// f32: p = 72 x 64 MiB per rank ran 855 us with 63-output waves (whose loads
// straddle lines: 1.09x the algorithmic bytes read) and 783 us with
// line-aligned ones (6.25 TB/s, above the aligned p = 64 case's 6.17), p =
// 24 x 64 MiB 294 -> 269 us; but the extra registers of the line-aligned shape
// (84 instead of 44, 5 waves per SIMD instead of 8) cost 2-4 % on grids of
// one or two workgroup generations (p = 72 at 4 and 16 MiB) and 5 % for
// bf16, so the host takes it for f32 grids of many generations only.
// The element path for every element of such chunks ran at 5.5 TB/s.

template <int D, bool LINES>
__global__ __launch_bounds__(kBlock) void reduce_scatter_shifted_kernel(const ReduceArgs a) {
  using S = Storage<D>;
  constexpr int VE = S::kVE;
  constexpr int B = 8;                                           // ranks whose loads are in flight together
  constexpr int kWaveOut = LINES ? 64 : 63;                      // output vectors per wave
  const int c = blockIdx.y;
  const int p = a.p;
  const int64_t off = c * a.q + (c < a.r ? c : a.r);
  const int64_t cnt = a.q + (c < a.r ? 1 : 0);
  const int rot = (c + 1) % p;
  const int shift = static_cast<int>(off % VE);
  const int64_t nvec = (cnt + shift) / VE >= 1 ? (cnt + shift) / VE - 1 : 0;   // output vectors
  // input vector v0 holds element off; the waves start at `base`, d vectors
  // before it (the line start at or before it, or v0 itself)
  const int64_t v0 = off / VE;
  int64_t base = v0;
  if (LINES && a.src_align > 16) {
    base -= ((a.src_phase + v0 * 16) % a.src_align) / 16;
    if (base < 0) base = 0;
  }
  const int64_t d = v0 - base;
  const int lane = threadIdx.x & 63;
  const int64_t t = (static_cast<int64_t>(blockIdx.x) * (kBlock / 64) + (threadIdx.x >> 6)) * kWaveOut + lane;
  const int64_t last = d + nvec;                                 // input vector last is only a neighbour
  const bool own = t >= d && t <= last;
  const int64_t boff = (base + t) * 16;
  float acc[VE];
  [[maybe_unused]] float acc2[VE];
  [[maybe_unused]] const bool extra = LINES && lane == 63 && t + 1 >= d && t + 1 <= last;
  for (int k0 = 0; k0 < p; k0 += B) {
    u32x4 raw[B];
    [[maybe_unused]] u32x4 raw2[B];
#pragma unroll
    for (int b = 0; b < B; ++b)
      if (k0 + b < p) {
        const void* src = a.leaf[(rot + k0 + b) % p];
        raw[b] = own ? ld16(src, boff) : u32x4{0, 0, 0, 0};
        // a cached load: its line is the next wave's first (1.3 % faster than streamed)
        if constexpr (LINES)
          raw2[b] = extra ? *reinterpret_cast<const u32x4*>(static_cast<const char*>(src) + boff + 16) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if (k0 + b < p) {
        float v[VE];
        S::widen(raw[b], v);
#pragma unroll
        for (int i = 0; i < VE; ++i) acc[i] = k0 + b == 0 ? v[i] : acc[i] + v[i];
        if constexpr (LINES) {
          S::widen(raw2[b], v);
#pragma unroll
          for (int i = 0; i < VE; ++i) acc2[i] = k0 + b == 0 ? v[i] : acc2[i] + v[i];
        }
      }
    }
  }
  float nb[VE];
#pragma unroll
  for (int i = 0; i < VE; ++i) {
    nb[i] = __shfl_down(acc[i], 1);
    if constexpr (LINES) {
      if (lane == 63) nb[i] = acc2[i];
    }
  }
  const int64_t j = t - d;                                       // output vector of this lane
  if (lane < kWaveOut && j >= 0 && j < nvec) {
    float o[VE];
#pragma unroll
    for (int i = 0; i < VE; ++i) {
      float x = acc[i];
#pragma unroll
      for (int k = 1; k < VE; ++k)
        if (shift == k) x = i + k < VE ? acc[i + k] : nb[i + k - VE];
      o[i] = x;
    }
    st16(a.dst[c], j * 16, S::narrow(o));
  }
  if (blockIdx.x == 0) {
    const int64_t tail = cnt - nvec * VE;                        // < 2 * VE
    if (threadIdx.x < tail) reduce_one<D, VCOLL_RING, 0, true>(a, c, p, rot, off + nvec * VE + threadIdx.x, off);
  }
}

// Waves (of the line-aligned shape) from which the unaligned reduce-scatter
// takes it: about four generations of 8 waves per SIMD on 256 compute units.
constexpr int64_t kShiftLinesMinWaves = 32768;

// ----------------------------------------------------------------------------
// small chunks with a run-time p: a workgroup stages a [slots][kSmallTile]
// tile of its chunk in LDS with every load of the tile in flight at once,
// sums each element out of LDS, and fans the results out. A slot is a rank
// (ring) or a group of the tree program (a folded pair added on the way in).
// Wave w moves slots w, w + 4, ...: each lane fetches two entries of every
// pointer table with one vector load (one memory round trip for all of
// them, where scalar loads of a workgroup alone on its compute unit miss the
// scalar cache a few pointers at a time), and each slot's address is read
// from the lane that holds it, uniform in the wave. The element accesses are
// buffer instructions whose size (the tile's elements, or nothing for a
// slot past the last) masks the rest, so no load or store waits on another
// and no slot needs a branch. (Per-lane buffer lookups made every access of
// a wave wait for the ones before it; a branch per slot cost p = 72 at 1 KiB
// per rank 4 us, scalar pointer loads 4 us at p = 24.) Against per-lane
// lookups and a shift-register stack for the trees, on MI355X: p = 24 at 1
// KiB per rank ring 4.4 -> 3.7 us, trees 6.4 -> 3.9-4.0; p = 72 at 10 KiB
// ring 8.8 -> 5.7, trees 14.3 -> 5.4-6.5, at 256 KiB ring 22.7 -> 14.5, trees
// 31.9 -> 14.6-16.1. Then 24 slots per wave for p <= 96 and an LDS tile
// sized to the slots moved: p = 72 at 1 KiB ring 5.8 -> 5.1 us, trees 5.4-6.6
// -> 5.0-5.7, at 256 KiB ring 14.5 -> 11.5, trees 14.6-16.2 -> 11.9-13.2; p =
// 96 12-23 % faster.

constexpr int kSmallTile = 64;                                   // elements of a chunk per workgroup

template <class E>
__device__ __forceinline__ E buf_ld1(__amdgpu_buffer_rsrc_t r, int voff) {
  if constexpr (sizeof(E) == 4) return __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, kPolicyCached);
  else return __builtin_amdgcn_raw_buffer_load_b16(r, voff, 0, kPolicyCached);
}

template <class E>
__device__ __forceinline__ void buf_st1(E v, __amdgpu_buffer_rsrc_t r, int voff) {
  if constexpr (sizeof(E) == 4) __builtin_amdgcn_raw_buffer_store_b32(v, r, voff, 0, kPolicyCached);
  else __builtin_amdgcn_raw_buffer_store_b16(v, r, voff, 0, kPolicyCached);
}

// Entry `i` (uniform, < 64) of a table whose entry l each lane l holds.
__device__ __forceinline__ const void* lane_ptr(uint64_t held, int i) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(held), i);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(held >> 32), i);
  return reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// NJ: slots per wave, 16 for p <= 64 (half the instructions), 24 for p <= 96
// and 32 beyond.
template <int D, int ALGO, bool RS, int NJ>
__global__ __launch_bounds__(kBlock) void reduce_small_kernel(const ReduceArgs a) {
  using S = Storage<D>;
  using E = typename S::elem;
  constexpr int ES = static_cast<int>(sizeof(E));
  constexpr int kWaves = kBlock / 64;
  constexpr int kPerWave = NJ;                                   // slots a wave moves, at most
  static_assert((NJ == 16 || NJ == 24 || NJ == 32) && NJ * kWaves <= kMaxRanks, "16, 24 or 32 slots per wave");
  constexpr bool kPairs = ALGO != VCOLL_RING && ALGO != VCOLL_BINARY_TREE;
  __shared__ float val[NJ * kWaves * kSmallTile];                // [slot][element], every slot written
  __shared__ float res[kSmallTile];
  const int c = blockIdx.y;
  const int p = a.p;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int64_t off = c * a.q + (c < a.r ? c : a.r);
  const int64_t cnt = a.q + (c < a.r ? 1 : 0);
  const int64_t e0 = static_cast<int64_t>(blockIdx.x) * kSmallTile;
  if (e0 >= cnt) return;                                         // the whole workgroup
  const int T = cnt - e0 < kSmallTile ? static_cast<int>(cnt - e0) : kSmallTile;
  const int64_t tile = (off + e0) * ES;                          // the tile's byte offset in every rank
  const int slots = ALGO == VCOLL_RING ? p : a.groups;
  static_assert(kMaxRanks == 128 && kWaves == 4, "two table entries per lane, slots below 64 for j < 16");
  constexpr int kLow = 16;                                       // j < kLow: slot below 64
  const uint64_t* const lt = reinterpret_cast<const uint64_t*>(a.leaf);
  const uint64_t* const dt = reinterpret_cast<const uint64_t*>(a.dst);
  constexpr bool kHigh = NJ > 16;                                // slots 64 and up
  const uint64_t leaf_lo = lt[lane];                             // leaf[l], leaf[64 + l]
  const uint64_t leaf_hi = kHigh ? lt[64 + lane] : 0;
  [[maybe_unused]] uint64_t pair_lo = 0, pair_hi = 0;            // leaf[128 + l], leaf[192 + l]
  if constexpr (kPairs) {
    pair_lo = lt[kMaxRanks + lane];
    pair_hi = kHigh ? lt[kMaxRanks + 64 + lane] : 0;
  }
  [[maybe_unused]] uint64_t dst_lo = 0, dst_hi = 0;              // dst[l], dst[64 + l]
  if constexpr (!RS) {
    dst_lo = dt[lane];
    dst_hi = kHigh ? dt[64 + lane] : 0;
  }
  E x[kPerWave];
  [[maybe_unused]] E y[kPerWave];
  [[maybe_unused]] bool pair[kPerWave];
#pragma unroll
  for (int j = 0; j < kPerWave; ++j) {
    const int s = wave + j * kWaves;                             // < kMaxRanks
    const int bytes = s < slots ? T * ES : 0;
    const int held = s - (j < kLow ? 0 : 64);
    const void* first = lane_ptr(j < kLow ? leaf_lo : leaf_hi, held);
    x[j] = buf_ld1<E>(raw_rsrc(first, tile, bytes), lane * ES);
    if constexpr (kPairs) {
      const void* second = lane_ptr(j < kLow ? pair_lo : pair_hi, held);
      pair[j] = second != nullptr;
      y[j] = buf_ld1<E>(raw_rsrc(pair[j] ? second : first, tile, pair[j] ? bytes : 0), lane * ES);
    }
  }
#pragma unroll
  for (int j = 0; j < kPerWave; ++j) {
    float v = S::widen1(x[j]);
    if constexpr (kPairs) v = pair[j] ? v + S::widen1(y[j]) : v;
    val[(wave + j * kWaves) * kSmallTile + lane] = v;
  }
  __syncthreads();
  if (threadIdx.x < T) {
    const int tid = threadIdx.x;
    float result;
    // the ring's chain is sequential in its adds, not in its LDS reads: the
    // reads of the next leaves go out ahead of the adds (p = 72 at 1 KiB per
    // rank 6.5 -> 5.1 us, at 256 KiB 25.8 -> 22.5 us)
    if constexpr (ALGO == VCOLL_RING) {
      int leaf = (c + 1) % p;                                    // chunk c's chain starts at rank c+1
      result = val[leaf * kSmallTile + tid];
#pragma unroll 8
      for (int k = 1; k < p; ++k) {
        leaf = leaf + 1 == p ? 0 : leaf + 1;
        result = result + val[leaf * kSmallTile + tid];
      }
    } else {
      constexpr int B = 8;
      float lvl[kLevels][1], out1[1];
#pragma unroll 1
      for (int q0 = 0; q0 < slots; q0 += B) {
        float xs[B];
#pragma unroll
        for (int b = 0; b < B; ++b) xs[b] = val[(q0 + b) * kSmallTile + tid];   // q0 + b < NJ * kWaves
        static_for<0, B>([&](auto bb) {
          constexpr int b = decltype(bb)::value;
          if (q0 + b < slots) {
            float v[1] = {xs[b]};
            counter_push<B, b>(lvl, v, q0);
          }
        });
      }
      counter_total(lvl, slots, out1);
      result = out1[0];
    }
    res[tid] = result;
  }
  __syncthreads();
  const E out = S::narrow1(res[lane]);                           // lanes past T store nothing
  if constexpr (RS) {
    if (wave == 0) buf_st1<E>(out, raw_rsrc(a.dst[c], e0 * ES, T * ES), lane * ES);
  } else {
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
      const int r = wave + j * kWaves;
      const void* dst = lane_ptr(j < kLow ? dst_lo : dst_hi, r - (j < kLow ? 0 : 64));
      buf_st1<E>(out, raw_rsrc(dst, tile, r < p ? T * ES : 0), lane * ES);
    }
  }
}

// When the run-time path stages its chunks through LDS: always for chunks of
// up to kSmallAlways elements, and up to kSmallMax while the grid has at
// most kSmallMaxGroups workgroups. Its 4-byte accesses cost bandwidth that
// the per-thread path's 16-byte ones save, so it wins while the call is
// latency-bound. Measured on MI355X (float32, all four algorithms): chunks
// of 1820-3972 elements on 1032-2100 workgroups (p = 24 x 256 KiB, p = 33 x
// 512 KiB, p = 72 and p = 100 x 512 KiB per rank) 25-45 % faster than the
// per-thread path; chunks of 2621-3641 elements on 4100 workgroups (p = 72
// and p = 100 x 1 MiB) up to 35 % slower.
constexpr int64_t kSmallAlways = 1024;
constexpr int64_t kSmallMax = 4096;
constexpr int64_t kSmallMaxGroups = 3072;

inline bool use_small(int64_t max_chunk, int chunks) {
  const int64_t groups = (max_chunk + kSmallTile - 1) / kSmallTile * chunks;
  return max_chunk <= kSmallAlways || (max_chunk <= kSmallMax && groups <= kSmallMaxGroups);
}

// 16-byte vectors per thread of the reduce kernel (all are loaded before the
// first add). p = 8: four against two on MI355X (float32, rank rows padded,
// ring and recursive doubling, with the pacing bound below counted in
// two-vector workgroups) 10 % faster at 4 MiB per rank, 4-6 % at 16-128 MiB,
// 1 % at 256 MiB, and 1 % slower for the trees on the 25 MiB bucket.
// Build-time override: -DVCOLL_V_P8=<n> for p = 8.
#ifndef VCOLL_V_P8
#define VCOLL_V_P8 4
#endif
// Threads per workgroup of the reduce kernel: one wave for p = 16 (measured
// +1-3% on the 16 x 192 MiB bf16 all-reduce, +7% at 4 MiB per rank) and for
// a run-time p (p = 33, 72 and 100 at 1-64 MiB per rank, float32, every
// algorithm: 3.5 % faster on geometric mean than four waves, 10 % at 2 MiB,
// 3-4 % at 4 and 64 MiB, even at 1 MiB; two waves 2 %), four waves
// otherwise. Build-time override for a run-time p: -DVCOLL_RT_BLOCK=<n>.
#ifndef VCOLL_RT_BLOCK
#define VCOLL_RT_BLOCK 64
#endif
template <int P>
constexpr int block_size() {
  return P == 16 ? 64 : (P == 0 ? VCOLL_RT_BLOCK : kBlock);
}

template <int P>
constexpr int vectors_per_thread() {
  return P == 0 ? 1 : (P <= 4 ? 4 : (P <= 8 ? VCOLL_V_P8 : 1));
}

// p = 8 grids of fewer than this many four-vector workgroups take two
// vectors per thread: latency-bound, they need the workgroups. On MI355X
// (float32) two vectors ran 0.5-2 MiB per rank (up to 128 four-vector
// workgroups) in 3.8-5.6 us against 4.6-6.7 with four, but 3 MiB (192) in
// 10.8 us against 8.2.
constexpr int64_t kP8FourVectorMinGroups = 192;

// p = 16 grids of at most this many one-vector workgroups take two vectors
// per thread instead: on MI355X (float32, rank rows padded) p = 16 x 16 MiB
// per rank 105 -> 90.7 us for the trees, 4-32 MiB 1-3 % faster, but 64 MiB
// 4 % slower (349 -> 364 us).
constexpr int64_t kP16TwoVectorMaxGroups = 32768;

// The compiled-p kernel with V vectors per thread (the LARGE variant carries
// the pacing and its load pipeline).
template <int D, int ALGO, bool RS, int P, int V>
hipError_t launch_fixed(const ReduceArgs& a, int64_t max_chunk, int chunks, hipStream_t stream) {
  constexpr int BS = block_size<P>();
  constexpr int64_t per_tile = static_cast<int64_t>(V) * BS * Storage<D>::kVE;
  const int64_t tiles = (max_chunk + per_tile - 1) / per_tile;
  if (tiles == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(tiles), chunks);
  ReduceArgs args = a;
  // the pacing bound was measured in workgroups of the p = 8 kernel's
  // two-vector shape; its four-vector workgroups count twice (counted once,
  // 16-28 MiB per rank fell back to the unpaced variant and lost 2-8 %)
  args.pace = !RS && tiles * a.p * (P == 8 ? (V + 1) / 2 : 1) >= VCOLL_PACE_MIN_GROUPS;
  if (args.pace) return launch(reduce_kernel<D, ALGO, P, V, RS, true, BS>, grid, BS, args, stream);
  return launch(reduce_kernel<D, ALGO, P, V, RS, false, BS>, grid, BS, args, stream);
}

template <int D, int ALGO, bool RS, int P>
hipError_t launch_reduce_p(const ReduceArgs& a, int64_t max_chunk, int chunks, hipStream_t stream) {
  constexpr int V = vectors_per_thread<P>();
  constexpr int BS = block_size<P>();
  constexpr int VE = Storage<D>::kVE;
  const int64_t per_tile = static_cast<int64_t>(V) * BS * VE;
  const int64_t tiles = (max_chunk + per_tile - 1) / per_tile;
  if (tiles == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(tiles), chunks);
  ReduceArgs args = a;
  args.pace = !RS && tiles * a.p >= VCOLL_PACE_MIN_GROUPS;
  if constexpr (P > 0) {
    if constexpr (P == 16) {
      if (tiles * chunks <= kP16TwoVectorMaxGroups) return launch_fixed<D, ALGO, RS, P, 2>(a, max_chunk, chunks, stream);
    }
    if constexpr (P == 8 && V == 4) {
      if (tiles * chunks < kP8FourVectorMinGroups) return launch_fixed<D, ALGO, RS, P, 2>(a, max_chunk, chunks, stream);
    }
    return launch_fixed<D, ALGO, RS, P, V>(a, max_chunk, chunks, stream);
  } else {
    if (use_small(max_chunk, chunks)) {
      const dim3 small(static_cast<unsigned>((max_chunk + kSmallTile - 1) / kSmallTile), chunks);
      if (a.p <= 64) return launch(reduce_small_kernel<D, ALGO, RS, 16>, small, args, stream);
      if (a.p <= 96) return launch(reduce_small_kernel<D, ALGO, RS, 24>, small, args, stream);
      return launch(reduce_small_kernel<D, ALGO, RS, 32>, small, args, stream);
    }
    if constexpr (RS && ALGO == VCOLL_RING) {
      bool aligned = true;
      for (int c = 0; c < chunks && aligned; ++c) aligned = (c * a.q + (c < a.r ? c : a.r)) % VE == 0;
      if (a.vec) {
        // waves cover d + nvec input vectors per chunk: d < 8 (the line start
        // before the chunk, line-aligned shape only), nvec < the chunk's vectors
        const int64_t in_vecs = (max_chunk + VE - 1) / VE + 8;
        const int64_t waves = (in_vecs + 63) / 64 * chunks;
        // the line-aligned shape also beats the reduce kernel on aligned
        // chunks (float32 on MI355X: p = 33 x 64 MiB per rank 397 -> 370 us,
        // p = 72 877 -> 812, p = 64 within 0.5 %); the 63-output shape does
        // not (p = 64 x 16 MiB 180 -> 198 us), so aligned chunks take only
        // the former
        if constexpr (D == VCOLL_F32) {
          if (waves >= kShiftLinesMinWaves) {
            const int64_t per_group = static_cast<int64_t>(kBlock / 64) * 64;
            const dim3 sg(static_cast<unsigned>((in_vecs + per_group - 1) / per_group), chunks);
            return launch(reduce_scatter_shifted_kernel<D, true>, sg, args, stream);
          }
        }
        if (!aligned) {
          const int64_t per_group = static_cast<int64_t>(kBlock / 64) * 63;
          const dim3 sg(static_cast<unsigned>((in_vecs + per_group - 1) / per_group), chunks);
          return launch(reduce_scatter_shifted_kernel<D, false>, sg, args, stream);
        }
      }
    }
    return launch(reduce_kernel<D, ALGO, P, V, RS, false, BS>, grid, BS, args, stream);
  }
}

template <int D, int ALGO, bool RS>
hipError_t launch_reduce_algo(const ReduceArgs& a, int64_t max_chunk, int chunks, hipStream_t stream) {
  static_assert(has_fixed_kernel(2) && has_fixed_kernel(4) && has_fixed_kernel(8) && has_fixed_kernel(16),
                "the host lays out leaf pointers by has_fixed_kernel()");
  switch (a.p) {
    case 2: return launch_reduce_p<D, ALGO, RS, 2>(a, max_chunk, chunks, stream);
    case 4: return launch_reduce_p<D, ALGO, RS, 4>(a, max_chunk, chunks, stream);
    case 8: return launch_reduce_p<D, ALGO, RS, 8>(a, max_chunk, chunks, stream);
    case 16: return launch_reduce_p<D, ALGO, RS, 16>(a, max_chunk, chunks, stream);
    default: return launch_reduce_p<D, ALGO, RS, 0>(a, max_chunk, chunks, stream);
  }
}

template <int D>
hipError_t launch_reduce_dtype(const ReduceArgs& a, vcoll_algo algo, bool scatter, int64_t max_chunk,
                               int chunks, hipStream_t stream) {
  if (scatter) {
    if (algo == VCOLL_RING) return launch_reduce_algo<D, VCOLL_RING, true>(a, max_chunk, chunks, stream);
    if (algo == VCOLL_BINARY_TREE)
      return launch_reduce_algo<D, VCOLL_BINARY_TREE, true>(a, max_chunk, chunks, stream);
    return launch_reduce_algo<D, VCOLL_RABENSEIFNER, true>(a, max_chunk, chunks, stream);
  }
  switch (algo) {
    case VCOLL_RING: return launch_reduce_algo<D, VCOLL_RING, false>(a, max_chunk, chunks, stream);
    case VCOLL_RECURSIVE_DOUBLING:
      return launch_reduce_algo<D, VCOLL_RECURSIVE_DOUBLING, false>(a, max_chunk, chunks, stream);
    case VCOLL_RABENSEIFNER:
      return launch_reduce_algo<D, VCOLL_RABENSEIFNER, false>(a, max_chunk, chunks, stream);
    default: return launch_reduce_algo<D, VCOLL_BINARY_TREE, false>(a, max_chunk, chunks, stream);
  }
}

// ----------------------------------------------------------------------------
// the ring all-reduce in two chip-wide phases (see BurstArgs)
//
// When the reduced vector (n elements) fits in the register files of one
// workgroup per compute unit, every workgroup first reads its tile of all p
// ranks and only then writes the tile's sums to all p outputs; the
// workgroups start together, so HBM sees a read phase and then a write
// phase instead of p read and p write streams interleaved throughout. On
// MI355X this took the DDP bucket all-reduce (p = 8 x 25 MiB float32) from
// 74 to 68 us and 16 MiB per rank from 46.6 to 42.5 us; with several
// workgroup generations (larger n) or fewer than ~16 vectors per thread
// (smaller n) the one-pass kernel above is faster, and the host picks.
//
// Loads and stores use buffer instructions: one resource per (rank, tile)
// whose size is the tile's valid bytes, so a ragged last tile needs no
// masks (loads beyond it return 0, stores beyond it are dropped), one
// 32-bit lane offset, and the vector index as an immediate scalar offset.
// The tiles of chunk c cover the 16-byte vectors that lie wholly inside the
// chunk, from the first one on a 128-byte cache-line boundary of every
// buffer (when the buffers share an address phase mod 128) and in tiles of
// whole lines, so no two waves write parts of one line; the chunk's
// remaining first and last elements (under 128 bytes' worth at each end)
// are summed one by one, in the same chain order, by workgroup 0 of the
// chunk after its tile (before it, their loads queue behind the whole
// chip's read phase and delay that workgroup's tile). Measured on MI355X at
// p = 72 x 16 MiB float32, whose chunk starts are only 16-byte aligned:
// tiles on 16-byte boundaries ran at 4.4 TB/s, on cache lines with the end
// elements first at 5.7 TB/s, and last at 5.9 TB/s. Buffers whose addresses
// differ mod 128 cannot all have their tiles on whole lines; there two
// waves write parts of one line, and the stores go through L2 (default
// policy), which merges those parts: against streaming stores, p = 8 x 16
// MiB with rows 16 bytes off a line apart went from 54.3 to 47.2 us and
// p = 72 from 524 to 474 us; aligned layouts gained 1-4 % with the buffers
// cycled out of the Infinity Cache (p = 4 to 16 at 16 MiB, the DDP bucket),
// except p = 2 (below). (Cached loads lost 5 %.)

constexpr int kBurstBlock = 256;                 // one wave per SIMD
constexpr int kBurstVecF32 = 25;                 // float32: 100 sums + 25 vectors in flight per thread
constexpr int kBurstVecBf16 = 16;                // bf16: 128 sums + 16 vectors in flight

// One element of a chunk, summed along the chunk's chain (the first leaf
// taken as it is, not added to zero) and stored to every output; the loads
// go out kOneBatch ranks at a time.
template <int D>
__device__ __forceinline__ void burst_one(const BurstArgs& a, int first_rank, int64_t e) {
  using S = Storage<D>;
  using E = typename S::elem;
  constexpr int kOneBatch = 64;
  const int p = a.p;
  float acc = 0.0f;
  int rank = first_rank;
  for (int k0 = 0; k0 < p; k0 += kOneBatch) {
    E raw[kOneBatch];
#pragma unroll
    for (int b = 0; b < kOneBatch; ++b) {
      if (k0 + b < p) {
        raw[b] = static_cast<const E*>(a.src[rank])[e];
        rank = rank + 1 == p ? 0 : rank + 1;
      }
    }
#pragma unroll
    for (int b = 0; b < kOneBatch; ++b)
      if (k0 + b < p) acc = k0 + b == 0 ? S::widen1(raw[b]) : acc + S::widen1(raw[b]);
  }
  const E out = S::narrow1(acc);
  for (int r = 0; r < p; ++r) static_cast<E*>(a.dst[r])[e] = out;
}

template <int D, int K, int SPOL>
__global__ __launch_bounds__(kBurstBlock) void burst_ring_kernel(const BurstArgs a) {
  using S = Storage<D>;
  constexpr int VE = S::kVE;
  const int p = a.p;
  const int c = blockIdx.y;
  const int first_rank = c + 1 == p ? 0 : c + 1;           // chunk c's chain: ranks c+1, ..., p-1, 0, ..., c
  const int64_t e0 = c * a.q + (c < a.r ? c : a.r);        // the chunk's elements [e0, e1)
  const int64_t e1 = e0 + a.q + (c < a.r ? 1 : 0);
  const int64_t vs = burst_first_vector(e0, VE, a.align, a.phase);   // the tiles' vectors [vs, ve)
  const int64_t ve = e1 / VE > vs ? e1 / VE : vs;
  // the elements outside the tiles: [e0, vs*VE) and [ve*VE, e1), or all of
  // them if the chunk has no tile vectors
  auto edges = [&]() {
    const int64_t head_end = vs * VE < e1 ? vs * VE : e1;
    const int64_t tail_lo = ve * VE > head_end ? ve * VE : head_end;
    const int64_t tail_begin = tail_lo < e1 ? tail_lo : e1;
    const int64_t head = head_end - e0;
    const int64_t n_one = head + (e1 - tail_begin);
    for (int64_t i = threadIdx.x; i < n_one; i += kBurstBlock)
      burst_one<D>(a, first_rank, i < head ? e0 + i : tail_begin + (i - head));
  };
  const int64_t cv = ve - vs;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * a.tv;
  const int64_t left = cv - t0;
  if (left <= 0) {                                         // the whole workgroup
    if (blockIdx.x == 0) edges();
    return;
  }
  const int bytes = static_cast<int>((left < a.tv ? left : a.tv) * 16);
  const int64_t off = (vs + t0) * 16;                      // tile's byte offset in every rank
  const int vo = threadIdx.x * 16;
  float acc[K][VE];
  u32x4 buf[K];
  int rank = first_rank;
  {
    const __amdgpu_buffer_rsrc_t r = raw_rsrc(a.src[rank], off, bytes);
#pragma unroll
    for (int j = 0; j < K; ++j)
      buf[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, vo, j * kBurstBlock * 16, kPolicyNT));
  }
  // leaf k: add it vector by vector and, as each vector's registers free up,
  // request the same vector of leaf k + 1 (every wait then covers exactly the
  // vector about to be added, with K loads in flight throughout)
  auto leaf = [&](auto first, auto reload, const __amdgpu_buffer_rsrc_t& next) {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      __builtin_amdgcn_sched_barrier(0);
      float v[VE];
      S::widen(buf[j], v);
#pragma unroll
      for (int i = 0; i < VE; ++i) acc[j][i] = decltype(first)::value ? v[i] : acc[j][i] + v[i];
      if constexpr (decltype(reload)::value)
        buf[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(next, vo, j * kBurstBlock * 16, kPolicyNT));
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  auto next_rsrc = [&]() {
    rank = rank + 1 == p ? 0 : rank + 1;
    return raw_rsrc(a.src[rank], off, bytes);
  };
  if (p == 1) {
    leaf(T_{}, F_{}, raw_rsrc(a.src[rank], off, bytes));
  } else {
    leaf(T_{}, T_{}, next_rsrc());
    for (int k = 1; k < p - 1; ++k) leaf(F_{}, T_{}, next_rsrc());
    leaf(F_{}, F_{}, raw_rsrc(a.src[rank], off, bytes));
  }
  u32x4 out[K];
#pragma unroll
  for (int j = 0; j < K; ++j) out[j] = S::narrow(acc[j]);
  for (int d = 0; d < p; ++d) {
    const __amdgpu_buffer_rsrc_t r = raw_rsrc(a.dst[d], off, bytes);
#pragma unroll
    for (int j = 0; j < K; ++j)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, out[j]), r, vo, j * kBurstBlock * 16, SPOL);
  }
  if (blockIdx.x == 0) edges();
}

}  // namespace

int64_t burst_tile_max(vcoll_dtype dtype) {
  return static_cast<int64_t>(dtype == VCOLL_F32 ? kBurstVecF32 : kBurstVecBf16) * kBurstBlock;
}

hipError_t launch_burst_ring(const BurstArgs& a, vcoll_dtype dtype, int tiles, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(a.p));
  // the write phase stores through L2 (see above), except for p <= 2, where
  // streaming stores measured 3.5 % faster (p = 2 x 16 MiB, buffers cycled
  // out of the Infinity Cache; p = 4 to 16 and the DDP bucket gained 1-4 %
  // from cached stores)
  const bool cached = a.p > 2;
  if (dtype == VCOLL_F32)
    return cached ? launch(burst_ring_kernel<VCOLL_F32, kBurstVecF32, kPolicyCached>, grid, kBurstBlock, a, stream)
                  : launch(burst_ring_kernel<VCOLL_F32, kBurstVecF32, kPolicyNT>, grid, kBurstBlock, a, stream);
  return cached ? launch(burst_ring_kernel<VCOLL_BF16, kBurstVecBf16, kPolicyCached>, grid, kBurstBlock, a, stream)
                : launch(burst_ring_kernel<VCOLL_BF16, kBurstVecBf16, kPolicyNT>, grid, kBurstBlock, a, stream);
}

hipError_t launch_reduce(const ReduceArgs& a, vcoll_dtype dtype, vcoll_algo algo, bool scatter,
                         int64_t max_chunk, int chunks, hipStream_t stream) {
  if (dtype == VCOLL_F32) return launch_reduce_dtype<VCOLL_F32>(a, algo, scatter, max_chunk, chunks, stream);
  return launch_reduce_dtype<VCOLL_BF16>(a, algo, scatter, max_chunk, chunks, stream);
}

}  // namespace vcoll
