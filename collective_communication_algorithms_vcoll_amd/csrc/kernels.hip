// Device kernels of libvcoll for gfx950 (MI355X): fused reduce + fan-out,
// all-gather fan-out, variable-split all-to-all row mover, plain copy.
//
// Summation orders come from "Networks and Collective Communication" (cs349e
// prerequisite lecture 5), sections 5.1 (ring) and 5.2 (recursive doubling,
// Rabenseifner, binomial tree); order.h writes each as a push / add program.
#include <type_traits>

#include "kernels.h"

namespace vcoll {
namespace {

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

template <int K, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (K < N) {
    f(std::integral_constant<int, K>{});
    static_for<K + 1, N>(f);
  }
}

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


// Row of leaf pointers of chunk c (p compiled in): the ring's order rotates
// with the chunk, the trees' order is the same for every chunk (row 0).
template <int ALGO>
__device__ __forceinline__ const void* const* leaf_row(const ReduceArgs& a, int c) {
  return &a.leaf[(ALGO == VCOLL_RING ? c : 0) * kFixedMax];
}

// ----------------------------------------------------------------------------
// order programs read at run time (any p): a shift-register stack keeps every
// index a compile-time constant, so the stack lives in registers

constexpr int kRuntimeDepth = 9;   // deepest stack of any program with p <= 128

template <int N>
__device__ __forceinline__ void rt_push(float (&st)[kRuntimeDepth][N], const float* v) {
#pragma unroll
  for (int s = kRuntimeDepth - 1; s > 0; --s)
#pragma unroll
    for (int i = 0; i < N; ++i) st[s][i] = st[s - 1][i];
#pragma unroll
  for (int i = 0; i < N; ++i) st[0][i] = v[i];
}

template <int N>
__device__ __forceinline__ void rt_merge(float (&st)[kRuntimeDepth][N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) st[0][i] = st[1][i] + st[0][i];
#pragma unroll
  for (int s = 1; s < kRuntimeDepth - 1; ++s)
#pragma unroll
    for (int i = 0; i < N; ++i) st[s][i] = st[s + 1][i];
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
  } else if constexpr (ALGO == VCOLL_RING) {
    result = S::widen1(static_cast<const E*>(a.leaf[rot % p])[e]);
    for (int k = 1; k < p; ++k)
      result = result + S::widen1(static_cast<const E*>(a.leaf[(rot + k) % p])[e]);
  } else {
    float st[kRuntimeDepth][1];
    for (int k = 0; k < p; ++k) {
      const float v = S::widen1(static_cast<const E*>(a.leaf[a.rank[k]])[e]);
      rt_push<1>(st, &v);
      for (int m = 0; m < a.merges[k]; ++m) rt_merge<1>(st);
    }
    for (int m = 0; m < a.final_merges; ++m) rt_merge<1>(st);
    result = st[0][0];
  }
  const E out = S::narrow1(result);
  if constexpr (RS) {
    static_cast<E*>(a.dst[c])[e - off] = out;
  } else {
    for (int r = 0; r < p; ++r) static_cast<E*>(a.dst[r])[e] = out;
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
#pragma unroll
      for (int j = 0; j < V; ++j) {
        if constexpr (FULL) {
          raw[k][j] = ld16(L[k], boff[j]);
        } else {
          raw[k][j] = valid[j] ? ld16(L[k], boff[j]) : u32x4{0, 0, 0, 0};
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
  constexpr int B = 8;
  float acc[VE];
  float st[kRuntimeDepth][VE];
  for (int k0 = 0; k0 < p; k0 += B) {
    u32x4 raw[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if (k0 + b < p) {
        const int rank = (ALGO == VCOLL_RING) ? (rot + k0 + b) % p : a.rank[k0 + b];
        raw[b] = valid ? ld16(a.leaf[rank], boff) : u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if (k0 + b < p) {
        float v[VE];
        S::widen(raw[b], v);
        if constexpr (ALGO == VCOLL_RING) {
          if (k0 + b == 0) {
#pragma unroll
            for (int i = 0; i < VE; ++i) acc[i] = v[i];
          } else {
#pragma unroll
            for (int i = 0; i < VE; ++i) acc[i] = acc[i] + v[i];
          }
        } else {
          rt_push<VE>(st, v);
          for (int m = 0; m < a.merges[k0 + b]; ++m) rt_merge<VE>(st);
        }
      }
    }
  }
  if constexpr (ALGO != VCOLL_RING) {
    for (int m = 0; m < a.final_merges; ++m) rt_merge<VE>(st);
#pragma unroll
    for (int i = 0; i < VE; ++i) acc[i] = st[0][i];
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

template <int D, int ALGO, int P, int V, bool RS, bool LARGE>
__global__ __launch_bounds__(kBlock) void reduce_kernel(const ReduceArgs a) {
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
  // sides must be vector aligned, so the chunk start must be
  const bool vec = a.vec != 0 && (!RS || (off % VE) == 0);

  if (vec) {
    const int64_t head = (VE - off % VE) % VE < cnt ? (VE - off % VE) % VE : cnt;
    const int64_t nvec = (cnt - head) / VE;
    const int64_t e_base = off + head;
    const int64_t v0 = static_cast<int64_t>(blockIdx.x) * (V * kBlock) + tid;
    if (static_cast<int64_t>(blockIdx.x) * (V * kBlock) < nvec) {
      if constexpr (P > 0) {
        int64_t boff[V];
        bool valid[V];
#pragma unroll
        for (int j = 0; j < V; ++j) {
          const int64_t v = v0 + j * kBlock;
          valid[j] = v < nvec;
          boff[j] = (e_base + v * VE) * ES;
        }
        if ((static_cast<int64_t>(blockIdx.x) + 1) * (V * kBlock) <= nvec) {
          reduce_vectors_fixed<D, ALGO, P, V, RS, LARGE, true>(a, c, boff, valid, off * ES);
        } else {
          reduce_vectors_fixed<D, ALGO, P, V, RS, LARGE, false>(a, c, boff, valid, off * ES);
        }
      } else {
#pragma unroll 1
        for (int j = 0; j < V; ++j) {
          const int64_t v = v0 + j * kBlock;
          reduce_vector_runtime<D, ALGO, RS>(a, c, p, rot, (e_base + v * VE) * ES, v < nvec,
                                             off * ES);
        }
      }
    }
    if (blockIdx.x == 0) {
      const int64_t tail = cnt - head - nvec * VE;
      if (tid < head) {
        reduce_one<D, ALGO, P, RS>(a, c, p, rot, off + tid, off);
      } else if (tid >= 16 && tid - 16 < tail) {
        reduce_one<D, ALGO, P, RS>(a, c, p, rot, e_base + nvec * VE + (tid - 16), off);
      }
    }
  } else {
    const int64_t e0 = static_cast<int64_t>(blockIdx.x) * (V * kBlock * VE);
#pragma unroll 1
    for (int j = 0; j < V * VE; ++j) {
      const int64_t i = e0 + j * kBlock + tid;
      if (i < cnt) reduce_one<D, ALGO, P, RS>(a, c, p, rot, off + i, off);
    }
  }
}

// ----------------------------------------------------------------------------
// hierarchical / 2D all-reduce ("Networks and Collective Communication",
// sections 6.1 and 6.3): ranks form `nodes` groups of `local`. In piece j of
// chunk l the value is an outer chain over the groups, starting after group
// j (the cross-group ring reduce-scatter), of inner chains over each group's
// ranks, starting after rank l of the group (the in-group ring
// reduce-scatter).

__device__ __forceinline__ void hier_segment(const HierArgs& a, int u, int& l, int& j, int64_t& off,
                                             int64_t& cnt) {
  const int N = a.nodes, Lc = a.local;
  l = u / N;
  j = u - l * N;
  const int64_t qL = a.n / Lc, rL = a.n % Lc;
  const int64_t offL = l * qL + (l < rL ? l : rL);
  const int64_t lenL = qL + (l < rL ? 1 : 0);
  const int64_t qN = lenL / N, rN = lenL % N;
  off = offL + j * qN + (j < rN ? j : rN);
  cnt = qN + (j < rN ? 1 : 0);
}

template <int D>
__device__ __forceinline__ void hier_one(const HierArgs& a, int N, int Lc, int l, int j, int64_t e) {
  using S = Storage<D>;
  using E = typename S::elem;
  float outer = 0.0f;
  for (int ko = 0; ko < N; ++ko) {
    const int g = (j + 1 + ko) % N;
    float inner = 0.0f;
    for (int ki = 0; ki < Lc; ++ki) {
      const float v = S::widen1(static_cast<const E*>(a.ptr.src[g * Lc + (l + 1 + ki) % Lc])[e]);
      inner = ki == 0 ? v : inner + v;
    }
    outer = ko == 0 ? inner : outer + inner;
  }
  const E out = S::narrow1(outer);
  for (int r = 0; r < N * Lc; ++r) static_cast<E*>(a.ptr.dst[r])[e] = out;
}

// One 16-byte vector per thread; the loads of group ko+1 go out before group
// ko is added (NN, LL compiled in; 0 = read from the arguments).
template <int D, int NN, int LL, bool LARGE, bool FULL>
__device__ __forceinline__ void hier_vector(const HierArgs& a, int l, int j, int64_t boff, bool valid) {
  using S = Storage<D>;
  constexpr int VE = S::kVE;
  float outer[VE], inner[VE], v[VE];
  if constexpr (NN > 0) {
    u32x4 raw[2][LL];
    static_for<0, NN + 1>([&](auto kc) {
      constexpr int ko = decltype(kc)::value;
      if constexpr (ko < NN) {
        const int g = (j + 1 + ko) % NN;
#pragma unroll
        for (int ki = 0; ki < LL; ++ki) {
          const void* src = a.ptr.src[g * LL + (l + 1 + ki) % LL];
          raw[ko & 1][ki] = (FULL || valid) ? ld16(src, boff) : u32x4{0, 0, 0, 0};
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (ko >= 1) {
        constexpr int q = ko - 1;
#pragma unroll
        for (int ki = 0; ki < LL; ++ki) {
          S::widen(raw[q & 1][ki], v);
#pragma unroll
          for (int i = 0; i < VE; ++i) inner[i] = ki == 0 ? v[i] : inner[i] + v[i];
        }
#pragma unroll
        for (int i = 0; i < VE; ++i) outer[i] = q == 0 ? inner[i] : outer[i] + inner[i];
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  } else {
    const int N = a.nodes, Lc = a.local;
    for (int ko = 0; ko < N; ++ko) {
      const int g = (j + 1 + ko) % N;
      for (int ki = 0; ki < Lc; ++ki) {
        const u32x4 w = valid ? ld16(a.ptr.src[g * Lc + (l + 1 + ki) % Lc], boff) : u32x4{0, 0, 0, 0};
        S::widen(w, v);
        for (int i = 0; i < VE; ++i) inner[i] = ki == 0 ? v[i] : inner[i] + v[i];
      }
      for (int i = 0; i < VE; ++i) outer[i] = ko == 0 ? inner[i] : outer[i] + inner[i];
    }
  }
  if (!FULL && !valid) return;
  const u32x4 out = S::narrow(outer);
  if constexpr (NN > 0) {
    static_for<0, NN * LL>([&](auto rc) {
      st16(a.ptr.dst[decltype(rc)::value], boff, out);
      if constexpr (LARGE) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_sleep(VCOLL_STORE_SLEEP);
        __builtin_amdgcn_sched_barrier(0);
      }
    });
  } else {
    for (int r = 0; r < a.nodes * a.local; ++r) st16(a.ptr.dst[r], boff, out);
  }
}

template <int D, int NN, int LL, bool LARGE>
__global__ __launch_bounds__(kBlock) void hier_kernel(const HierArgs a) {
  using S = Storage<D>;
  constexpr int VE = S::kVE;
  constexpr int ES = 16 / VE;
  const int N = NN > 0 ? NN : a.nodes, Lc = LL > 0 ? LL : a.local;
  int l, j;
  int64_t off, cnt;
  hier_segment(a, blockIdx.y, l, j, off, cnt);
  const int tid = threadIdx.x;
  if (a.vec) {
    const int64_t head = (VE - off % VE) % VE < cnt ? (VE - off % VE) % VE : cnt;
    const int64_t nvec = (cnt - head) / VE;
    const int64_t e_base = off + head;
    const int64_t v = static_cast<int64_t>(blockIdx.x) * kBlock + tid;
    if (static_cast<int64_t>(blockIdx.x) * kBlock < nvec) {
      const int64_t boff = (e_base + v * VE) * ES;
      if ((static_cast<int64_t>(blockIdx.x) + 1) * kBlock <= nvec) {
        hier_vector<D, NN, LL, LARGE, true>(a, l, j, boff, true);
      } else {
        hier_vector<D, NN, LL, LARGE, false>(a, l, j, boff, v < nvec);
      }
    }
    if (blockIdx.x == 0) {
      const int64_t tail = cnt - head - nvec * VE;
      if (tid < head) hier_one<D>(a, N, Lc, l, j, off + tid);
      else if (tid >= 16 && tid - 16 < tail) hier_one<D>(a, N, Lc, l, j, e_base + nvec * VE + (tid - 16));
    }
  } else {
    const int64_t e0 = static_cast<int64_t>(blockIdx.x) * (kBlock * VE);
#pragma unroll 1
    for (int k = 0; k < VE; ++k) {
      const int64_t i = e0 + k * kBlock + tid;
      if (i < cnt) hier_one<D>(a, N, Lc, l, j, off + i);
    }
  }
}

// ----------------------------------------------------------------------------
// all-gather: block i of every output is a copy of input i

template <int ES, int V>
__global__ __launch_bounds__(kBlock) void all_gather_kernel(const GatherArgs a) {
  const int i = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t bytes = a.m * ES;
  const int64_t dst_off = i * bytes;
  const void* src = a.ptr.src[i];
  if (a.vec) {
    const int64_t nvec = bytes / 16;
    const int64_t v0 = static_cast<int64_t>(blockIdx.x) * (V * kBlock) + tid;
    u32x4 x[V];
    bool valid[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int64_t v = v0 + j * kBlock;
      valid[j] = v < nvec;
      x[j] = valid[j] ? ld16(src, v * 16) : u32x4{0, 0, 0, 0};
    }
    for (int r = 0; r < a.p; ++r) {
#pragma unroll
      for (int j = 0; j < V; ++j)
        if (valid[j]) st16(a.ptr.dst[r], dst_off + (v0 + j * kBlock) * 16, x[j]);
    }
  } else {
    using E = typename std::conditional<ES == 4, uint32_t, uint16_t>::type;
    constexpr int VE = 16 / ES;
    const int64_t e0 = static_cast<int64_t>(blockIdx.x) * (V * kBlock * VE) + tid;
#pragma unroll 1
    for (int j = 0; j < V * VE; ++j) {
      const int64_t e = e0 + j * kBlock;
      if (e < a.m) {
        const E x = static_cast<const E*>(src)[e];
        for (int r = 0; r < a.p; ++r) static_cast<E*>(a.ptr.dst[r])[i * a.m + e] = x;
      }
    }
  }
}

// ----------------------------------------------------------------------------
// broadcast: every receive buffer gets the root's words ("Networks and
// Collective Communication", section 4.1). Whatever the algorithm, the
// result is a copy, so one pass reads the root once and writes q copies.

template <int ES, int V, bool PACE>
__global__ __launch_bounds__(kBlock) void broadcast_kernel(const BcastArgs a) {
  using E = typename std::conditional<ES == 4, uint32_t, uint16_t>::type;
  constexpr int VE = 16 / ES;
  const int tid = threadIdx.x;
  if (a.vec) {
    const int64_t nvec = a.n / VE;
    const int64_t v0 = static_cast<int64_t>(blockIdx.x) * (V * kBlock) + tid;
    u32x4 x[V];
    bool valid[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int64_t v = v0 + j * kBlock;
      valid[j] = v < nvec;
      x[j] = valid[j] ? ld16(a.src, v * 16) : u32x4{0, 0, 0, 0};
    }
    for (int r = 0; r < a.q; ++r) {
#pragma unroll
      for (int j = 0; j < V; ++j)
        if (valid[j]) st16(a.dst[r], (v0 + j * kBlock) * 16, x[j]);
      if constexpr (PACE) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_sleep(VCOLL_STORE_SLEEP);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // the last n mod VE elements
    if (blockIdx.x == 0 && tid < a.n - nvec * VE) {
      const int64_t e = nvec * VE + tid;
      const E w = static_cast<const E*>(a.src)[e];
      for (int r = 0; r < a.q; ++r) static_cast<E*>(a.dst[r])[e] = w;
    }
  } else {
    const int64_t e0 = static_cast<int64_t>(blockIdx.x) * (V * kBlock * VE) + tid;
#pragma unroll 1
    for (int j = 0; j < V * VE; ++j) {
      const int64_t e = e0 + j * kBlock;
      if (e < a.n) {
        const E w = static_cast<const E*>(a.src)[e];
        for (int r = 0; r < a.q; ++r) static_cast<E*>(a.dst[r])[e] = w;
      }
    }
  }
}

// ----------------------------------------------------------------------------
// all-to-all: workgroup t moves rows_per_tile rows of one (i -> j) block

__global__ __launch_bounds__(kBlock) void all_to_all_kernel(const A2AArgs a) {
  const int t = blockIdx.x;
  // the block this workgroup belongs to: last one whose first tile <= t
  int lo = 0, hi = a.nblocks - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (a.b[mid].tile_start <= t) lo = mid;
    else hi = mid - 1;
  }
  const A2ABlock& B = a.b[lo];
  const int r0 = (t - B.tile_start) * a.rows_per_tile;
  const int tid = threadIdx.x;
  for (int rr = 0; rr < a.rows_per_tile; ++rr) {
    const int k = r0 + rr;
    if (k >= B.rows) break;
    const int64_t sr = B.src_idx ? static_cast<int64_t>(B.src_idx[k]) : k;
    const int64_t dr = B.dst_idx ? static_cast<int64_t>(B.dst_idx[k]) : k;
    if (sr < 0 || sr >= B.src_limit || dr < 0 || dr >= B.dst_limit) continue;
    const char* src = B.src + sr * a.row_bytes;
    char* dst = B.dst + dr * a.row_bytes;
    if (a.vec) {
      const int64_t nvec = a.row_bytes / 16;
      constexpr int U = 4;
      for (int64_t x0 = tid; x0 < nvec; x0 += U * kBlock) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t x = x0 + u * kBlock;
          v[u] = x < nvec ? ld16(src, x * 16) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t x = x0 + u * kBlock;
          if (x < nvec) st16(dst, x * 16, v[u]);
        }
      }
    } else if (a.esize == 4) {
      for (int64_t x = tid; x < a.row_bytes / 4; x += kBlock)
        reinterpret_cast<uint32_t*>(dst)[x] = reinterpret_cast<const uint32_t*>(src)[x];
    } else if (a.esize == 2) {
      for (int64_t x = tid; x < a.row_bytes / 2; x += kBlock)
        reinterpret_cast<uint16_t*>(dst)[x] = reinterpret_cast<const uint16_t*>(src)[x];
    } else {
      for (int64_t x = tid; x < a.row_bytes; x += kBlock)
        reinterpret_cast<uint8_t*>(dst)[x] = reinterpret_cast<const uint8_t*>(src)[x];
    }
  }
}

// ----------------------------------------------------------------------------
// FP8 dispatch ("Networks and Collective Communication", section 7.4): rows
// gathered from a bfloat16 token table and quantised on the way to E4M3
// (sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, 448
// the largest value) with one power-of-two scale per 128 elements.

// Smallest k with amax <= 448 * 2^k, clamped to [-126, 126]; 0 for amax = 0.
// amax = 1.m * 2^(E-127) and 448 = 1.75 * 2^8, so k = E - 135 when
// 1.m <= 1.75 (fraction field <= 0x600000) and E - 134 otherwise.
__device__ __forceinline__ int fp8_group_exponent(float amax) {
  const uint32_t u = __float_as_uint(amax);
  if (u == 0) return 0;
  const int E = static_cast<int>(u >> 23);
  if (E == 0) return -126;
  const int k = (u & 0x7FFFFFu) <= 0x600000u ? E - 135 : E - 134;
  return k < -126 ? -126 : (k > 126 ? 126 : k);
}

// |y| <= 448 (or non-finite) -> E4M3 code, round to nearest, ties to even,
// done on the float32 bit pattern.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t b = __float_as_uint(y);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t u = b & 0x7FFFFFFFu;
  if (u >= 0x7F800000u) return 0x7Fu;                 // infinity or NaN
  const int E = static_cast<int>(u >> 23);
  if (E == 0) return sign;                             // zero, or a float32 subnormal (< 2^-126)
  const int e = E - 127;
  const uint32_t mant = (u & 0x7FFFFFu) | 0x800000u;   // 1.f times 2^23
  // normal results keep 1 + 3 fraction bits; below 2^-6 the grid is 2^-9:
  // y * 2^9 = mant * 2^(e - 14)
  const int shift = e >= -6 ? 20 : 14 - e;
  if (shift > 24) return sign;                         // below 2^-10: rounds to zero
  uint32_t q = mant >> shift;
  const uint32_t rem = mant & ((1u << shift) - 1u);
  const uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (q & 1u))) ++q;
  if (e >= -6) {
    int ee = e;
    if (q == 16u) {
      q = 8u;
      ++ee;
    }
    return sign | (static_cast<uint32_t>(ee + 7) << 3) | (q - 8u);
  }
  return sign | q;                                     // 0..8 (8 is 2^-6: exponent field 1)
}

__global__ __launch_bounds__(kBlock) void dispatch_fp8_kernel(const Fp8Args a) {
  const int t = blockIdx.x;
  int lo = 0, hi = a.nblocks - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (a.b[mid].tile_start <= t) lo = mid;
    else hi = mid - 1;
  }
  const A2ABlock& B = a.b[lo];
  const int r0 = (t - B.tile_start) * a.rows_per_tile;
  const int tid = threadIdx.x;
  const int64_t nvec = a.hidden / 8;                   // 16-byte vectors; 16 of them per group
  for (int rr = 0; rr < a.rows_per_tile; ++rr) {
    const int k = r0 + rr;
    if (k >= B.rows) break;
    const int64_t sr = B.src_idx[k];
    if (sr < 0 || sr >= B.src_limit) continue;
    const char* src = B.src + sr * a.hidden * 2;
    char* dst = B.dst + static_cast<int64_t>(k) * a.out_row_bytes;
    // nvec and kBlock are multiples of 16, so the 16 lanes of a group are
    // always active together for the shuffles below
    for (int64_t x = tid; x < nvec; x += kBlock) {
      const u32x4 w = ld16(src, x * 16);
      float f[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float v = fabsf(f[i]);
        m = v <= 3.402823466e38f ? fmaxf(m, v) : m;    // finite values only
      }
      m = fmaxf(m, __shfl_xor(m, 8, 16));
      m = fmaxf(m, __shfl_xor(m, 4, 16));
      m = fmaxf(m, __shfl_xor(m, 2, 16));
      m = fmaxf(m, __shfl_xor(m, 1, 16));
      const int kx = fp8_group_exponent(m);
      const float inv = __uint_as_float(static_cast<uint32_t>(127 - kx) << 23);
      uint32_t c0 = 0, c1 = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c0 |= e4m3_code(f[i] * inv) << (8 * i);
        c1 |= e4m3_code(f[4 + i] * inv) << (8 * i);
      }
      reinterpret_cast<uint32_t*>(dst + x * 8)[0] = c0;
      reinterpret_cast<uint32_t*>(dst + x * 8)[1] = c1;
      if ((x & 15) == 0)
        *reinterpret_cast<float*>(dst + a.hidden + (x / 16) * 4) =
            __uint_as_float(static_cast<uint32_t>(kx + 127) << 23);
    }
  }
}

// ----------------------------------------------------------------------------
// stepwise all-reduce: the operations of one algorithm step on float32
// working buffers (one launch per step, messages moved through memory)

__device__ __forceinline__ float round_bf16(float f) { return __uint_as_float(bf16_rne(f) << 16); }

// Four consecutive elements of an operation, vector or scalar access.
__device__ __forceinline__ void step_apply4(const StepLaunchOp& o, int64_t e, bool vec) {
  float* d = static_cast<float*>(o.dst);
  const float* sf = static_cast<const float*>(o.src);
  float x[4], y[4];
  switch (o.kind) {
    case SK_ADD:
    case SK_XADD:
      if (vec) {
        const u32x4 a = ld16(o.src, e * 4), b = ld16(o.dst, e * 4);
        for (int i = 0; i < 4; ++i) { x[i] = __uint_as_float(a[i]); y[i] = __uint_as_float(b[i]); }
      } else {
        for (int i = 0; i < 4; ++i) { x[i] = sf[e + i]; y[i] = d[e + i]; }
      }
      for (int i = 0; i < 4; ++i) y[i] = y[i] + x[i];
      if (vec) {
        const u32x4 r = {__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]), __float_as_uint(y[3])};
        st16(o.dst, e * 4, r);
        if (o.kind == SK_XADD) st16(const_cast<void*>(o.src), e * 4, r);
      } else {
        for (int i = 0; i < 4; ++i) {
          d[e + i] = y[i];
          if (o.kind == SK_XADD) const_cast<float*>(sf)[e + i] = y[i];
        }
      }
      break;
    case SK_COPY:
      if (vec) st16(o.dst, e * 4, ld16(o.src, e * 4));
      else for (int i = 0; i < 4; ++i) d[e + i] = sf[e + i];
      break;
    case SK_NARROW:
      for (int i = 0; i < 4; ++i) d[e + i] = round_bf16(d[e + i]);
      break;
    case SK_WIDEN_BF16: {
      const uint16_t* sb = static_cast<const uint16_t*>(o.src);
      for (int i = 0; i < 4; ++i) d[e + i] = __uint_as_float(uint32_t(sb[e + i]) << 16);
      break;
    }
    default: {  // SK_STORE_BF16
      uint16_t* db = static_cast<uint16_t*>(o.dst);
      for (int i = 0; i < 4; ++i) db[e + i] = static_cast<uint16_t>(bf16_rne(sf[e + i]));
      break;
    }
  }
}

__device__ __forceinline__ void step_apply1(const StepLaunchOp& o, int64_t e) {
  float* d = static_cast<float*>(o.dst);
  const float* sf = static_cast<const float*>(o.src);
  switch (o.kind) {
    case SK_ADD: d[e] = d[e] + sf[e]; break;
    case SK_XADD: { const float v = d[e] + sf[e]; d[e] = v; const_cast<float*>(sf)[e] = v; break; }
    case SK_COPY: d[e] = sf[e]; break;
    case SK_NARROW: d[e] = round_bf16(d[e]); break;
    case SK_WIDEN_BF16: d[e] = __uint_as_float(uint32_t(static_cast<const uint16_t*>(o.src)[e]) << 16); break;
    default: static_cast<uint16_t*>(o.dst)[e] = static_cast<uint16_t>(bf16_rne(sf[e])); break;
  }
}

__global__ __launch_bounds__(kBlock) void step_kernel(const StepArgs a) {
  const int t = blockIdx.x;
  int lo = 0, hi = a.nops - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (a.op[mid].tile_start <= t) lo = mid;
    else hi = mid - 1;
  }
  const StepLaunchOp& o = a.op[lo];
  const int64_t e0 = static_cast<int64_t>(t - o.tile_start) * kStepTile;
  const int64_t e1 = o.count < e0 + kStepTile ? o.count : e0 + kStepTile;
  // float32 sides move as 16-byte vectors when both ends are aligned
  const bool vec = (o.kind == SK_ADD || o.kind == SK_XADD || o.kind == SK_COPY) &&
                   ((reinterpret_cast<uintptr_t>(o.src) | reinterpret_cast<uintptr_t>(o.dst)) & 15u) == 0;
  const int64_t groups = (e1 - e0) / 4;
  for (int64_t g = threadIdx.x; g < groups; g += kBlock) step_apply4(o, e0 + 4 * g, vec);
  const int64_t tail = e0 + 4 * groups + threadIdx.x;
  if (tail < e1) step_apply1(o, tail);
}

// ----------------------------------------------------------------------------
// plain copy: the streaming ceiling the collectives are measured against

__global__ __launch_bounds__(kBlock) void copy_kernel(const void* src, void* dst, int64_t nvec) {
  constexpr int V = 4;
  const int64_t v0 = static_cast<int64_t>(blockIdx.x) * (V * kBlock) + threadIdx.x;
  u32x4 x[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int64_t v = v0 + j * kBlock;
    x[j] = v < nvec ? ld16(src, v * 16) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int64_t v = v0 + j * kBlock;
    if (v < nvec) st16(dst, v * 16, x[j]);
  }
}

// ----------------------------------------------------------------------------
// launch helpers

template <class K, class Arg>
hipError_t launch(K kernel, dim3 grid, const Arg& arg, hipStream_t stream) {
  void* args[] = {const_cast<Arg*>(&arg)};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, dim3(kBlock), args, 0, stream);
}

// 16-byte vectors per thread of the reduce kernel (all are loaded before the
// first add). Build-time override: -DVCOLL_V_P8=<n> for p = 8.
#ifndef VCOLL_V_P8
#define VCOLL_V_P8 2
#endif
template <int P>
constexpr int vectors_per_thread() {
  return P == 0 ? 1 : (P <= 4 ? 4 : (P <= 8 ? VCOLL_V_P8 : 1));
}

// Workgroups from which a launch paces its stores (see VCOLL_STORE_SLEEP).
#ifndef VCOLL_PACE_MIN_GROUPS
#define VCOLL_PACE_MIN_GROUPS 2048
#endif

template <int D, int ALGO, bool RS, int P>
hipError_t launch_reduce_p(const ReduceArgs& a, int64_t max_chunk, int chunks, hipStream_t stream) {
  constexpr int V = vectors_per_thread<P>();
  constexpr int VE = Storage<D>::kVE;
  const int64_t per_tile = static_cast<int64_t>(V) * kBlock * VE;
  const int64_t tiles = (max_chunk + per_tile - 1) / per_tile;
  if (tiles == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(tiles), chunks);
  ReduceArgs args = a;
  args.pace = !RS && tiles * a.p >= VCOLL_PACE_MIN_GROUPS;
  if constexpr (P > 0) {
    // the compile-time variant carries the pacing (and its load pipeline)
    if (args.pace) return launch(reduce_kernel<D, ALGO, P, V, RS, true>, grid, args, stream);
    return launch(reduce_kernel<D, ALGO, P, V, RS, false>, grid, args, stream);
  } else {
    return launch(reduce_kernel<D, ALGO, P, V, RS, false>, grid, args, stream);
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

}  // namespace

hipError_t launch_reduce(const ReduceArgs& a, vcoll_dtype dtype, vcoll_algo algo, bool scatter,
                         int64_t max_chunk, int chunks, hipStream_t stream) {
  if (dtype == VCOLL_F32) return launch_reduce_dtype<VCOLL_F32>(a, algo, scatter, max_chunk, chunks, stream);
  return launch_reduce_dtype<VCOLL_BF16>(a, algo, scatter, max_chunk, chunks, stream);
}

hipError_t launch_broadcast(const BcastArgs& a, vcoll_dtype dtype, hipStream_t stream) {
  constexpr int V = 2;
  const int ES = dtype == VCOLL_F32 ? 4 : 2;
  const int64_t per_tile = static_cast<int64_t>(V) * kBlock * (16 / ES);
  const int64_t tiles = (a.n + per_tile - 1) / per_tile;
  if (tiles == 0 || a.q == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(tiles));
  const bool pace = a.vec && tiles >= VCOLL_PACE_MIN_GROUPS;
  if (ES == 4) {
    if (pace) return launch(broadcast_kernel<4, V, true>, grid, a, stream);
    return launch(broadcast_kernel<4, V, false>, grid, a, stream);
  }
  if (pace) return launch(broadcast_kernel<2, V, true>, grid, a, stream);
  return launch(broadcast_kernel<2, V, false>, grid, a, stream);
}

hipError_t launch_all_gather(const GatherArgs& a, vcoll_dtype dtype, hipStream_t stream) {
  constexpr int V = 2;
  const int ES = dtype == VCOLL_F32 ? 4 : 2;
  const int64_t per_tile = static_cast<int64_t>(V) * kBlock * (16 / ES);
  const int64_t tiles = (a.m + per_tile - 1) / per_tile;
  if (tiles == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(tiles), a.p);
  if (ES == 4) return launch(all_gather_kernel<4, V>, grid, a, stream);
  return launch(all_gather_kernel<2, V>, grid, a, stream);
}

hipError_t launch_dispatch_fp8(const Fp8Args& a, int32_t tiles, hipStream_t stream) {
  if (tiles == 0) return hipSuccess;
  return launch(dispatch_fp8_kernel, dim3(static_cast<unsigned>(tiles)), a, stream);
}

hipError_t launch_all_to_all(const A2AArgs& a, int32_t tiles, hipStream_t stream) {
  if (tiles == 0) return hipSuccess;
  return launch(all_to_all_kernel, dim3(static_cast<unsigned>(tiles)), a, stream);
}

namespace {

template <int D, int NN, int LL>
hipError_t launch_hier_shape(const HierArgs& a, dim3 grid, bool large, hipStream_t stream) {
  if (large) return launch(hier_kernel<D, NN, LL, true>, grid, a, stream);
  return launch(hier_kernel<D, NN, LL, false>, grid, a, stream);
}

template <int D>
hipError_t launch_hier_dtype(const HierArgs& a, dim3 grid, bool large, hipStream_t stream) {
  const int N = a.nodes, L = a.local;
  if (N == 2 && L == 8) return launch_hier_shape<D, 2, 8>(a, grid, large, stream);
  if (N == 4 && L == 4) return launch_hier_shape<D, 4, 4>(a, grid, large, stream);
  if (N == 4 && L == 8) return launch_hier_shape<D, 4, 8>(a, grid, large, stream);
  if (N == 2 && L == 4) return launch_hier_shape<D, 2, 4>(a, grid, large, stream);
  if (N == 8 && L == 8) return launch_hier_shape<D, 8, 8>(a, grid, large, stream);
  if (N == 4 && L == 2) return launch_hier_shape<D, 4, 2>(a, grid, large, stream);
  return launch(hier_kernel<D, 0, 0, false>, grid, a, stream);
}

}  // namespace

hipError_t launch_hierarchical(const HierArgs& a, vcoll_dtype dtype, int64_t max_segment, hipStream_t stream) {
  const int64_t per_tile = static_cast<int64_t>(kBlock) * (dtype == VCOLL_F32 ? 4 : 8);
  const int64_t tiles = (max_segment + per_tile - 1) / per_tile;
  if (tiles == 0) return hipSuccess;
  const int p = a.nodes * a.local;
  const dim3 grid(static_cast<unsigned>(tiles), p);
  const bool large = tiles * p >= VCOLL_PACE_MIN_GROUPS;
  if (dtype == VCOLL_F32) return launch_hier_dtype<VCOLL_F32>(a, grid, large, stream);
  return launch_hier_dtype<VCOLL_BF16>(a, grid, large, stream);
}

hipError_t launch_step(const StepArgs& a, int32_t tiles, hipStream_t stream) {
  if (tiles == 0) return hipSuccess;
  return launch(step_kernel, dim3(static_cast<unsigned>(tiles)), a, stream);
}

hipError_t launch_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream) {
  const int64_t nvec = bytes / 16;
  const int64_t per_tile = 4LL * kBlock;
  const int64_t tiles = (nvec + per_tile - 1) / per_tile;
  if (tiles == 0) return hipSuccess;
  void* args[] = {const_cast<const void**>(&src), &dst, const_cast<int64_t*>(&nvec)};
  return hipLaunchKernel(reinterpret_cast<const void*>(copy_kernel), dim3(static_cast<unsigned>(tiles)),
                         dim3(kBlock), args, 0, stream);
}

}  // namespace vcoll
