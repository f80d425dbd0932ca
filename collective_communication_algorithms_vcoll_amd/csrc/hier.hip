// The fused hierarchical / 2D all-reduce kernel of libvcoll for gfx950.
#include "device.h"
#include "hier.h"

namespace vcoll {
namespace {

using namespace dev;

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

// Threads per workgroup by shape (p = NN x LL compiled in; a run-time shape
// takes four waves). Measured on MI355X against four waves: p = 16, two
// waves took the 4 x 4 hierarchy of 16 x 192 MiB bf16 from 1206-1213 to 1163
// us and of 16 x 16 MiB float32 from 126-127 to 121-122 us (2 x 8 within 1
// %); p = 32 (4 x 8 x 16 MiB float32) 234-236 -> 222 us with two waves; p =
// 64 (8 x 8 x 8 MiB) 243-245 -> 220-221 us with one (two waves: 246); p = 8
// keeps four, 0.5-1.5 % ahead on the 25 MiB bucket (two waves won 3.5 % at
// 80 MiB).
template <int NN, int LL>
constexpr int hier_block() {
  return NN * LL == 16 || NN * LL == 32 ? 128 : (NN * LL == 64 ? 64 : kBlock);
}

template <int D, int NN, int LL, bool LARGE>
__global__ __launch_bounds__((hier_block<NN, LL>())) void hier_kernel(const HierArgs a) {
  constexpr int BS = hier_block<NN, LL>();
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
    const int64_t v = static_cast<int64_t>(blockIdx.x) * BS + tid;
    if (static_cast<int64_t>(blockIdx.x) * BS < nvec) {
      const int64_t boff = (e_base + v * VE) * ES;
      if ((static_cast<int64_t>(blockIdx.x) + 1) * BS <= nvec) {
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
    const int64_t e0 = static_cast<int64_t>(blockIdx.x) * (BS * VE);
#pragma unroll 1
    for (int k = 0; k < VE; ++k) {
      const int64_t i = e0 + k * BS + tid;
      if (i < cnt) hier_one<D>(a, N, Lc, l, j, off + i);
    }
  }
}

// ----------------------------------------------------------------------------
// launchers

// Grid (tiles of BS threads x VE elements, segment); large grids pace their
// stores (VCOLL_PACE_MIN_GROUPS counted in four-wave workgroups).
template <int D, int NN, int LL>
hipError_t launch_hier_shape(const HierArgs& a, int64_t max_segment, hipStream_t stream) {
  constexpr int BS = hier_block<NN, LL>();
  constexpr int64_t per_tile = static_cast<int64_t>(BS) * Storage<D>::kVE;
  const int64_t tiles = (max_segment + per_tile - 1) / per_tile;
  if (tiles == 0) return hipSuccess;
  const int p = a.nodes * a.local;
  const dim3 grid(static_cast<unsigned>(tiles), p);
  const bool large = tiles * p * BS >= static_cast<int64_t>(VCOLL_PACE_MIN_GROUPS) * kBlock;
  if constexpr (NN > 0) {
    if (large) return launch(hier_kernel<D, NN, LL, true>, grid, BS, a, stream);
  }
  return launch(hier_kernel<D, NN, LL, false>, grid, BS, a, stream);
}

template <int D>
hipError_t launch_hier_dtype(const HierArgs& a, int64_t max_segment, hipStream_t stream) {
  const int N = a.nodes, L = a.local;
  if (N == 2 && L == 8) return launch_hier_shape<D, 2, 8>(a, max_segment, stream);
  if (N == 4 && L == 4) return launch_hier_shape<D, 4, 4>(a, max_segment, stream);
  if (N == 4 && L == 8) return launch_hier_shape<D, 4, 8>(a, max_segment, stream);
  if (N == 2 && L == 4) return launch_hier_shape<D, 2, 4>(a, max_segment, stream);
  if (N == 8 && L == 8) return launch_hier_shape<D, 8, 8>(a, max_segment, stream);
  if (N == 4 && L == 2) return launch_hier_shape<D, 4, 2>(a, max_segment, stream);
  return launch_hier_shape<D, 0, 0>(a, max_segment, stream);
}

}  // namespace

hipError_t launch_hierarchical(const HierArgs& a, vcoll_dtype dtype, int64_t max_segment, hipStream_t stream) {
  if (dtype == VCOLL_F32) return launch_hier_dtype<VCOLL_F32>(a, max_segment, stream);
  return launch_hier_dtype<VCOLL_BF16>(a, max_segment, stream);
}

}  // namespace vcoll
