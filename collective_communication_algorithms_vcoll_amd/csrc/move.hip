// Data-movement kernels of libvcoll for gfx950: all-gather fan-out,
// broadcast, variable-split all-to-all and the FP8 and token-major MoE
// dispatches and combine. Nothing here adds; every byte is read once and
// written to its destinations.
#include "device.h"
#include "move.h"

namespace vcoll {
namespace {

using namespace dev;

// ----------------------------------------------------------------------------
// store of a fan-out (one load, several copies stored): streamed past every
// cache level, or cached. The streamed form is a buffer store whose resource
// base is the workgroup's tile in the destination (uniform), the lane's
// place in it a 32-bit offset. Measured on MI355X (launches that write up to
// 1 GiB): with the source still in the Infinity Cache, sc0|nt|sc1 stores ran
// 7-19% faster than nt-only global stores (an all-gather of 3.125 MiB f32
// blocks at p = 8 and a 25 MiB broadcast to 8 buffers +19%, 1 MiB blocks at
// p = 8 +7%); with the source read from HBM the two are within 2% (64 KiB
// bf16 blocks at p = 72 +2%), and every fan-out shape tried -- one load then
// all stores per tile, or a whole chip-wide read phase before the writes --
// runs at 5.4-5.5 TB/s.
// Where the workgroups' tiles are not whole 128-byte lines of the outputs
// (receive buffers off a line, or all-gather blocks that are not a whole
// number of lines), neighbouring workgroups write parts of one line, and
// cached stores let L2 merge them: with the source read from HBM, 9-20%
// faster than the streamed ones (p = 8 blocks of 819,204 f32 57.1 -> 52.3
// us, a 25 MiB broadcast to rows 16 bytes off a line 57.2 -> 51.1 us, p = 72
// bf16 blocks of 32,776 elements 98.7 -> 81.9 us), within 1.5% on aligned
// tiles. The large fan-outs write faster through L2 with cached stores
// too: the all-gather and broadcast beyond 1 GiB written (4-6%) and the bf16
// token-major MoE dispatch, 8 copies of each token row (3%; its FP8 codes
// 2.2%). One-to-one movers (all-to-all, combine, the row-major FP8 codes)
// lost 1-8% with cached stores and keep streaming ones.

template <bool NT>
__device__ __forceinline__ void fan_st16(void* base, int64_t tile_off, int lane_off, u32x4 v) {
  if constexpr (NT) {
    __builtin_amdgcn_raw_buffer_store_b128(v, raw_rsrc(base, tile_off, 0x7fffffff), lane_off, 0, kPolicyThrough);
  } else {
    *reinterpret_cast<u32x4*>(static_cast<char*>(base) + tile_off + lane_off) = v;
  }
}

// ----------------------------------------------------------------------------
// all-gather: block i of every output is a copy of input i

template <int ES, int V, int BS, bool NT>
__global__ __launch_bounds__(BS) void all_gather_kernel(const GatherArgs a) {
  const int i = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t bytes = a.m * ES;
  const int64_t dst_off = i * bytes;
  const void* src = a.ptr.src[i];
  if (a.vec) {
    const int64_t nvec = bytes / 16;
    const int64_t v0 = static_cast<int64_t>(blockIdx.x) * (V * BS) + tid;
    const int64_t tile_off = dst_off + static_cast<int64_t>(blockIdx.x) * (V * BS) * 16;
    u32x4 x[V];
    bool valid[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int64_t v = v0 + j * BS;
      valid[j] = v < nvec;
      x[j] = valid[j] ? ld16(src, v * 16) : u32x4{0, 0, 0, 0};
    }
    for (int r = 0; r < a.p; ++r) {
#pragma unroll
      for (int j = 0; j < V; ++j)
        if (valid[j]) fan_st16<NT>(a.ptr.dst[r], tile_off, (tid + j * BS) * 16, x[j]);
    }
  } else {
    using E = typename std::conditional<ES == 4, uint32_t, uint16_t>::type;
    constexpr int VE = 16 / ES;
    const int64_t e0 = static_cast<int64_t>(blockIdx.x) * (V * BS * VE) + tid;
#pragma unroll 1
    for (int j = 0; j < V * VE; ++j) {
      const int64_t e = e0 + j * BS;
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

template <int ES, int V, int BS, bool NT>
__global__ __launch_bounds__(BS) void broadcast_kernel(const BcastArgs a) {
  using E = typename std::conditional<ES == 4, uint32_t, uint16_t>::type;
  constexpr int VE = 16 / ES;
  static_assert(BS >= VE, "workgroup 0 copies the n mod VE tail elements, one per thread");
  const int tid = threadIdx.x;
  if (a.vec) {
    const int64_t nvec = a.n / VE;
    const int64_t v0 = static_cast<int64_t>(blockIdx.x) * (V * BS) + tid;
    const int64_t tile_off = static_cast<int64_t>(blockIdx.x) * (V * BS) * 16;
    u32x4 x[V];
    bool valid[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int64_t v = v0 + j * BS;
      valid[j] = v < nvec;
      x[j] = valid[j] ? ld16(a.src, v * 16) : u32x4{0, 0, 0, 0};
    }
    for (int r = 0; r < a.q; ++r) {
#pragma unroll
      for (int j = 0; j < V; ++j)
        if (valid[j]) fan_st16<NT>(a.dst[r], tile_off, (tid + j * BS) * 16, x[j]);
    }
    // the last n mod VE elements
    if (blockIdx.x == 0 && tid < a.n - nvec * VE) {
      const int64_t e = nvec * VE + tid;
      const E w = static_cast<const E*>(a.src)[e];
      for (int r = 0; r < a.q; ++r) static_cast<E*>(a.dst[r])[e] = w;
    }
  } else {
    const int64_t e0 = static_cast<int64_t>(blockIdx.x) * (V * BS * VE) + tid;
#pragma unroll 1
    for (int j = 0; j < V * VE; ++j) {
      const int64_t e = e0 + j * BS;
      if (e < a.n) {
        const E w = static_cast<const E*>(a.src)[e];
        for (int r = 0; r < a.q; ++r) static_cast<E*>(a.dst[r])[e] = w;
      }
    }
  }
}

// ----------------------------------------------------------------------------
// all-to-all: workgroup t moves rows_per_tile rows of one (i -> j) block

template <int BS>
__global__ __launch_bounds__(BS) void all_to_all_kernel(const A2AArgs a) {
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
  if (a.vec && !B.src_idx && !B.dst_idx) {
    // rows contiguous on both sides: the tile's rows are one run of bytes,
    // copied with every load of a round in flight before its stores
    const int k1 = r0 + a.rows_per_tile < B.rows ? r0 + a.rows_per_tile : B.rows;
    const char* src = B.src + static_cast<int64_t>(r0) * a.row_bytes;
    char* dst = B.dst + static_cast<int64_t>(r0) * a.row_bytes;
    const int64_t nvec = static_cast<int64_t>(k1 - r0) * a.row_bytes / 16;
    constexpr int U = 8;
    for (int64_t x0 = tid; x0 < nvec; x0 += U * BS) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t x = x0 + u * BS;
        v[u] = x < nvec ? ld16(src, x * 16) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t x = x0 + u * BS;
        if (x < nvec) st16(dst, x * 16, v[u]);
      }
    }
    return;
  }
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
      for (int64_t x0 = tid; x0 < nvec; x0 += U * BS) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t x = x0 + u * BS;
          v[u] = x < nvec ? ld16(src, x * 16) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t x = x0 + u * BS;
          if (x < nvec) st16(dst, x * 16, v[u]);
        }
      }
    } else if (a.esize == 4) {
      for (int64_t x = tid; x < a.row_bytes / 4; x += BS)
        reinterpret_cast<uint32_t*>(dst)[x] = reinterpret_cast<const uint32_t*>(src)[x];
    } else if (a.esize == 2) {
      for (int64_t x = tid; x < a.row_bytes / 2; x += BS)
        reinterpret_cast<uint16_t*>(dst)[x] = reinterpret_cast<const uint16_t*>(src)[x];
    } else {
      for (int64_t x = tid; x < a.row_bytes; x += BS)
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

// Quantise 16 bfloat16 values (two 16-byte vectors) of a 128-element group
// spread over 8 consecutive lanes: the group's amax by shuffles within the 8
// lanes (all 8 must call this together), its power-of-two scale, and the 16
// codes packed little-endian, element k in byte k of the 16-byte result.
__device__ __forceinline__ void quantise16(const u32x4 w0, const u32x4 w1, u32x4& codes, float& scale) {
  float f[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w0[i] << 16);
    f[2 * i + 1] = __uint_as_float(w0[i] & 0xFFFF0000u);
    f[8 + 2 * i] = __uint_as_float(w1[i] << 16);
    f[8 + 2 * i + 1] = __uint_as_float(w1[i] & 0xFFFF0000u);
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float v = fabsf(f[i]);
    m = v <= 3.402823466e38f ? fmaxf(m, v) : m;        // finite values only
  }
  m = fmaxf(m, __shfl_xor(m, 4, 8));
  m = fmaxf(m, __shfl_xor(m, 2, 8));
  m = fmaxf(m, __shfl_xor(m, 1, 8));
  const int kx = fp8_group_exponent(m);
  const float inv = __uint_as_float(static_cast<uint32_t>(127 - kx) << 23);
  // Every scaled value is exact and |x * 2^-k| <= 448, so gfx950's fp32 ->
  // E4M3 pack (OCP format, round to nearest even under the default mode)
  // gives the code directly. It writes NaN with the input's sign (0xFF for
  // a negative NaN or -inf), so lanes holding a non-finite value rewrite
  // those bytes as 0x7F.
  bool nonfinite = false;
#pragma unroll
  for (int i = 0; i < 16; ++i) nonfinite |= !(fabsf(f[i]) <= 3.402823466e38f);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * w] * inv, f[4 * w + 1] * inv, 0, false);
    codes[w] = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * w + 2] * inv, f[4 * w + 3] * inv, lo, true);
  }
  if (nonfinite) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (!(fabsf(f[i]) <= 3.402823466e38f))
        codes[i / 4] = (codes[i / 4] & ~(0xFFu << (8 * (i % 4)))) | (0x7Fu << (8 * (i % 4)));
    }
  }
  scale = __uint_as_float(static_cast<uint32_t>(kx + 127) << 23);
}

// Store one lane's 16 codes (elements 16y .. 16y+15 of the row) and, from the
// first lane of each group, the group's scale. CACHED: 16-byte code stores
// through L2, which on MI355X made the token-major dispatch (8 copies of each
// quantised row, rows of 7392 bytes that share cache lines) 2.2 % faster and
// the row-major one (each row written once) 5 % slower than streaming ones.
template <bool CACHED>
__device__ __forceinline__ void store_codes(char* row, int64_t hidden, int64_t y, const u32x4 codes, float scale,
                                            bool vec) {
  if (vec) {
    if constexpr (CACHED) *reinterpret_cast<u32x4*>(row + y * 16) = codes;
    else st16(row, y * 16, codes);
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) __builtin_nontemporal_store(codes[w], reinterpret_cast<uint32_t*>(row + y * 16) + w);
  }
  // A wave writes 32 bytes of the row's scale tail; ordinary (cached) stores
  // let L2 merge those pieces into whole lines before they reach HBM, where
  // streaming stores of them cost 13 % on the token-major dispatch.
  if ((y & 7) == 0) *reinterpret_cast<float*>(row + hidden + (y / 8) * 4) = scale;
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
  for (int rr = 0; rr < a.rows_per_tile; ++rr) {
    const int k = r0 + rr;
    if (k >= B.rows) break;
    const int64_t sr = B.src_idx[k];
    if (sr < 0 || sr >= B.src_limit) continue;
    const char* src = B.src + sr * a.hidden * 2;
    char* dst = B.dst + static_cast<int64_t>(k) * a.out_row_bytes;
    // hidden / 16 lane tasks of 16 elements, a multiple of 8, and kBlock a
    // multiple of 8: the 8 lanes of a group are always active together
    const int64_t nq = a.hidden / 16;
    for (int64_t y = tid; y < nq; y += kBlock) {
      u32x4 codes;
      float scale;
      quantise16(ld16(src, y * 32), ld16(src, y * 32 + 16), codes, scale);
      store_codes<false>(dst, a.hidden, y, codes, scale, a.vec_out);
    }
  }
}

// ----------------------------------------------------------------------------
// token-major MoE dispatch: each token row of each sending rank is read once
// and written to the received-row slot of every (token, chosen expert) pair,
// copied as it is or quantised to FP8 once for all its copies

constexpr int kPushUnroll = 4;     // 16-byte vectors in flight per thread (a 7168 bf16 row is 3.5)
constexpr int kPushFp8Block = 512;  // threads per workgroup of the FP8 token-major dispatch

// bf16 token rows longer than this many 16-byte vectors are cut into
// segments of it, one per one-wave workgroup (the workgroups of one token
// then write its copies in parallel): on the 7168-element MoE workload,
// seven 2 KiB segments took the dispatch from 836 to 775 us on MI355X.
constexpr int kPushSegVec = 128;

template <bool FP8, int BS>
__global__ __launch_bounds__(BS) void dispatch_push_kernel(const PushArgs a) {
  const int tid = threadIdx.x;
  const int i = blockIdx.y;                                    // sending rank
  const int seg = static_cast<int>(blockIdx.x % a.segments);   // segment of every row of the tile
  const int64_t t0 = static_cast<int64_t>(blockIdx.x / a.segments) * a.tokens_per_tile;
  for (int64_t t = t0; t < t0 + a.tokens_per_tile && t < a.tokens; ++t) {
    const char* src = static_cast<const char*>(a.table[i]) + t * a.row_bytes;
    const int32_t* slot = a.slots[i] + 2 * t * a.topk;
    // destination k of this token (uniform across the workgroup), or null
    auto dest = [&](int k) -> char* {
      const int j = slot[2 * k], r = slot[2 * k + 1];
      if (j < 0 || j >= a.p || r < 0 || r >= a.recv_rows[j]) return nullptr;
      return static_cast<char*>(a.recv[j]) + static_cast<int64_t>(r) * a.out_row_bytes;
    };
    if constexpr (FP8) {
      // hidden / 16 lane tasks, a multiple of 8: each 8-lane group is whole
      const int64_t nq = a.hidden / 16;
      for (int64_t y0 = tid; y0 < nq; y0 += kPushUnroll / 2 * BS) {
        u32x4 w[kPushUnroll];
#pragma unroll
        for (int u = 0; u < kPushUnroll / 2; ++u) {
          const int64_t y = y0 + u * BS;
          w[2 * u] = y < nq ? ld16(src, y * 32) : u32x4{0, 0, 0, 0};
          w[2 * u + 1] = y < nq ? ld16(src, y * 32 + 16) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kPushUnroll / 2; ++u) {
          const int64_t y = y0 + u * BS;
          if (y >= nq) break;                        // uniform over each 8-lane group
          u32x4 codes;
          float scale;
          quantise16(w[2 * u], w[2 * u + 1], codes, scale);
          for (int k = 0; k < a.topk; ++k) {
            char* d = dest(k);
            if (d) store_codes<true>(d, a.hidden, y, codes, scale, a.vec_out);
          }
        }
      }
    } else if (a.vec) {
      const int64_t nall = a.row_bytes / 16;
      const int64_t per = (nall + a.segments - 1) / a.segments;
      const int64_t nvec = (seg + 1) * per < nall ? (seg + 1) * per : nall;
      for (int64_t x0 = seg * per + tid; x0 < nvec; x0 += kPushUnroll * BS) {
        u32x4 v[kPushUnroll];
#pragma unroll
        for (int u = 0; u < kPushUnroll; ++u) {
          const int64_t x = x0 + u * BS;
          v[u] = x < nvec ? ld16(src, x * 16) : u32x4{0, 0, 0, 0};
        }
        for (int k = 0; k < a.topk; ++k) {
          char* d = dest(k);
          if (!d) continue;
#pragma unroll
          for (int u = 0; u < kPushUnroll; ++u) {
            const int64_t x = x0 + u * BS;
            if (x < nvec) fan_st16<false>(d, x * 16, 0, v[u]);
          }
        }
      }
    } else {
      for (int64_t x = tid; x < a.row_bytes / 2; x += BS) {
        const uint16_t v = reinterpret_cast<const uint16_t*>(src)[x];
        for (int k = 0; k < a.topk; ++k) {
          char* d = dest(k);
          if (d) reinterpret_cast<uint16_t*>(d)[x] = v;
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// token-major MoE combine: the reverse all-to-all of the dispatch, written in
// (token, slot) order. Each output row pulls its expert-output row, so the
// writes stream through each rank's output while the reads gather; the
// scattering form of the same permutation writes rows in send order instead.

constexpr int kCombineRows = 2;    // output rows whose loads are in flight together
// Rows longer than this many 16-byte vectors are cut into segments of it,
// one per one-wave workgroup: fourteen 1 KiB segments took the MoE
// workload's combine from 1420 to 1337 us on MI355X.
constexpr int kPullSegVec = 64;

template <int BS>
__global__ __launch_bounds__(BS) void combine_pull_kernel(const CombineArgs a) {
  const int tid = threadIdx.x;
  const int i = blockIdx.y;                                    // rank that owns the tokens
  const int seg = static_cast<int>(blockIdx.x % a.segments);
  const int64_t total = a.tokens * a.topk;
  const int64_t x_begin = static_cast<int64_t>(blockIdx.x / a.segments) * a.tokens_per_tile * a.topk;
  const int64_t x_end = x_begin + static_cast<int64_t>(a.tokens_per_tile) * a.topk < total
                            ? x_begin + static_cast<int64_t>(a.tokens_per_tile) * a.topk
                            : total;
  const int32_t* slot = a.slots[i];
  char* out = static_cast<char*>(a.out[i]);
  // the expert-output row of output row x (uniform across the workgroup), or null
  auto source = [&](int64_t x) -> const char* {
    const int j = slot[2 * x], r = slot[2 * x + 1];
    if (j < 0 || j >= a.p || r < 0 || r >= a.src_rows[j]) return nullptr;
    return static_cast<const char*>(a.src[j]) + static_cast<int64_t>(r) * a.row_bytes;
  };
  for (int64_t x = x_begin; x < x_end; x += kCombineRows) {
    const char* src[kCombineRows];
#pragma unroll
    for (int q = 0; q < kCombineRows; ++q) src[q] = x + q < x_end ? source(x + q) : nullptr;
    if (a.vec) {
      const int64_t nall = a.row_bytes / 16;
      const int64_t per = (nall + a.segments - 1) / a.segments;
      const int64_t nvec = (seg + 1) * per < nall ? (seg + 1) * per : nall;
      for (int64_t v0 = seg * per + tid; v0 < nvec; v0 += kPushUnroll * BS) {
        u32x4 w[kCombineRows][kPushUnroll];
#pragma unroll
        for (int q = 0; q < kCombineRows; ++q)
#pragma unroll
          for (int u = 0; u < kPushUnroll; ++u) {
            const int64_t v = v0 + u * BS;
            w[q][u] = src[q] && v < nvec ? ld16(src[q], v * 16) : u32x4{0, 0, 0, 0};
          }
#pragma unroll
        for (int q = 0; q < kCombineRows; ++q)
#pragma unroll
          for (int u = 0; u < kPushUnroll; ++u) {
            const int64_t v = v0 + u * BS;
            if (src[q] && v < nvec) st16(out + (x + q) * a.row_bytes, v * 16, w[q][u]);
          }
      }
    } else {
      for (int64_t e = tid; e < a.row_bytes / 2; e += BS) {
#pragma unroll
        for (int q = 0; q < kCombineRows; ++q)
          if (src[q])
            reinterpret_cast<uint16_t*>(out + (x + q) * a.row_bytes)[e] = reinterpret_cast<const uint16_t*>(src[q])[e];
      }
    }
  }
}

// Fan-out shape of the all-gather and the broadcast, chosen by the bytes a
// launch writes; both use one-wave workgroups. Measured on MI355X against
// four-wave workgroups with two streaming-stored vectors per thread: up to
// kFanLargeBytes, four vectors per thread with streaming stores gained 3-12%
// (all-gathers of 64 KiB blocks at p = 72, of 1 MiB and 3.125 MiB blocks at
// p = 8); beyond it, one vector per thread with cached stores gained 4-6%
// (the p = 16 all-gather of 12 MiB blocks, a 192 MiB broadcast to 16
// buffers), where the four-vector form lost 3%.
constexpr int kFanBlock = 64;
constexpr int64_t kFanLargeBytes = int64_t(1) << 30;

template <int ES, int V, class Args, class Kernel>
hipError_t launch_fan(Kernel kernel, int64_t elems, unsigned blocks_y, const Args& a, hipStream_t stream) {
  const int64_t per_tile = static_cast<int64_t>(V) * kFanBlock * (16 / ES);
  const int64_t tiles = (elems + per_tile - 1) / per_tile;
  if (tiles == 0) return hipSuccess;
  if (tiles > int64_t(UINT32_MAX)) return hipErrorInvalidConfiguration;   // beyond any grid (and any HBM)
  return launch(kernel, dim3(static_cast<unsigned>(tiles), blocks_y), kFanBlock, a, stream);
}

template <int ES>
hipError_t launch_broadcast_es(const BcastArgs& a, hipStream_t stream) {
  if (a.n * ES > kFanLargeBytes / a.q)                     // bytes written, without overflow
    return launch_fan<ES, 1>(broadcast_kernel<ES, 1, kFanBlock, false>, a.n, 1, a, stream);
  if (!a.lines) return launch_fan<ES, 4>(broadcast_kernel<ES, 4, kFanBlock, false>, a.n, 1, a, stream);
  return launch_fan<ES, 4>(broadcast_kernel<ES, 4, kFanBlock, true>, a.n, 1, a, stream);
}

template <int ES>
hipError_t launch_all_gather_es(const GatherArgs& a, hipStream_t stream) {
  if (a.m * ES * a.p > kFanLargeBytes / a.p)
    return launch_fan<ES, 1>(all_gather_kernel<ES, 1, kFanBlock, false>, a.m, a.p, a, stream);
  if (!a.lines) return launch_fan<ES, 4>(all_gather_kernel<ES, 4, kFanBlock, false>, a.m, a.p, a, stream);
  return launch_fan<ES, 4>(all_gather_kernel<ES, 4, kFanBlock, true>, a.m, a.p, a, stream);
}

}  // namespace

hipError_t launch_broadcast(const BcastArgs& a, vcoll_dtype dtype, hipStream_t stream) {
  if (a.q == 0) return hipSuccess;
  return dtype == VCOLL_F32 ? launch_broadcast_es<4>(a, stream) : launch_broadcast_es<2>(a, stream);
}

hipError_t launch_all_gather(const GatherArgs& a, vcoll_dtype dtype, hipStream_t stream) {
  return dtype == VCOLL_F32 ? launch_all_gather_es<4>(a, stream) : launch_all_gather_es<2>(a, stream);
}

hipError_t launch_dispatch_fp8(const Fp8Args& a, int32_t tiles, hipStream_t stream) {
  if (tiles == 0) return hipSuccess;
  return launch(dispatch_fp8_kernel, dim3(static_cast<unsigned>(tiles)), a, stream);
}

int32_t push_segments(int64_t row_bytes, bool fp8, bool vec) {
  if (fp8 || !vec) return 1;
  const int64_t nvec = row_bytes / 16;
  return static_cast<int32_t>(nvec > kPushSegVec ? (nvec + kPushSegVec - 1) / kPushSegVec : 1);
}

int32_t pull_segments(int64_t row_bytes, bool vec) {
  if (!vec) return 1;
  const int64_t nvec = row_bytes / 16;
  return static_cast<int32_t>(nvec > kPullSegVec ? (nvec + kPullSegVec - 1) / kPullSegVec : 1);
}

hipError_t launch_dispatch_push(const PushArgs& a, bool fp8, hipStream_t stream) {
  const int64_t tiles = (a.tokens + a.tokens_per_tile - 1) / a.tokens_per_tile;
  if (tiles == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(tiles), a.p);
  // FP8: one 16-element quantisation task per thread for rows up to 8192
  // elements. On the 7168-element workload 512-thread workgroups measured
  // 3% faster than 256 with 8 destinations per token and 2% slower with the
  // deduplicated plan's ~3; 1024 gained 6% and lost 20%. bf16 copies lost
  // 2.5% with 512 or 1024 and keep 256.
  if (fp8) return launch(dispatch_push_kernel<true, kPushFp8Block>, grid, kPushFp8Block, a, stream);
  if (a.segments > 1) {
    const dim3 seg_grid(static_cast<unsigned>(tiles * a.segments), a.p);
    return launch(dispatch_push_kernel<false, 64>, seg_grid, 64, a, stream);
  }
  return launch(dispatch_push_kernel<false, kBlock>, grid, kBlock, a, stream);
}

hipError_t launch_combine_pull(const CombineArgs& a, hipStream_t stream) {
  const int64_t tiles = (a.tokens + a.tokens_per_tile - 1) / a.tokens_per_tile;
  if (tiles == 0) return hipSuccess;
  // 512 threads per token's output rows: 2% faster than 256 on the MoE
  // workload (1024: 1% slower)
  constexpr int kPullBlock = 512;
  if (a.segments > 1)
    return launch(combine_pull_kernel<64>, dim3(static_cast<unsigned>(tiles * a.segments), a.p), 64, a, stream);
  return launch(combine_pull_kernel<kPullBlock>, dim3(static_cast<unsigned>(tiles), a.p), kPullBlock, a, stream);
}

hipError_t launch_all_to_all(const A2AArgs& a, int32_t tiles, hipStream_t stream) {
  if (tiles == 0) return hipSuccess;
  // a launch whose blocks all copy contiguous rows (no gather or scatter
  // index) runs the run-of-bytes path in 1024-thread workgroups, fewer of
  // them resident per CU: 3% faster on the MoE splits, where the indexed
  // forms lost 5-11% with them and keep 256
  bool flat = a.vec != 0;
  for (int k = 0; flat && k < a.nblocks; ++k) flat = !a.b[k].src_idx && !a.b[k].dst_idx;
  if (flat) return launch(all_to_all_kernel<1024>, dim3(static_cast<unsigned>(tiles)), 1024, a, stream);
  return launch(all_to_all_kernel<kBlock>, dim3(static_cast<unsigned>(tiles)), kBlock, a, stream);
}

}  // namespace vcoll
