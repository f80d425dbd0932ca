// Summation orders of the all-reduce algorithms as push / add programs.
//
// Every algorithm of "Networks and Collective Communication" (cs349e
// prerequisite lecture 5), sections 5.1 and 5.2, ends with every element
// equal to a sum of the p inputs whose association is fixed by the steps.
// A program says: for k = 0..p-1 push input rank[k] onto a stack, then
// replace the top two entries by their float32 sum merges[k] times; at the
// end do final_merges more such adds. IEEE addition is commutative, so only
// which partial sums meet matters, and that is what the program fixes.
//
// The functions are constexpr so that kernels specialised for a fixed p can
// unfold the whole program at compile time.
#pragma once

#include "vcoll.h"

namespace vcoll {

constexpr int kMaxRanks = VCOLL_MAX_RANKS;

struct OrderProgram {
  int p = 0;
  int rank[kMaxRanks] = {};
  int merges[kMaxRanks] = {};
  int final_merges = 0;
  int max_depth = 0;   // stack entries alive at the deepest point
};

constexpr bool is_pow2(int p) { return p >= 1 && (p & (p - 1)) == 0; }

constexpr int floor_log2(int p) {
  int k = 0;
  while ((2 << k) <= p) ++k;
  return k;
}

constexpr int ctz_int(int v) {
  int k = 0;
  while (v > 0 && (v & 1) == 0) {
    v >>= 1;
    ++k;
  }
  return k;
}

constexpr int popcount_int(int v) {
  int k = 0;
  for (; v; v &= v - 1) ++k;
  return k;
}

constexpr int bitrev_int(int v, int bits) {
  int r = 0;
  for (int b = 0; b < bits; ++b) r |= ((v >> b) & 1) << (bits - 1 - b);
  return r;
}

// Fold for p not a power of two (Thakur, Rabenseifner and Gropp, 2005, in
// the lecture's reading list): p2 = largest power of two <= p, r = p - p2;
// new rank nr < r stands for the pair of old ranks (2nr, 2nr+1), already
// added, and new rank nr >= r for old rank nr + r.
struct Fold {
  int p2 = 1, r = 0;
  constexpr explicit Fold(int p) : p2(1 << floor_log2(p)), r(p - (1 << floor_log2(p))) {}
  constexpr int old_rank(int nr) const { return nr < r ? 2 * nr + 1 : nr + r; }
};

// algo: VCOLL_RING gives the chain of the ring (leaf k is the k-th rank after
// the chunk's owner, rotated per chunk by the caller); the tree algorithms
// give their chunk-independent orders.
constexpr OrderProgram order_program(int algo, int p) {
  OrderProgram g;
  g.p = p;
  int k = 0;
  if (algo == VCOLL_RING) {
    // section 5.1: the partial sum of a chunk travels the ring and each rank
    // on the way adds its own piece: a left-to-right chain
    for (int i = 0; i < p; ++i) {
      g.rank[i] = i;
      g.merges[i] = i > 0 ? 1 : 0;
    }
  } else if (algo == VCOLL_BINARY_TREE) {
    // binomial reduce to rank 0 (masks 1, 2, 4, ..): rank i's subtree is the
    // power-of-two aligned range of ranks starting at i, so the leaves are
    // the ranks in order, a binary counter closes each complete subtree, and
    // the subtrees left over (one per set bit of p) are added right to left
    for (int i = 0; i < p; ++i) {
      g.rank[i] = i;
      g.merges[i] = ctz_int(i + 1);
    }
    g.final_merges = popcount_int(p) - 1;
  } else {
    // recursive doubling pairs partners that differ in bit 0 first; the
    // Rabenseifner halving pairs partners that differ in the top bit first,
    // which is the same balanced tree over the new ranks in bit-reversed
    // order. Folded pairs are added before they enter the tree.
    const Fold f(p);
    const int bits = floor_log2(f.p2);
    for (int q = 0; q < f.p2; ++q) {
      const int nr = (algo == VCOLL_RABENSEIFNER) ? bitrev_int(q, bits) : q;
      const int closes = ctz_int(q + 1);
      if (nr < f.r) {
        g.rank[k] = 2 * nr;
        g.merges[k] = 0;
        ++k;
        g.rank[k] = 2 * nr + 1;
        g.merges[k] = 1 + closes;
        ++k;
      } else {
        g.rank[k] = nr + f.r;
        g.merges[k] = closes;
        ++k;
      }
    }
  }
  int depth = 0, maxd = 0;
  for (int i = 0; i < p; ++i) {
    ++depth;
    maxd = depth > maxd ? depth : maxd;
    depth -= g.merges[i];
  }
  g.max_depth = maxd;
  return g;
}

// The tree programs above are binary counters over groups: a group is one
// leaf, or a folded pair of leaves added to each other first; after group q
// the counter closes ctz(q + 1) complete subtrees (older partial + newer),
// and at the end the subtrees still open, one per set bit of the group
// count, are added from the smallest up. Fills first[q] = the program leaf
// that starts group q (first[groups] = p) and returns the group count; the
// ring, a chain, has no groups (returns 0).
constexpr int order_groups(int algo, int p, int* first) {
  if (algo == VCOLL_RING) return 0;
  if (algo == VCOLL_BINARY_TREE) {
    for (int q = 0; q <= p; ++q) first[q] = q;
    return p;
  }
  const Fold f(p);
  const int bits = floor_log2(f.p2);
  int k = 0;
  for (int q = 0; q < f.p2; ++q) {
    const int nr = (algo == VCOLL_RABENSEIFNER) ? bitrev_int(q, bits) : q;
    first[q] = k;
    k += nr < f.r ? 2 : 1;
  }
  first[f.p2] = k;
  return f.p2;
}

}  // namespace vcoll
