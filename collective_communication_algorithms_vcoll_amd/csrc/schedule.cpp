// Host-side schedules: combination checks, message ledger, MoE plan.
//
// Sources, by page title: "Networks and Collective Communication" (cs349e
// prerequisite lecture 5) sections 4.1-4.3, 5.1, 5.2 and 7.4; "11-1.
// Distributed training" (HPC101), "Ring Algorithm". The readings used where
// the pages leave a step open are stated next to the code that takes them.
#include "schedule.h"

#include <algorithm>
#include <tuple>

namespace vcoll {

vcoll_status check_combination(vcoll_op op, vcoll_algo algo, int p) {
  switch (op) {
    case VCOLL_OP_ALLREDUCE:
      return (algo >= VCOLL_RING && algo <= VCOLL_BINARY_TREE) ? VCOLL_OK : VCOLL_ERR_INVALID_ARG;
    case VCOLL_OP_REDUCE_SCATTER:
      if (algo == VCOLL_RING) return VCOLL_OK;
      if (algo == VCOLL_RABENSEIFNER) return is_pow2(p) ? VCOLL_OK : VCOLL_ERR_UNSUPPORTED;
      return (algo >= VCOLL_RING && algo <= VCOLL_BINARY_TREE) ? VCOLL_ERR_UNSUPPORTED
                                                               : VCOLL_ERR_INVALID_ARG;
    case VCOLL_OP_ALL_GATHER:
      if (algo == VCOLL_RING) return VCOLL_OK;
      if (algo == VCOLL_RECURSIVE_DOUBLING) return is_pow2(p) ? VCOLL_OK : VCOLL_ERR_UNSUPPORTED;
      return (algo >= VCOLL_RING && algo <= VCOLL_BINARY_TREE) ? VCOLL_ERR_UNSUPPORTED
                                                               : VCOLL_ERR_INVALID_ARG;
    case VCOLL_OP_ALL_TO_ALL:
      return VCOLL_OK;
  }
  return VCOLL_ERR_INVALID_ARG;
}

void block_offsets(int p, const int64_t* splits, std::vector<int64_t>& send_off,
                   std::vector<int64_t>& recv_off) {
  send_off.assign(static_cast<size_t>(p) * p, 0);
  recv_off.assign(static_cast<size_t>(p) * p, 0);
  for (int i = 0; i < p; ++i)
    for (int j = 1; j < p; ++j)
      send_off[i * p + j] = send_off[i * p + j - 1] + splits[i * p + j - 1];
  for (int j = 0; j < p; ++j)
    for (int i = 1; i < p; ++i)
      recv_off[i * p + j] = recv_off[(i - 1) * p + j] + splits[(i - 1) * p + j];
}

namespace {

struct LedgerBuilder {
  std::vector<vcoll_msg>& out;
  int64_t esize;
  int32_t steps = 0;
  void add(int step, int src, int dst, int64_t src_off, int64_t dst_off, int64_t count) {
    vcoll_msg m{};
    m.step = step;
    m.src = src;
    m.dst = dst;
    m.src_off = src_off;
    m.dst_off = dst_off;
    m.count = count;
    m.bytes = count * esize;
    out.push_back(m);
    steps = std::max(steps, step + 1);
  }
};

// Ring reduce-scatter ([NCC] 5.1): step s, rank i passes chunk (i-1-s) mod p
// to rank i+1 (rank c ends owning chunk c, as [HPC]'s reduce-scatter
// definition gives process k the k-th piece).
int ring_rs(LedgerBuilder& L, int p, const Chunks& ch, int step) {
  for (int s = 0; s < p - 1; ++s)
    for (int i = 0; i < p; ++i) {
      const int c = ((i - 1 - s) % p + p) % p;
      L.add(step + s, i, (i + 1) % p, ch.off(c), ch.off(c), ch.count(c));
    }
  return step + (p - 1);
}

// Ring all-gather: step s, rank i forwards chunk (i-s) mod p, the complete
// chunk it holds most recently.
int ring_ag(LedgerBuilder& L, int p, const std::vector<int64_t>& off, int step) {
  for (int s = 0; s < p - 1; ++s)
    for (int i = 0; i < p; ++i) {
      const int c = ((i - s) % p + p) % p;
      L.add(step + s, i, (i + 1) % p, off[c], off[c], off[c + 1] - off[c]);
    }
  return step + (p - 1);
}

// Recursive halving over new ranks 0..p2-1 (distance p2/2 first), chunk
// bounds off[0..p2]: keep the half holding your own chunk, send the other.
int halving(LedgerBuilder& L, const Fold& f, const std::vector<int64_t>& off, int step) {
  for (int d = f.p2 / 2; d >= 1; d /= 2, ++step)
    for (int nr = 0; nr < f.p2; ++nr) {
      const int base = nr & ~(2 * d - 1);
      const int lo = (nr & d) ? base : base + d;
      L.add(step, f.old_rank(nr), f.old_rank(nr ^ d), off[lo], off[lo], off[lo + d] - off[lo]);
    }
  return step;
}

// Recursive doubling of complete ranges (distance 1, 2, .., p2/2).
int doubling(LedgerBuilder& L, const Fold& f, const std::vector<int64_t>& off, int step) {
  for (int d = 1; d < f.p2; d *= 2, ++step)
    for (int nr = 0; nr < f.p2; ++nr) {
      const int base = nr & ~(d - 1);
      L.add(step, f.old_rank(nr), f.old_rank(nr ^ d), off[base], off[base], off[base + d] - off[base]);
    }
  return step;
}

std::vector<int64_t> chunk_offsets(int64_t n, int p) {
  Chunks ch(n, p);
  std::vector<int64_t> off(p + 1);
  for (int c = 0; c <= p; ++c) off[c] = c < p ? ch.off(c) : n;
  return off;
}

}  // namespace

vcoll_status build_ledger(vcoll_op op, vcoll_algo algo, int p, int64_t n, int64_t elem_bytes,
                          const int64_t* splits, int64_t row_elems, std::vector<vcoll_msg>& out,
                          int32_t* n_steps) {
  out.clear();
  LedgerBuilder L{out, elem_bytes};
  if (op == VCOLL_OP_ALL_TO_ALL) {
    std::vector<int64_t> so, ro;
    block_offsets(p, splits, so, ro);
    for (int s = 1; s < p; ++s)
      for (int i = 0; i < p; ++i) {
        const int j = (i + s) % p;
        L.add(s - 1, i, j, so[i * p + j] * row_elems, ro[i * p + j] * row_elems,
              splits[i * p + j] * row_elems);
      }
  } else if (op == VCOLL_OP_ALL_GATHER) {
    std::vector<int64_t> off(p + 1);
    for (int c = 0; c <= p; ++c) off[c] = c * n;
    if (algo == VCOLL_RING) ring_ag(L, p, off, 0);
    else doubling(L, Fold(p), off, 0);
  } else if (op == VCOLL_OP_REDUCE_SCATTER) {
    if (algo == VCOLL_RING) ring_rs(L, p, Chunks(n, p), 0);
    else halving(L, Fold(p), chunk_offsets(n, p), 0);
  } else {  // all-reduce
    if (algo == VCOLL_RING) {
      const int step = ring_rs(L, p, Chunks(n, p), 0);
      ring_ag(L, p, chunk_offsets(n, p), step);
    } else if (algo == VCOLL_BINARY_TREE) {
      // binomial reduce to rank 0: a rank whose lowest set bit is the mask
      // sends its full vector to rank - mask; then the mirrored broadcast
      std::vector<int> masks;
      for (int m = 1; m < p; m <<= 1) masks.push_back(m);
      int step = 0;
      for (int m : masks) {
        for (int i = 0; i < p; ++i)
          if ((i & -i) == m) L.add(step, i, i - m, 0, 0, n);
        ++step;
      }
      for (auto it = masks.rbegin(); it != masks.rend(); ++it, ++step)
        for (int i = 0; i < p; i += 2 * *it)
          if (i + *it < p) L.add(step, i, i + *it, 0, 0, n);
    } else {
      const Fold f(p);
      int step = 0;
      if (f.r > 0) {
        for (int j = 0; j < f.r; ++j) L.add(step, 2 * j, 2 * j + 1, 0, 0, n);
        ++step;
      }
      if (algo == VCOLL_RECURSIVE_DOUBLING) {
        for (int d = 1; d < f.p2; d *= 2, ++step)
          for (int nr = 0; nr < f.p2; ++nr) L.add(step, f.old_rank(nr), f.old_rank(nr ^ d), 0, 0, n);
      } else {
        const std::vector<int64_t> off = chunk_offsets(n, f.p2);
        step = halving(L, f, off, step);
        step = doubling(L, f, off, step);
      }
      if (f.r > 0)
        for (int j = 0; j < f.r; ++j) L.add(step, 2 * j + 1, 2 * j, 0, 0, n);
    }
  }
  std::sort(out.begin(), out.end(), [](const vcoll_msg& a, const vcoll_msg& b) {
    return std::tie(a.step, a.src, a.dst, a.src_off) < std::tie(b.step, b.src, b.dst, b.src_off);
  });
  if (n_steps) *n_steps = L.steps;
  return VCOLL_OK;
}

vcoll_status build_ledger_hierarchical(int nodes, int local, int64_t n, int64_t elem_bytes,
                                       std::vector<vcoll_msg>& out, int32_t* n_steps) {
  out.clear();
  LedgerBuilder L{out, elem_bytes};
  const int N = nodes, Lc = local;
  const Chunks ch(n, Lc);
  // piece j of chunk l
  auto piece = [&](int l, int j, int64_t* off, int64_t* cnt) {
    const Chunks sub(ch.count(l), N);
    *off = ch.off(l) + sub.off(j);
    *cnt = sub.count(j);
  };
  int step = 0;
  // (1) reduce-scatter inside every group: group rank i sends chunk (i-1-s)
  for (int s = 0; s < Lc - 1; ++s, ++step)
    for (int g = 0; g < N; ++g)
      for (int i = 0; i < Lc; ++i) {
        const int c = ((i - 1 - s) % Lc + Lc) % Lc;
        L.add(step, g * Lc + i, g * Lc + (i + 1) % Lc, ch.off(c), ch.off(c), ch.count(c));
      }
  // (2) across groups, for every index l: ring reduce-scatter then all-gather
  // of chunk l's N pieces (group g sends piece (g-1-s), then (g-s))
  for (int phase = 0; phase < 2; ++phase)
    for (int s = 0; s < N - 1; ++s, ++step)
      for (int l = 0; l < Lc; ++l)
        for (int g = 0; g < N; ++g) {
          const int j = ((g - (phase == 0 ? 1 : 0) - s) % N + N) % N;
          int64_t off, cnt;
          piece(l, j, &off, &cnt);
          L.add(step, g * Lc + l, ((g + 1) % N) * Lc + l, off, off, cnt);
        }
  // (3) all-gather inside every group: group rank i forwards chunk (i-s)
  for (int s = 0; s < Lc - 1; ++s, ++step)
    for (int g = 0; g < N; ++g)
      for (int i = 0; i < Lc; ++i) {
        const int c = ((i - s) % Lc + Lc) % Lc;
        L.add(step, g * Lc + i, g * Lc + (i + 1) % Lc, ch.off(c), ch.off(c), ch.count(c));
      }
  std::sort(out.begin(), out.end(), [](const vcoll_msg& a, const vcoll_msg& b) {
    return std::tie(a.step, a.src, a.dst, a.src_off) < std::tie(b.step, b.src, b.dst, b.src_off);
  });
  if (n_steps) *n_steps = L.steps;
  return VCOLL_OK;
}

vcoll_status build_ledger_rooted(vcoll_op op, vcoll_algo algo, int p, int64_t n, int64_t elem_bytes, int root,
                                 int64_t blocks, std::vector<vcoll_msg>& out, int32_t* n_steps) {
  if (p < 1 || root < 0 || root >= p || n < 0) return VCOLL_ERR_INVALID_ARG;
  out.clear();
  LedgerBuilder L{out, elem_bytes};
  auto abs = [&](int v) { return (v + root) % p; };
  int masks = 0;                                  // ceil(log2 p)
  while ((1 << masks) < p) ++masks;
  if (op == VCOLL_OP_REDUCE) {
    if (algo != VCOLL_BINARY_TREE) return VCOLL_ERR_UNSUPPORTED;
    // [NCC] 5.2 binomial reduce: masks ascending, a relative rank whose
    // lowest set bit is the mask sends its whole vector to v - mask
    for (int s = 0; s < masks; ++s)
      for (int v = 1; v < p; ++v)
        if ((v & -v) == (1 << s)) L.add(s, abs(v), abs(v - (1 << s)), 0, 0, n);
  } else if (op == VCOLL_OP_BROADCAST) {
    switch (algo) {
      case VCOLL_NAIVE:                           // [NCC] 5.5: one receiver per step
        for (int s = 0; s + 1 < p; ++s) L.add(s, abs(0), abs(s + 1), 0, 0, n);
        break;
      case VCOLL_BINARY_TREE:                     // masks descending
        for (int s = 0; s < masks; ++s) {
          const int m = 1 << (masks - 1 - s);
          for (int v = 0; v + m < p; v += 2 * m) L.add(s, abs(v), abs(v + m), 0, 0, n);
        }
        break;
      case VCOLL_SCATTER_ALLGATHER: {             // [NCC] 4.2: scatter in one step, ring all-gather
        if (p == 1) break;
        const Chunks ch(n, p);
        for (int v = 1; v < p; ++v) L.add(0, abs(0), abs(v), ch.off(v), ch.off(v), ch.count(v));
        for (int s = 0; s < p - 1; ++s)
          for (int v = 0; v < p; ++v) {
            const int c = ((v - s) % p + p) % p;
            L.add(1 + s, abs(v), abs((v + 1) % p), ch.off(c), ch.off(c), ch.count(c));
          }
        break;
      }
      case VCOLL_PIPELINED_CHAIN: {               // [NCC] 5.5: k blocks down the chain 0 -> 1 -> .. -> p-1
        if (blocks < 1) return VCOLL_ERR_INVALID_ARG;
        if (p == 1) break;
        const int64_t qb = n / blocks, rb = n % blocks;
        auto boff = [&](int64_t b) { return b * qb + (b < rb ? b : rb); };
        for (int64_t t = 0; t < p - 2 + blocks; ++t)
          for (int v = 0; v + 1 < p; ++v) {
            const int64_t b = t - v;
            if (b >= 0 && b < blocks) L.add(static_cast<int>(t), abs(v), abs(v + 1), boff(b), boff(b), qb + (b < rb ? 1 : 0));
          }
        break;
      }
      default:
        return (algo >= VCOLL_RING && algo <= VCOLL_PIPELINED_CHAIN) ? VCOLL_ERR_UNSUPPORTED : VCOLL_ERR_INVALID_ARG;
    }
  } else {
    return VCOLL_ERR_INVALID_ARG;
  }
  std::sort(out.begin(), out.end(), [](const vcoll_msg& a, const vcoll_msg& b) {
    return std::tie(a.step, a.src, a.dst, a.src_off) < std::tie(b.step, b.src, b.dst, b.src_off);
  });
  if (n_steps) *n_steps = L.steps;
  return VCOLL_OK;
}

int build_step_program(vcoll_algo algo, int p, int64_t n, bool narrow,
                       std::vector<std::vector<StepOp>>& steps) {
  // Start from the ledger: it is the list of messages, step by step. Each
  // algorithm's phases decide whether a message adds or copies.
  std::vector<vcoll_msg> msgs;
  int32_t n_steps = 0;
  build_ledger(VCOLL_OP_ALLREDUCE, algo, p, n, 4, nullptr, 0, msgs, &n_steps);
  std::vector<std::vector<vcoll_msg>> by_step(static_cast<size_t>(n_steps));
  for (const vcoll_msg& m : msgs) by_step[static_cast<size_t>(m.step)].push_back(m);
  steps.assign(static_cast<size_t>(n_steps), {});
  std::vector<StepOp> narrowing;
  auto add_narrow = [&](int rank, int64_t off, int64_t count) {
    if (count > 0) narrowing.push_back({STEP_NARROW, rank, rank, off, count});
  };
  const Fold f(p);
  // kind of every message step, and where results become complete
  int rs_end = 0;                 // steps [first_rs, rs_end) add; later ones copy
  int first_rs = 0;
  if (algo == VCOLL_RING) {
    rs_end = p - 1;
  } else if (algo == VCOLL_BINARY_TREE) {
    int k = 0;
    while ((1 << k) < p) ++k;
    rs_end = k;
  } else {
    first_rs = f.r > 0 ? 1 : 0;                        // fold pre-step adds too
    rs_end = first_rs + floor_log2(f.p2);
  }
  for (int s = 0; s < n_steps; ++s) {
    const bool adds = s < rs_end;
    for (const vcoll_msg& m : by_step[static_cast<size_t>(s)]) {
      if (algo == VCOLL_RECURSIVE_DOUBLING && adds && s >= first_rs) {
        // core steps exchange full vectors: one XADD per partner pair
        if (m.src < m.dst) steps[s].push_back({STEP_XADD, m.src, m.dst, m.src_off, m.count});
      } else {
        steps[s].push_back({adds ? STEP_ADD : STEP_COPY, m.src, m.dst, m.src_off, m.count});
      }
    }
  }
  // results are complete after the last adding step; rounding them to
  // bfloat16 is a step of its own, so that it follows every add
  if (narrow && rs_end > 0) {
    if (algo == VCOLL_RING) {
      const Chunks ch(n, p);
      for (int c = 0; c < p; ++c) add_narrow(c, ch.off(c), ch.count(c));
    } else if (algo == VCOLL_BINARY_TREE) {
      add_narrow(0, 0, n);
    } else if (algo == VCOLL_RECURSIVE_DOUBLING) {
      for (int nr = 0; nr < f.p2; ++nr) add_narrow(f.old_rank(nr), 0, n);
    } else {
      const Chunks ch(n, f.p2);
      for (int nr = 0; nr < f.p2; ++nr) add_narrow(f.old_rank(nr), ch.off(nr), ch.count(nr));
    }
    steps.insert(steps.begin() + rs_end, narrowing);
  }
  return n_steps;
}

vcoll_status moe_plan(int p, int64_t tokens, int topk, int experts_per_rank,
                      const int32_t* topk_ids, int64_t* splits, int32_t* src_rows,
                      int32_t* dst_rows) {
  const int64_t experts = static_cast<int64_t>(p) * experts_per_rank;
  const int64_t rows = tokens * topk;
  std::vector<int64_t> count(experts), start(experts);
  for (int i = 0; i < p; ++i) {
    const int32_t* ids = topk_ids + static_cast<int64_t>(i) * rows;
    std::fill(count.begin(), count.end(), 0);
    for (int64_t x = 0; x < rows; ++x) {
      if (ids[x] < 0 || ids[x] >= experts) return VCOLL_ERR_INVALID_ARG;
      ++count[ids[x]];
    }
    // rows ordered by (destination rank, expert, token): destination rank is
    // monotone in the expert id, so a counting sort on the expert id, filled
    // in token order, gives that order
    int64_t acc = 0;
    for (int64_t e = 0; e < experts; ++e) { start[e] = acc; acc += count[e]; }
    for (int j = 0; j < p; ++j) {
      int64_t s = 0;
      for (int64_t e = static_cast<int64_t>(j) * experts_per_rank; e < (j + 1LL) * experts_per_rank; ++e)
        s += count[e];
      splits[static_cast<int64_t>(i) * p + j] = s;
    }
    int32_t* src = src_rows + static_cast<int64_t>(i) * rows;
    int32_t* dst = dst_rows + static_cast<int64_t>(i) * rows;
    for (int64_t t = 0; t < tokens; ++t)
      for (int k = 0; k < topk; ++k) {
        const int64_t pos = start[ids[t * topk + k]]++;
        src[pos] = static_cast<int32_t>(t);
        dst[pos] = static_cast<int32_t>(t * topk + k);
      }
  }
  return VCOLL_OK;
}

vcoll_status moe_plan_dedup(int p, int64_t tokens, int topk, int experts_per_rank,
                            const int32_t* topk_ids, int64_t* splits_unique, int32_t* src_unique,
                            int32_t* expand, int64_t* expand_count) {
  const int64_t rows = tokens * topk;
  std::vector<int64_t> splits(static_cast<size_t>(p) * p);
  std::vector<int32_t> src(static_cast<size_t>(p) * rows), dst(static_cast<size_t>(p) * rows);
  const vcoll_status st = moe_plan(p, tokens, topk, experts_per_rank, topk_ids, splits.data(), src.data(), dst.data());
  if (st != VCOLL_OK) return st;
  // where[j * tokens + t]: position of token t inside rank i's block for
  // rank j of the deduplicated send (-1: t does not go to j)
  std::vector<int32_t> where(static_cast<size_t>(p) * tokens);
  auto dedup_rank = [&](int i) {
    std::fill(where.begin(), where.end(), -1);
    const int32_t* ids = topk_ids + static_cast<int64_t>(i) * rows;
    for (int64_t t = 0; t < tokens; ++t)
      for (int k = 0; k < topk; ++k) where[static_cast<size_t>(ids[t * topk + k] / experts_per_rank) * tokens + t] = 0;
    int64_t pos = 0;
    for (int j = 0; j < p; ++j) {
      int32_t n = 0;
      for (int64_t t = 0; t < tokens; ++t) {
        int32_t& w = where[static_cast<size_t>(j) * tokens + t];
        if (w < 0) continue;
        w = n++;
        src_unique[static_cast<int64_t>(i) * rows + pos++] = static_cast<int32_t>(t);
      }
      splits_unique[static_cast<int64_t>(i) * p + j] = n;
    }
  };
  // rank j's plain layout holds the blocks of ranks 0..p-1, each in the
  // sender's (expert, token) order; its deduplicated buffer the same blocks,
  // each in token order
  const int64_t cap = static_cast<int64_t>(p) * rows;
  std::vector<int64_t> xoff(p, 0), uoff(p, 0);
  for (int i = 0; i < p; ++i) {
    dedup_rank(i);                        // rank i's unique rows, splits_unique row i and `where`
    int64_t s0 = 0;                       // offset of block (i -> j) in rank i's plain send order
    for (int j = 0; j < p; ++j) {
      const int64_t nij = splits[static_cast<size_t>(i) * p + j];
      for (int64_t r = 0; r < nij; ++r) {
        const int32_t t = src[static_cast<size_t>(i) * rows + s0 + r];
        expand[static_cast<int64_t>(j) * cap + xoff[j] + r] =
            static_cast<int32_t>(uoff[j] + where[static_cast<size_t>(j) * tokens + t]);
      }
      s0 += nij;
      xoff[j] += nij;
      uoff[j] += splits_unique[static_cast<int64_t>(i) * p + j];
    }
  }
  for (int j = 0; j < p; ++j) expand_count[j] = xoff[j];
  return VCOLL_OK;
}

vcoll_status moe_slots(int p, int64_t tokens, int topk, const int64_t* splits, const int32_t* dst_rows,
                       int32_t* slots) {
  const int64_t rows = tokens * topk;
  std::vector<int64_t> so, ro;
  block_offsets(p, splits, so, ro);
  for (int i = 0; i < p; ++i) {
    int32_t* out = slots + 2 * static_cast<int64_t>(i) * rows;
    std::fill(out, out + 2 * rows, -1);
    const int32_t* pairs = dst_rows + static_cast<int64_t>(i) * rows;
    int64_t pos = 0;
    for (int j = 0; j < p; ++j)
      for (int64_t r = 0; r < splits[static_cast<size_t>(i) * p + j]; ++r, ++pos) {
        if (pos >= rows) return VCOLL_ERR_INVALID_ARG;
        const int32_t pair = pairs[pos];            // t * topk + k
        if (pair < 0 || pair >= rows) return VCOLL_ERR_INVALID_ARG;
        out[2 * pair] = j;
        out[2 * pair + 1] = static_cast<int32_t>(ro[static_cast<size_t>(i) * p + j] + r);
      }
  }
  return VCOLL_OK;
}

vcoll_status moe_expand_slots(int64_t unique_rows, int topk, const int32_t* expand, int64_t expand_count,
                              int32_t* slots) {
  std::fill(slots, slots + 2 * unique_rows * topk, -1);
  std::vector<int32_t> used(static_cast<size_t>(unique_rows), 0);
  for (int64_t x = 0; x < expand_count; ++x) {
    const int32_t u = expand[x];
    if (u < 0 || u >= unique_rows || used[static_cast<size_t>(u)] >= topk) return VCOLL_ERR_INVALID_ARG;
    const int64_t k = used[static_cast<size_t>(u)]++;
    slots[2 * (u * topk + k)] = 0;
    slots[2 * (u * topk + k) + 1] = static_cast<int32_t>(x);
  }
  return VCOLL_OK;
}

vcoll_status moe_dedup_slots(int p, int64_t tokens, int width, const int64_t* splits_unique,
                             const int32_t* src_unique, int32_t* slots) {
  std::vector<int64_t> so, ro;
  block_offsets(p, splits_unique, so, ro);
  std::vector<int32_t> used(static_cast<size_t>(tokens));
  for (int i = 0; i < p; ++i) {
    int32_t* out = slots + 2 * static_cast<int64_t>(i) * tokens * width;
    std::fill(out, out + 2 * tokens * width, -1);
    std::fill(used.begin(), used.end(), 0);
    int64_t pos = 0;
    for (int j = 0; j < p; ++j)
      for (int64_t q = 0; q < splits_unique[static_cast<size_t>(i) * p + j]; ++q, ++pos) {
        const int32_t t = src_unique[static_cast<int64_t>(i) * tokens * width + pos];
        if (t < 0 || t >= tokens || used[static_cast<size_t>(t)] >= width) return VCOLL_ERR_INVALID_ARG;
        const int64_t k = used[static_cast<size_t>(t)]++;
        out[2 * (t * width + k)] = j;
        out[2 * (t * width + k) + 1] = static_cast<int32_t>(ro[static_cast<size_t>(i) * p + j] + q);
      }
  }
  return VCOLL_OK;
}

}  // namespace vcoll
