// Alpha-beta (Hockney) cost model: closed forms and a simulated clock over
// the message ledger. Host only.
//
// "Networks and Collective Communication" (cs349e prerequisite lecture 5):
// section 2.1 prices one n-byte message at alpha + n/beta; sections 5.1 and
// 5.2 (and exercise 2) give the all-reduce closed forms; the lecture's
// comm_sim advances a clock step by step, which the ledger version does with
// full-duplex ports (a device sends and receives concurrently at beta).
#include <algorithm>
#include <cmath>
#include <map>
#include <vector>

#include "schedule.h"
#include "vcoll.h"

using namespace vcoll;

namespace {

// Two link classes ([NCC] 2.3): ranks r and s share a node when
// r / local == s / local. Each rank has a sending and a receiving port per
// class; a step lasts as long as its slowest port that carries a message
// (alpha + bytes / beta of that port's class; a 0-byte message still costs
// alpha). With local >= p every message is of the inner class.
double two_class_clock(const vcoll_msg* msgs, int64_t count, int p, int local, double alpha_in, double beta_in,
                       double alpha_out, double beta_out) {
  // per step: port key (class, direction, rank) -> bytes
  std::map<int32_t, std::map<int64_t, int64_t>> per_step;
  for (int64_t i = 0; i < count; ++i) {
    const vcoll_msg& m = msgs[i];
    const int across = (m.src / local != m.dst / local) ? 1 : 0;
    std::map<int64_t, int64_t>& ports = per_step[m.step];
    ports[(static_cast<int64_t>(across) * 2 + 0) * p + m.src] += m.bytes;
    ports[(static_cast<int64_t>(across) * 2 + 1) * p + m.dst] += m.bytes;
  }
  double t = 0.0;
  for (const auto& step : per_step) {
    double slowest = 0.0;
    for (const auto& port : step.second) {
      const bool across = port.first >= 2 * p;
      slowest = std::max(slowest, (across ? alpha_out : alpha_in) +
                                      static_cast<double>(port.second) / (across ? beta_out : beta_in));
    }
    t += slowest;
  }
  return t;
}

}  // namespace

extern "C" {

vcoll_status vcoll_model_formula(vcoll_algo algo, int p, double bytes, double alpha, double beta,
                                 double* seconds) {
  if (p < 1 || p > (1 << 20) || !(bytes >= 0) || !(alpha >= 0) || !(beta > 0) || !seconds)
    return VCOLL_ERR_INVALID_ARG;
  if (algo < VCOLL_RING || algo > VCOLL_BINARY_TREE) return VCOLL_ERR_INVALID_ARG;
  if (p == 1) {
    *seconds = 0.0;
    return VCOLL_OK;
  }
  const double full = alpha + bytes / beta;
  switch (algo) {
    case VCOLL_RING:  // 2(p-1) steps of n/p bytes
      *seconds = 2.0 * (p - 1) * (alpha + bytes / (p * beta));
      return VCOLL_OK;
    case VCOLL_BINARY_TREE: {  // 2 ceil(log2 p) full-vector steps
      int k = 0;
      while ((1 << k) < p) ++k;
      *seconds = 2.0 * k * full;
      return VCOLL_OK;
    }
    default: {
      // powers of two as printed; otherwise the fold adds a full-vector
      // pre-step and post-step around the p2 = 2^floor(log2 p) core
      const int p2 = 1 << floor_log2(p);
      const int k = floor_log2(p2);
      const double extra = p2 == p ? 0.0 : 2.0 * full;
      if (algo == VCOLL_RECURSIVE_DOUBLING) *seconds = k * full + extra;
      else *seconds = 2.0 * k * alpha + 2.0 * (p2 - 1) / p2 * bytes / beta + extra;
      return VCOLL_OK;
    }
  }
}

vcoll_status vcoll_model_ledger_time(vcoll_op op, vcoll_algo algo, int p, int64_t n, vcoll_dtype dtype,
                                     const int64_t* splits, int64_t row_elems, double alpha, double beta,
                                     double* seconds, int32_t* n_steps) {
  if (!(alpha >= 0) || !(beta > 0) || !seconds) return VCOLL_ERR_INVALID_ARG;
  int64_t count = 0;
  vcoll_status st = vcoll_ledger(op, algo, p, n, dtype, splits, row_elems, nullptr, 0, &count,
                                 nullptr, nullptr, nullptr);
  if (st != VCOLL_OK) return st;
  std::vector<vcoll_msg> msgs(static_cast<size_t>(std::max<int64_t>(count, 1)));
  int32_t steps = 0;
  st = vcoll_ledger(op, algo, p, n, dtype, splits, row_elems, msgs.data(), count, &count, nullptr,
                    nullptr, &steps);
  if (st != VCOLL_OK) return st;
  // per step: bytes each rank sends and receives; the busiest port sets the pace
  std::map<int32_t, std::pair<std::vector<int64_t>, std::vector<int64_t>>> per_step;
  for (int64_t i = 0; i < count; ++i) {
    const vcoll_msg& m = msgs[static_cast<size_t>(i)];
    auto& slot = per_step[m.step];
    if (slot.first.empty()) {
      slot.first.assign(p, 0);
      slot.second.assign(p, 0);
    }
    slot.first[m.src] += m.bytes;
    slot.second[m.dst] += m.bytes;
  }
  double t = 0.0;
  for (const auto& kv : per_step) {
    int64_t busiest = 0;
    for (int r = 0; r < p; ++r) busiest = std::max({busiest, kv.second.first[r], kv.second.second[r]});
    t += alpha + static_cast<double>(busiest) / beta;
  }
  *seconds = t;
  if (n_steps) *n_steps = steps;
  return VCOLL_OK;
}

vcoll_status vcoll_model_ledger_time_nodes(int hierarchical, vcoll_algo algo, int nodes, int local, int64_t n,
                                           vcoll_dtype dtype, double alpha_in, double beta_in,
                                           double alpha_out, double beta_out, double* seconds,
                                           int32_t* n_steps) {
  if (!(alpha_in >= 0) || !(beta_in > 0) || !(alpha_out >= 0) || !(beta_out > 0) || !seconds)
    return VCOLL_ERR_INVALID_ARG;
  // each factor is bounded before the product is formed (no int overflow)
  if (nodes < 1 || local < 1 || nodes > VCOLL_MAX_RANKS || local > VCOLL_MAX_RANKS) return VCOLL_ERR_INVALID_ARG;
  const int p = nodes * local;
  int64_t count = 0;
  vcoll_status st = hierarchical
                        ? vcoll_ledger_hierarchical(nodes, local, n, dtype, nullptr, 0, &count, nullptr, nullptr, nullptr)
                        : vcoll_ledger(VCOLL_OP_ALLREDUCE, algo, p, n, dtype, nullptr, 0, nullptr, 0, &count,
                                       nullptr, nullptr, nullptr);
  if (st != VCOLL_OK) return st;
  std::vector<vcoll_msg> msgs(static_cast<size_t>(std::max<int64_t>(count, 1)));
  int32_t steps = 0;
  st = hierarchical ? vcoll_ledger_hierarchical(nodes, local, n, dtype, msgs.data(), count, &count, nullptr,
                                                nullptr, &steps)
                    : vcoll_ledger(VCOLL_OP_ALLREDUCE, algo, p, n, dtype, nullptr, 0, msgs.data(), count,
                                   &count, nullptr, nullptr, &steps);
  if (st != VCOLL_OK) return st;
  *seconds = two_class_clock(msgs.data(), count, p, local, alpha_in, beta_in, alpha_out, beta_out);
  if (n_steps) *n_steps = steps;
  return VCOLL_OK;
}

vcoll_status vcoll_model_clock(const vcoll_msg* msgs, int64_t n_msgs, int p, int local, double alpha_in,
                               double beta_in, double alpha_out, double beta_out, double* seconds) {
  if (!(alpha_in >= 0) || !(beta_in > 0) || !(alpha_out >= 0) || !(beta_out > 0) || !seconds)
    return VCOLL_ERR_INVALID_ARG;
  if (p < 1 || local < 1 || n_msgs < 0 || (n_msgs > 0 && !msgs)) return VCOLL_ERR_INVALID_ARG;
  for (int64_t i = 0; i < n_msgs; ++i)
    if (msgs[i].src < 0 || msgs[i].src >= p || msgs[i].dst < 0 || msgs[i].dst >= p || msgs[i].bytes < 0)
      return VCOLL_ERR_INVALID_ARG;
  *seconds = two_class_clock(msgs, n_msgs, p, local, alpha_in, beta_in, alpha_out, beta_out);
  return VCOLL_OK;
}

vcoll_status vcoll_model_broadcast_formula(vcoll_algo algo, int p, double nbytes, int64_t blocks, double alpha,
                                           double beta, double* seconds) {
  if (p < 1 || p > (1 << 20) || !(nbytes >= 0) || !(alpha >= 0) || !(beta > 0) || !seconds)
    return VCOLL_ERR_INVALID_ARG;
  if (algo == VCOLL_PIPELINED_CHAIN && blocks < 1) return VCOLL_ERR_INVALID_ARG;
  double t = 0.0;
  int k = 0;
  while ((1 << k) < p) ++k;
  switch (algo) {
    case VCOLL_NAIVE: t = (p - 1) * (alpha + nbytes / beta); break;
    case VCOLL_BINARY_TREE: t = k * (alpha + nbytes / beta); break;
    case VCOLL_PIPELINED_CHAIN:
      t = p == 1 ? 0.0 : (p - 2 + static_cast<double>(blocks)) * (alpha + nbytes / (static_cast<double>(blocks) * beta));
      break;
    case VCOLL_SCATTER_ALLGATHER:
      t = p == 1 ? 0.0
                 : (alpha + (p - 1.0) / p * nbytes / beta) + (p - 1) * (alpha + nbytes / (static_cast<double>(p) * beta));
      break;
    default: return VCOLL_ERR_INVALID_ARG;
  }
  *seconds = t;
  return VCOLL_OK;
}

vcoll_status vcoll_model_chain_optimum(int p, double nbytes, double alpha, double beta, double* blocks,
                                       double* seconds) {
  if (p < 3 || !(nbytes > 0) || !(alpha > 0) || !(beta > 0) || !blocks || !seconds) return VCOLL_ERR_INVALID_ARG;
  // minimise (p-2+k)(alpha + n/(k beta)) over real k
  *blocks = std::sqrt((p - 2) * nbytes / (alpha * beta));
  const double root = std::sqrt((p - 2) * alpha) + std::sqrt(nbytes / beta);
  *seconds = root * root;
  return VCOLL_OK;
}

}  // extern "C"
