// Replay-unit assignment of the online planner (host only; no device code).
//
// "Splitting Prompt Prefill from Response Replay ...", §3.4 (replay units and grid
// assignment): a plan candidate has b response-replay rounds of s lanes each; the planner
// places the U replay units (one complete response path each, with a work estimate w_k) on
// that grid so as to minimise the sum over rounds of the largest lane load in the round,
// exactly by dynamic programming over subsets of units when U is at most a small cap, and by
// largest-first greedy balancing otherwise. Every cell of the grid holds at least one unit
// (candidates with empty lanes are filtered out before assignment; with empty cells allowed a
// single round would always be optimal, since stacking two rounds' lanes never exceeds the sum
// of their maxima).
//
// Exact path: sum[A] = total weight of unit set A; lane[t][A] = the least largest load of A
// split over t non-empty lanes; round[r][A] = the least sum of round maxima of A split over r
// non-empty rounds of s lanes. Each split enumerates the subsets that contain A's lowest unit,
// in a fixed order, keeping the first strictly better choice, so the result is deterministic.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <limits>
#include <numeric>
#include <vector>

#include "../../include/augtree.h"
#include "kernels.hpp"

namespace augtree {
namespace {

constexpr double kBig = std::numeric_limits<double>::infinity();

struct Choice {
  std::vector<double> val;   // per subset
  std::vector<uint32_t> arg;  // chosen part containing the lowest unit (0: none)
};

// Splits every subset into `parts` non-empty parts, each part valued by part_val, combined by
// comb (max for lanes, + for rounds); prev = the table for parts - 1.
template <typename Comb>
void split_level(const std::vector<double>& part_val, const Choice& prev, Choice& out, int n, Comb comb) {
  const uint32_t full = (1u << n) - 1u;
  out.val.assign((size_t)full + 1, kBig);
  out.arg.assign((size_t)full + 1, 0u);
  for (uint32_t mask = 1; mask <= full; ++mask) {
    const uint32_t low = mask & (~mask + 1u);
    const uint32_t rest = mask ^ low;
    double best = kBig;
    uint32_t barg = 0;
    // parts A = low | sub, sub a proper subset of rest (the remainder mask ^ A is non-empty)
    for (uint32_t sub = rest;; sub = (sub - 1u) & rest) {
      const uint32_t a = low | sub;
      if (a != mask) {
        const double v = comb(part_val[a], prev.val[mask ^ a]);
        if (v < best) {
          best = v;
          barg = a;
        }
      }
      if (sub == 0) break;
    }
    out.val[mask] = best;
    out.arg[mask] = barg;
  }
}

augtree_status assign_exact(const double* w, int n, int rounds, int lanes, int32_t* cell, double* cost) {
  const uint32_t full = (1u << n) - 1u;
  std::vector<double> sum((size_t)full + 1, 0.0);
  for (uint32_t mask = 1; mask <= full; ++mask) {
    const int k = __builtin_ctz(mask);
    sum[mask] = sum[mask & (mask - 1u)] + w[k];
  }
  auto take_max = [](double a, double b) { return a > b ? a : b; };
  auto take_sum = [](double a, double b) { return a + b; };
  // lanes: level t holds t non-empty lanes
  std::vector<Choice> lane(lanes + 1);
  lane[1].val = sum;
  lane[1].val[0] = kBig;
  lane[1].arg.assign((size_t)full + 1, 0u);
  for (int t = 2; t <= lanes; ++t) split_level(sum, lane[t - 1], lane[t], n, take_max);
  const std::vector<double>& round_val = lane[lanes].val;  // one round: exactly `lanes` lanes
  std::vector<Choice> rnd(rounds + 1);
  rnd[1].val = round_val;
  rnd[1].arg.assign((size_t)full + 1, 0u);
  for (int r = 2; r <= rounds; ++r) split_level(round_val, rnd[r - 1], rnd[r], n, take_sum);
  if (!(rnd[rounds].val[full] < kBig)) return set_error(AUGTREE_ERR_INVALID_ARGUMENT, "no assignment with every cell non-empty");
  *cost = rnd[rounds].val[full];
  // reconstruct: peel rounds (the part holding the lowest unit is the last round), then lanes
  uint32_t mask = full;
  for (int r = rounds; r >= 1; --r) {
    const uint32_t rmask = r == 1 ? mask : rnd[r].arg[mask];
    uint32_t lm = rmask;
    for (int t = lanes; t >= 1; --t) {
      const uint32_t part = t == 1 ? lm : lane[t].arg[lm];
      for (int k = 0; k < n; ++k)
        if (part >> k & 1u) cell[k] = (r - 1) * lanes + (t - 1);
      lm ^= part;
    }
    mask ^= rmask;
  }
  return AUGTREE_OK;
}

augtree_status assign_greedy(const double* w, int n, int rounds, int lanes, int32_t* cell, double* cost) {
  std::vector<int> order(n);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return w[a] > w[b]; });
  const int cells = rounds * lanes;
  std::vector<double> load(cells, 0.0), rmax(rounds, 0.0);
  std::vector<int> count(cells, 0);
  int empty = cells;
  for (int k : order) {
    int best = -1;
    double best_inc = kBig;
    for (int c = 0; c < cells; ++c) {
      if (empty > 0 && count[c] != 0) continue;  // fill every cell first
      const int r = c / lanes;
      const double inc = std::max(rmax[r], load[c] + w[k]) - rmax[r];
      if (inc < best_inc || (inc == best_inc && best >= 0 && load[c] < load[best])) {
        best = c;
        best_inc = inc;
      }
    }
    cell[k] = best;
    if (count[best]++ == 0) --empty;
    load[best] += w[k];
    rmax[best / lanes] = std::max(rmax[best / lanes], load[best]);
  }
  double total = 0.0;
  for (int r = 0; r < rounds; ++r) total += rmax[r];
  *cost = total;
  return AUGTREE_OK;
}

}  // namespace
}  // namespace augtree

using namespace augtree;

extern "C" augtree_status augtree_assign_units(const double* w, int32_t num_units, int32_t rounds, int32_t lanes,
                                                int32_t exact_max, int32_t* cell, double* cost) {
  if (w == nullptr || cell == nullptr || cost == nullptr)
    return set_error(AUGTREE_ERR_INVALID_ARGUMENT, "augtree_assign_units: NULL pointer");
  if (num_units < 1 || rounds < 1 || lanes < 1)
    return set_error(AUGTREE_ERR_INVALID_ARGUMENT, "augtree_assign_units: num_units, rounds and lanes must be >= 1");
  if ((int64_t)rounds * lanes > num_units)
    return set_error(AUGTREE_ERR_INVALID_ARGUMENT, "augtree_assign_units: fewer units than grid cells (every cell needs a unit)");
  if (exact_max < 0 || exact_max > AUGTREE_ASSIGN_EXACT_MAX)
    return set_error(AUGTREE_ERR_INVALID_ARGUMENT, "augtree_assign_units: exact_max outside [0, AUGTREE_ASSIGN_EXACT_MAX]");
  for (int k = 0; k < num_units; ++k)
    if (!isfinite(w[k]) || w[k] < 0.0)
      return set_error(AUGTREE_ERR_INVALID_ARGUMENT, "augtree_assign_units: weights must be finite and >= 0");
  try {
    if (num_units <= exact_max) return assign_exact(w, num_units, rounds, lanes, cell, cost);
    return assign_greedy(w, num_units, rounds, lanes, cell, cost);
  } catch (...) {
    return set_error(AUGTREE_ERR_INVALID_ARGUMENT, "augtree_assign_units: out of host memory");
  }
}
