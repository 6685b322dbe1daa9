// Per-expert format allocation for the routed experts of a stack: which of
// ternary (TERN160), Q2_0 and Q3 each expert is packed in.
//
// "[Strata] DeepSeek V4.1 Flash on a single 4090", section 5.1: the byte
// budget is that of the whole stack in Q2_0 (budget neutral); a Lagrangian
// relaxation with bisection on the multiplier, then a greedy fill of what is
// left; the cost of an expert's format is its held-out output error divided
// by its layer's routed output energy, so that every layer weighs the same,
// with the first two and the last three layers counted twice; at most half of
// a layer's experts ternary; experts seen by fewer than 8 held-out tokens
// stay Q2_0.  Host code only (no device).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <queue>
#include <vector>

#include "../../include/moe.h"

namespace {

constexpr int kF = 3;                                    // candidate formats, in this order
constexpr int kFmtTag[kF] = {MOE_FMT_TERN160, MOE_FMT_Q2_0, MOE_FMT_Q3};
constexpr int kTern = 0, kQ2 = 1;
// the order in which equal values are taken: Q2_0 first, then ternary, then Q3
constexpr int kTieOrder[kF] = {kQ2, kTern, 2};

struct Problem {
  int L, E;
  std::vector<double> cost;        // [L][E][kF]
  std::vector<uint8_t> locked;     // [L][E]
  double bytes[kF];
  int cap;                         // ternary experts allowed per layer
};

// The Lagrangian choice for one multiplier: per expert the format of least
// cost + lam * bytes (ties in kTieOrder), then per layer the cap on ternary
// experts: those whose second-best value is closest to their ternary value go
// back to their best other format (ties: the higher expert id first).
void choose(const Problem& p, double lam, std::vector<int8_t>& f) {
  std::vector<std::pair<double, int>> tern;
  for (int l = 0; l < p.L; ++l) {
    tern.clear();
    for (int e = 0; e < p.E; ++e) {
      const size_t i = static_cast<size_t>(l) * p.E + e;
      if (p.locked[i]) {
        f[i] = kQ2;
        continue;
      }
      int best = -1;
      double bv = 0.0;
      for (int o = 0; o < kF; ++o) {
        const int c = kTieOrder[o];
        const double v = p.cost[i * kF + c] + lam * p.bytes[c];
        if (best < 0 || v < bv) {
          best = c;
          bv = v;
        }
      }
      f[i] = static_cast<int8_t>(best);
      if (best == kTern) {
        double alt = 0.0;
        bool have = false;
        for (int o = 0; o < kF; ++o) {
          const int c = kTieOrder[o];
          if (c == kTern) continue;
          const double v = p.cost[i * kF + c] + lam * p.bytes[c];
          if (!have || v < alt) {
            alt = v;
            have = true;
          }
        }
        tern.emplace_back(alt - bv, e);
      }
    }
    const int over = static_cast<int>(tern.size()) - p.cap;
    if (over <= 0) continue;
    std::sort(tern.begin(), tern.end(), [](const std::pair<double, int>& a, const std::pair<double, int>& b) {
      return a.first != b.first ? a.first < b.first : a.second > b.second;
    });
    for (int q = 0; q < over; ++q) {
      const size_t i = static_cast<size_t>(l) * p.E + tern[static_cast<size_t>(q)].second;
      int best = -1;
      double bv = 0.0;
      for (int o = 0; o < kF; ++o) {
        const int c = kTieOrder[o];
        if (c == kTern) continue;
        const double v = p.cost[i * kF + c] + lam * p.bytes[c];
        if (best < 0 || v < bv) {
          best = c;
          bv = v;
        }
      }
      f[i] = static_cast<int8_t>(best);
    }
  }
}

double total_bytes(const Problem& p, const std::vector<int8_t>& f) {
  double b = 0.0;
  for (int8_t c : f) b += p.bytes[c];
  return b;
}

}  // namespace

extern "C" int moe_allocate_formats(int32_t n_layers, int32_t n_experts, const double* err,
                                    const int32_t* tokens, const double* energy, const uint64_t* fmt_bytes,
                                    double max_tern_frac, int32_t min_tokens, int32_t edge_first,
                                    int32_t edge_last, uint8_t* fmt_out, double* cost_out,
                                    uint64_t* bytes_out) {
  if (n_layers <= 0 || n_experts <= 0 || !err || !tokens || !energy || !fmt_bytes || !fmt_out)
    return MOE_EINVAL;
  if (!(max_tern_frac >= 0.0 && max_tern_frac <= 1.0) || min_tokens < 0 || edge_first < 0 || edge_last < 0)
    return MOE_EINVAL;
  if (!(fmt_bytes[0] < fmt_bytes[1] && fmt_bytes[1] < fmt_bytes[2])) return MOE_EINVAL;
  Problem p;
  p.L = n_layers;
  p.E = n_experts;
  const size_t n = static_cast<size_t>(n_layers) * n_experts;
  p.cost.resize(n * kF);
  p.locked.resize(n);
  for (int c = 0; c < kF; ++c) p.bytes[c] = static_cast<double>(fmt_bytes[c]);
  p.cap = static_cast<int>(std::floor(max_tern_frac * n_experts));
  for (int l = 0; l < n_layers; ++l) {
    if (!(energy[l] > 0.0) || !std::isfinite(energy[l])) return MOE_EINVAL;
    const double wl = (l < edge_first || l >= n_layers - edge_last) ? 2.0 : 1.0;
    for (int e = 0; e < n_experts; ++e) {
      const size_t i = static_cast<size_t>(l) * n_experts + e;
      p.locked[i] = tokens[i] < min_tokens ? 1 : 0;
      for (int c = 0; c < kF; ++c) {
        const double v = err[i * kF + c];
        if (!(v >= 0.0) || !std::isfinite(v)) return MOE_EINVAL;
        p.cost[i * kF + c] = wl * v / energy[l];
      }
    }
  }
  const double budget = static_cast<double>(n) * p.bytes[kQ2];   // every expert Q2_0
  std::vector<int8_t> f(n), g(n);
  choose(p, 0.0, f);
  if (total_bytes(p, f) > budget) {
    // the multiplier at which the choice fits: bytes fall as it grows, and at
    // hi every free expert that the cap allows is ternary, which fits
    double lo = 0.0, hi = 1.0;
    for (;;) {
      choose(p, hi, g);
      if (total_bytes(p, g) <= budget || hi > 1e300) break;
      lo = hi;
      hi *= 2.0;
    }
    for (int it = 0; it < 200 && hi - lo > 0.0; ++it) {
      const double mid = lo + (hi - lo) * 0.5;
      if (mid <= lo || mid >= hi) break;
      choose(p, mid, g);
      if (total_bytes(p, g) <= budget) hi = mid;
      else lo = mid;
    }
    choose(p, hi, f);
  }
  // greedy fill: the budget left goes to the upgrades (a larger format of
  // lower cost) with the largest cost saving per byte that still fit
  double left = budget - total_bytes(p, f);
  struct Up {
    double ratio;
    size_t i;
    int to;
    int ver;
  };
  auto worse = [](const Up& a, const Up& b) {   // priority: ratio desc, then (i, to) asc
    if (a.ratio != b.ratio) return a.ratio < b.ratio;
    if (a.i != b.i) return a.i > b.i;
    return a.to > b.to;
  };
  std::priority_queue<Up, std::vector<Up>, decltype(worse)> heap(worse);
  std::vector<int> ver(n, 0);
  auto push_ups = [&](size_t i) {
    if (p.locked[i]) return;
    const int cur = f[i];
    for (int c = 0; c < kF; ++c) {
      const double extra = p.bytes[c] - p.bytes[cur];
      const double gain = p.cost[i * kF + cur] - p.cost[i * kF + c];
      if (extra > 0.0 && gain > 0.0) heap.push(Up{gain / extra, i, c, ver[i]});
    }
  };
  for (size_t i = 0; i < n; ++i) push_ups(i);
  while (!heap.empty()) {
    const Up u = heap.top();
    heap.pop();
    if (u.ver != ver[u.i]) continue;   // the expert changed since
    const double extra = p.bytes[u.to] - p.bytes[f[u.i]];
    if (extra > left) continue;
    left -= extra;
    f[u.i] = static_cast<int8_t>(u.to);
    ++ver[u.i];
    push_ups(u.i);
  }
  double cost = 0.0;
  for (size_t i = 0; i < n; ++i) {
    fmt_out[i] = static_cast<uint8_t>(kFmtTag[f[i]]);
    cost += p.cost[i * kF + f[i]];
  }
  if (cost_out) *cost_out = cost;
  if (bytes_out) *bytes_out = static_cast<uint64_t>(total_bytes(p, f));
  return MOE_OK;
}
