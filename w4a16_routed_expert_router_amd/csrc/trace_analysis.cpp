// Offline analysis of routing traces (host only, no HIP dependency).
//
// Captured router traces are replayed through cache policies offline and the
// hit rate is reported per capacity ("F51 Nitro / Nitro-MoE", "The
// simulator"); LRU and LFU hit rates at a fixed cache size are compared ("An
// expert-offloading engine, from scratch", "What the numbers say"); the share
// of selections that a static pin of the most popular experts would serve is
// quoted ("F51 Nitro / Nitro-MoE", "Layer 1 - expert persistence cache").
//
// A trace is one layer's routed groups, row-major [n_steps, width] int32; an
// entry < 0 is padding and an expert named twice in one row counts once.
//
// Definitions used (the pages name these analyses without defining them):
//   - OPT is Belady's farthest-next-use rule carried over to groups: every
//     expert of a step's group must be resident at once, so a miss takes a free
//     slot if there is one, else evicts the resident expert outside the group
//     whose next use (the first later step naming it) is farthest away, an
//     expert never named again counting as infinitely far, ties to the lower
//     id.  Hits are counted before the misses of the same step are filled.
//   - selection count of an expert = steps whose group names it; the top-p
//     share = the summed counts of the ceil(p * E) most-selected experts (ties
//     to the lower id) over all selections; entropy in bits of the selection
//     frequencies; coverage(C) = the top-C share, i.e. the hit rate of a static
//     pin of those C experts.
#include <math.h>

#include <algorithm>
#include <limits>
#include <vector>

#include "policy.hpp"

namespace {

// Rows of the trace as ascending distinct ids; false on an id out of range.
bool trace_groups(const int32_t* ids, int32_t n_steps, int32_t width, int32_t n_experts,
                  std::vector<std::vector<int32_t>>& out) {
  out.assign(n_steps, {});
  for (int32_t t = 0; t < n_steps; ++t) {
    std::vector<int32_t>& g = out[t];
    for (int32_t j = 0; j < width; ++j) {
      const int32_t e = ids[(int64_t)t * width + j];
      if (e < 0) continue;
      if (e >= n_experts) return false;
      g.push_back(e);
    }
    std::sort(g.begin(), g.end());
    g.erase(std::unique(g.begin(), g.end()), g.end());
  }
  return true;
}

bool bad_trace_args(const int32_t* ids, int32_t n_steps, int32_t width, int32_t n_experts) {
  return n_steps < 0 || width < 0 || n_experts < 1 || (n_steps > 0 && width > 0 && !ids);
}

// Selection counts in id order.
std::vector<int64_t> selection_counts(const std::vector<std::vector<int32_t>>& gs, int32_t n_experts) {
  std::vector<int64_t> c(n_experts, 0);
  for (const auto& g : gs)
    for (int32_t e : g) c[e] += 1;
  return c;
}

double top_share_of(const std::vector<int64_t>& c, int64_t n_top) {
  int64_t total = 0;
  for (int64_t v : c) total += v;
  if (total == 0) return 0.0;
  std::vector<int32_t> order(c.size());
  for (size_t e = 0; e < c.size(); ++e) order[e] = (int32_t)e;
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return c[a] > c[b]; });
  int64_t s = 0;
  for (int64_t i = 0; i < n_top && i < (int64_t)order.size(); ++i) s += c[order[i]];
  return (double)s / (double)total;
}

}  // namespace

extern "C" {

moe_status moe_trace_opt(const int32_t* ids, int32_t n_steps, int32_t width, int32_t n_experts,
                         int32_t capacity, int64_t* hits, int64_t* misses) {
  if (bad_trace_args(ids, n_steps, width, n_experts) || capacity < 1 || !hits || !misses) return MOE_E_ARG;
  std::vector<std::vector<int32_t>> gs;
  if (!trace_groups(ids, n_steps, width, n_experts, gs)) return MOE_E_ARG;
  for (const auto& g : gs)
    if ((int32_t)g.size() > capacity) return MOE_E_CAPACITY;
  // nxt[t][i]: first step after t that names gs[t][i] (kNever if none)
  const int64_t kNever = std::numeric_limits<int64_t>::max();
  std::vector<std::vector<int64_t>> nxt(n_steps);
  {
    std::vector<int64_t> seen(n_experts, kNever);
    for (int32_t t = n_steps - 1; t >= 0; --t) {
      nxt[t].resize(gs[t].size());
      for (size_t i = 0; i < gs[t].size(); ++i) nxt[t][i] = seen[gs[t][i]];
      for (int32_t e : gs[t]) seen[e] = t;
    }
  }
  std::vector<char> resident(n_experts, 0), in_group(n_experts, 0);
  std::vector<int64_t> next_use(n_experts, kNever);  // of resident experts
  std::vector<int32_t> res_list;                     // resident experts
  int64_t h = 0, m = 0;
  for (int32_t t = 0; t < n_steps; ++t) {
    const auto& g = gs[t];
    for (int32_t e : g) in_group[e] = 1;
    for (int32_t e : g) h += resident[e] ? 1 : 0;
    for (size_t i = 0; i < g.size(); ++i) {
      const int32_t e = g[i];
      if (!resident[e]) {
        ++m;
        if ((int32_t)res_list.size() >= capacity) {
          int32_t vi = -1;
          for (size_t r = 0; r < res_list.size(); ++r) {
            const int32_t x = res_list[r];
            if (in_group[x]) continue;
            if (vi < 0) {
              vi = (int32_t)r;
              continue;
            }
            const int32_t v = res_list[vi];
            if (next_use[x] > next_use[v] || (next_use[x] == next_use[v] && x < v)) vi = (int32_t)r;
          }
          resident[res_list[vi]] = 0;
          res_list[vi] = res_list.back();
          res_list.pop_back();
        }
        resident[e] = 1;
        res_list.push_back(e);
      }
      next_use[e] = nxt[t][i];
    }
    for (int32_t e : g) in_group[e] = 0;
  }
  *hits = h;
  *misses = m;
  return MOE_OK;
}

moe_status moe_trace_policy(int32_t policy, const int32_t* ids, int32_t n_steps, int32_t width,
                            int32_t n_experts, int32_t capacity, int64_t* hits, int64_t* misses) {
  if (policy < MOE_POLICY_LRU || policy > MOE_POLICY_LRU_FREQ) return MOE_E_ARG;
  if (bad_trace_args(ids, n_steps, width, n_experts) || capacity < 1 || !hits || !misses) return MOE_E_ARG;
  std::vector<std::vector<int32_t>> gs;
  if (!trace_groups(ids, n_steps, width, n_experts, gs)) return MOE_E_ARG;
  for (const auto& g : gs)
    if ((int32_t)g.size() > capacity) return MOE_E_CAPACITY;
  moe::PolicyEngine eng(policy, n_experts, capacity, 0);
  std::vector<moe::PolicyEngine::Decision> d;
  for (int32_t t = 0; t < n_steps; ++t)
    if (eng.access(gs[t].data(), (int)gs[t].size(), t, d) != 0) return MOE_E_ARG;
  *hits = eng.hits();
  *misses = eng.misses();
  return MOE_OK;
}

moe_status moe_trace_policy_pinned(int32_t policy, const int32_t* ids, int32_t n_steps, int32_t width,
                                   int32_t n_experts, int32_t capacity, const int32_t* hot, int32_t n_hot,
                                   int64_t* hits, int64_t* misses) {
  if (policy < MOE_POLICY_LRU || policy > MOE_POLICY_LRU_FREQ) return MOE_E_ARG;
  if (bad_trace_args(ids, n_steps, width, n_experts) || capacity < 1 || !hits || !misses) return MOE_E_ARG;
  if (n_hot < 0 || (n_hot > 0 && !hot)) return MOE_E_ARG;
  std::vector<std::vector<int32_t>> gs;
  if (!trace_groups(ids, n_steps, width, n_experts, gs)) return MOE_E_ARG;
  moe::PolicyEngine eng(policy, n_experts, capacity, 0);
  std::vector<moe::PolicyEngine::Decision> d;
  const int prc = eng.pin(hot, n_hot, 0, d);
  if (prc == 2) return MOE_E_CAPACITY;
  if (prc != 0) return MOE_E_ARG;
  for (int32_t t = 0; t < n_steps; ++t) {
    const int rc = eng.access(gs[t].data(), (int)gs[t].size(), t, d);
    if (rc == 2) return MOE_E_CAPACITY;
    if (rc != 0) return MOE_E_ARG;
  }
  *hits = eng.hits();
  *misses = eng.misses();
  return MOE_OK;
}

moe_status moe_trace_top_share(const int32_t* ids, int32_t n_steps, int32_t width, int32_t n_experts,
                               int32_t n_top, double* share) {
  if (bad_trace_args(ids, n_steps, width, n_experts) || n_top < 0 || !share) return MOE_E_ARG;
  std::vector<std::vector<int32_t>> gs;
  if (!trace_groups(ids, n_steps, width, n_experts, gs)) return MOE_E_ARG;
  *share = top_share_of(selection_counts(gs, n_experts), n_top);
  return MOE_OK;
}

moe_status moe_trace_skew(const int32_t* ids, int32_t n_steps, int32_t width, int32_t n_experts,
                          moe_skew_report* out) {
  if (bad_trace_args(ids, n_steps, width, n_experts) || !out) return MOE_E_ARG;
  std::vector<std::vector<int32_t>> gs;
  if (!trace_groups(ids, n_steps, width, n_experts, gs)) return MOE_E_ARG;
  const std::vector<int64_t> c = selection_counts(gs, n_experts);
  int64_t total = 0;
  int32_t distinct = 0;
  for (int64_t v : c) {
    total += v;
    distinct += v > 0 ? 1 : 0;
  }
  double ent = 0.0;
  for (int64_t v : c)
    if (v) {
      const double p = (double)v / (double)total;
      ent -= p * log2(p);
    }
  out->top10 = top_share_of(c, (int64_t)ceil(0.1 * n_experts));
  out->top20 = top_share_of(c, (int64_t)ceil(0.2 * n_experts));
  out->top30 = top_share_of(c, (int64_t)ceil(0.3 * n_experts));
  out->entropy_bits = ent;
  out->distinct = distinct;
  out->selections = total;
  return MOE_OK;
}

}  // extern "C"
