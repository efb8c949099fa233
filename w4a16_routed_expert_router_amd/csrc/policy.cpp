// Host-side decision procedure of the expert-slot pool (no HIP dependency).
//
// The pool keeps C slots per routed layer.  A routed group whose experts are all
// resident reads existing copies; each miss takes a free slot or evicts a
// resident expert outside the group, discarding its GPU copy ("Horizon RunMap",
// "Partial-residency contract: immutable authority and miss lifecycle").
// Victim rules: least recently used / least frequently used ("An
// expert-offloading engine, from scratch", "Terms used here", "What the numbers
// say"), and the score frequency*1000 - age with frequencies scaled by 0.75
// after every 2*capacity misses ("F51 Nitro / Nitro-MoE", "Layer 1 - expert
// persistence cache").
//
// Details the pages leave open, as implemented:
//   - one clock tick per access call (one routed group);
//   - the group is processed in ascending expert id, every hit first, then every
//     miss; a miss takes the lowest-index free slot, else the victim with the
//     smallest key among resident experts not in the group;
//   - keys: LRU (last, id); LFU (count, last, id) with count = number of calls
//     that named the expert, kept across evictions; LRU-FREQ
//     (sfreq*1000 - (clock - last), id) in double, sfreq = 1 on fill and +1 per
//     hit, all sfreq *= 0.75 right after the miss that completes each 2*C.
//
// Next-layer prefetch: the next layer's experts are guessed by running its
// router on the current state, and their reads start early so that they
// overlap with computing ("An expert-offloading engine, from scratch", "Terms
// used here" and "What the numbers say").  As implemented, a prefetch neither
// ticks the clock nor counts as a use; each guessed expert that is not
// resident is filled like a miss (last = the current clock, LFU count
// unchanged, sfreq = 1), is not a miss for the LRU-FREQ decay, and stays
// pending until an access names it, which counts a hit on the prefetched copy.
//
// Static / hybrid hot sets ("An expert-offloading engine, from scratch", "What
// the numbers say": a hot set measured on one prompt did worse than LFU on
// another; "F51 Nitro / Nitro-MoE", "The simulator": static per-layer and
// global hot sets against dynamic LRU): pinned experts fill slots 0 .. n-1 of a
// cold pool in ascending id and are never victims; the other slots stay
// dynamic, and a group fits when its experts outside the hot set number at
// most C - n.
#include "policy.hpp"

#include <algorithm>

namespace moe {

PolicyEngine::PolicyEngine(int policy, int n_experts, int capacity, int layer)
    : policy_(policy), E_(n_experts), C_(capacity), layer_(layer),
      pending_(n_experts, 0), pinned_(n_experts, 0), slot_of_(n_experts, -1), expert_in_(capacity, -1), last_(n_experts, 0),
      count_(n_experts, 0), sfreq_(capacity, 0.0) {}

#pragma clang fp contract(off)
static inline double freq_score(double sfreq, int64_t clock, int64_t last) {
  const double a = sfreq * 1000.0;
  const double b = (double)(clock - last);
  return a - b;
}

bool PolicyEngine::less_key(int a, int b) const {
  // true when expert a is a better victim than expert b
  switch (policy_) {
    case 1:  // LRU
      if (last_[a] != last_[b]) return last_[a] < last_[b];
      return a < b;
    case 2:  // LFU
      if (count_[a] != count_[b]) return count_[a] < count_[b];
      if (last_[a] != last_[b]) return last_[a] < last_[b];
      return a < b;
    default: {  // LRU-FREQ
      const double sa = freq_score(sfreq_[slot_of_[a]], clock_, last_[a]);
      const double sb = freq_score(sfreq_[slot_of_[b]], clock_, last_[b]);
      if (sa != sb) return sa < sb;
      return a < b;
    }
  }
}

int PolicyEngine::check_group(const int32_t* experts, int n, std::vector<int32_t>& g) const {
  if (n < 0) return 1;
  if (n > C_) return 2;
  g.assign(experts, experts + n);
  for (int e : g)
    if (e < 0 || e >= E_) return 1;
  std::sort(g.begin(), g.end());
  for (int i = 1; i < n; ++i)
    if (g[i] == g[i - 1]) return 1;
  int outside = 0;
  for (int e : g) outside += pinned_[e] ? 0 : 1;
  if (outside > C_ - n_pinned_) return 2;
  return 0;
}

int PolicyEngine::pin(const int32_t* experts, int n, int step, std::vector<Decision>& out) {
  out.clear();
  std::vector<int32_t> g;
  if (n < 0) return 1;
  g.assign(experts, experts + n);
  for (int e : g)
    if (e < 0 || e >= E_) return 1;
  std::sort(g.begin(), g.end());
  for (int i = 1; i < n; ++i)
    if (g[i] == g[i - 1]) return 1;
  if (n >= C_) return 2;
  bool cold = clock_ == 0 && n_pinned_ == 0;
  for (int s = 0; s < C_; ++s) cold = cold && expert_in_[s] < 0;
  if (!cold) return 3;
  for (int i = 0; i < n; ++i) {
    const int e = g[i];
    expert_in_[i] = e;
    slot_of_[e] = i;
    last_[e] = 0;
    count_[e] = 0;
    sfreq_[i] = 1.0;
    pinned_[e] = 1;
    out.push_back(Decision{e, i, -1, false, kPin});
  }
  n_pinned_ = n;
  for (const Decision& d : out)
    log_.push_back(moe_cache_event{step, layer_, d.expert, d.kind, d.slot, d.victim});
  return 0;
}

int PolicyEngine::take_slot(const std::vector<char>& in_group, int& victim) {
  victim = -1;
  for (int s = 0; s < C_; ++s)
    if (expert_in_[s] < 0) return s;
  for (int s = 0; s < C_; ++s) {
    const int x = expert_in_[s];
    if (in_group[x] || pinned_[x]) continue;
    if (victim < 0 || less_key(x, victim)) victim = x;
  }
  const int slot = slot_of_[victim];
  slot_of_[victim] = -1;
  pending_[victim] = 0;
  return slot;
}

int PolicyEngine::access(const int32_t* experts, int n, int step, std::vector<Decision>& out) {
  out.clear();
  std::vector<int32_t> g;
  if (const int rc = check_group(experts, n, g)) return rc;
  std::vector<char> in_group(E_, 0);
  for (int e : g) in_group[e] = 1;
  ++clock_;
  std::vector<char> hit(n, 0);
  for (int i = 0; i < n; ++i) {
    const int e = g[i];
    const int s = slot_of_[e];
    if (s < 0) continue;
    hit[i] = 1;
    last_[e] = clock_;
    count_[e] += 1;
    sfreq_[s] += 1.0;
    ++hits_;
    int kind = kHit;
    if (pending_[e]) {
      pending_[e] = 0;
      ++prefetch_used_;
      kind = kPrefetchHit;
    }
    out.push_back(Decision{e, s, -1, true, kind});
  }
  for (int i = 0; i < n; ++i) {
    if (hit[i]) continue;
    const int e = g[i];
    int victim = -1;
    const int slot = take_slot(in_group, victim);
    expert_in_[slot] = e;
    slot_of_[e] = slot;
    last_[e] = clock_;
    count_[e] += 1;
    sfreq_[slot] = 1.0;
    ++misses_;
    out.push_back(Decision{e, slot, victim, false, kMiss});
    if (policy_ == 3 && misses_ % (2 * (int64_t)C_) == 0)
      for (double& f : sfreq_) f *= 0.75;
  }
  for (const Decision& d : out)
    log_.push_back(moe_cache_event{step, layer_, d.expert, d.kind, d.slot, d.victim});
  return 0;
}

int PolicyEngine::prefetch(const int32_t* experts, int n, int step, std::vector<Decision>& out) {
  out.clear();
  std::vector<int32_t> g;
  if (const int rc = check_group(experts, n, g)) return rc;
  std::vector<char> in_group(E_, 0);
  for (int e : g) in_group[e] = 1;
  for (int i = 0; i < n; ++i) {
    const int e = g[i];
    if (slot_of_[e] >= 0) continue;
    int victim = -1;
    const int slot = take_slot(in_group, victim);
    expert_in_[slot] = e;
    slot_of_[e] = slot;
    last_[e] = clock_;
    sfreq_[slot] = 1.0;
    pending_[e] = 1;
    ++prefetches_;
    out.push_back(Decision{e, slot, victim, false, kPrefetch});
  }
  for (const Decision& d : out)
    log_.push_back(moe_cache_event{step, layer_, d.expert, d.kind, d.slot, d.victim});
  return 0;
}

}  // namespace moe

// ---- C ABI of the host-only engine ---------------------------------------------
struct moe_policy_engine {
  moe::PolicyEngine eng;
};

extern "C" {

moe_policy_engine* moe_policy_new(int32_t policy, int32_t n_experts, int32_t capacity,
                                  int32_t layer) {
  if (policy < 1 || policy > 3 || n_experts < 1 || capacity < 1) return nullptr;
  return new moe_policy_engine{moe::PolicyEngine(policy, n_experts, capacity, layer)};
}

void moe_policy_free(moe_policy_engine* p) { delete p; }

moe_status moe_policy_access(moe_policy_engine* p, const int32_t* experts, int32_t n,
                             int32_t step, int32_t* slots) {
  if (!p || (n > 0 && (!experts || !slots))) return MOE_E_ARG;
  std::vector<moe::PolicyEngine::Decision> d;
  const int rc = p->eng.access(experts, n, step, d);
  if (rc == 1) return MOE_E_ARG;
  if (rc == 2) return MOE_E_CAPACITY;
  for (int i = 0; i < n; ++i) slots[i] = p->eng.slot_of(experts[i]);
  return MOE_OK;
}

moe_status moe_policy_prefetch(moe_policy_engine* p, const int32_t* experts, int32_t n, int32_t step) {
  if (!p || (n > 0 && !experts)) return MOE_E_ARG;
  std::vector<moe::PolicyEngine::Decision> d;
  const int rc = p->eng.prefetch(experts, n, step, d);
  if (rc == 1) return MOE_E_ARG;
  if (rc == 2) return MOE_E_CAPACITY;
  return MOE_OK;
}
moe_status moe_policy_pin(moe_policy_engine* p, const int32_t* experts, int32_t n, int32_t step) {
  if (!p || (n > 0 && !experts)) return MOE_E_ARG;
  std::vector<moe::PolicyEngine::Decision> d;
  const int rc = p->eng.pin(experts, n, step, d);
  if (rc == 2) return MOE_E_CAPACITY;
  return rc == 0 ? MOE_OK : MOE_E_ARG;
}
int32_t moe_policy_event_count(const moe_policy_engine* p) {
  return p ? (int32_t)p->eng.log().size() : 0;
}

int32_t moe_policy_events(const moe_policy_engine* p, moe_cache_event* buf, int32_t cap) {
  if (!p || !buf || cap <= 0) return 0;
  const auto& lg = p->eng.log();
  const int32_t n = std::min<int32_t>(cap, (int32_t)lg.size());
  std::copy(lg.begin(), lg.begin() + n, buf);
  return n;
}

}  // extern "C"
