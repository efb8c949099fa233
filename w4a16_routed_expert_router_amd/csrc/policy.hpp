// Slot-pool decision engine (host only, no HIP dependency).
#pragma once

#include <stdint.h>

#include <vector>

#include "../../include/moe_w4a16.h"

namespace moe {

class PolicyEngine {
 public:
  // event kinds (the `hit` field of moe_cache_event)
  enum Kind { kMiss = 0, kHit = 1, kPrefetch = 2, kPrefetchHit = 3, kPin = 4 };
  struct Decision {
    int32_t expert;
    int32_t slot;
    int32_t victim;  // -1 if none
    bool hit;        // resident when named (kHit or kPrefetchHit)
    int kind;
  };

  PolicyEngine(int policy, int n_experts, int capacity, int layer);

  // One routed group.  Returns 0 on success, 1 for a bad or repeated id,
  // 2 when n exceeds the capacity; on failure nothing changes.  `out` gets
  // the decisions in event order (hits ascending, then misses ascending).
  int access(const int32_t* experts, int n, int step, std::vector<Decision>& out);
  // Speculative fill of a guessed group (no clock tick, no use): each guessed
  // expert that is not resident is filled like a miss and stays pending until
  // an access names it.  Same return codes; `out` gets the fills.
  int prefetch(const int32_t* experts, int n, int step, std::vector<Decision>& out);
  // Hot set on a cold pool: the experts (ascending id) take slots 0 .. n-1 and
  // are never victims.  0 ok, 1 bad or repeated id, 2 n >= C (no dynamic slot
  // left), 3 the pool is not cold.  `out` gets the fills.
  int pin(const int32_t* experts, int n, int step, std::vector<Decision>& out);
  int pinned_count() const { return n_pinned_; }
  bool is_pinned(int e) const { return pinned_[e] != 0; }

  int32_t slot_of(int e) const { return slot_of_[e]; }
  const std::vector<moe_cache_event>& log() const { return log_; }
  int64_t hits() const { return hits_; }
  int64_t misses() const { return misses_; }
  int64_t prefetches() const { return prefetches_; }
  int64_t prefetch_used() const { return prefetch_used_; }
  int capacity() const { return C_; }

 private:
  bool less_key(int a, int b) const;
  int check_group(const int32_t* experts, int n, std::vector<int32_t>& g) const;
  // slot for a fill of a non-resident expert outside `in_group`: the lowest
  // free slot, else the victim's (which is evicted); victim out, -1 if none
  int take_slot(const std::vector<char>& in_group, int& victim);

  int policy_, E_, C_, layer_;
  int64_t clock_ = 0, misses_ = 0, hits_ = 0, prefetches_ = 0, prefetch_used_ = 0;
  std::vector<char> pending_;       // expert -> prefetched, not yet named by an access
  std::vector<char> pinned_;        // expert -> in the hot set (never a victim)
  int n_pinned_ = 0;
  std::vector<int32_t> slot_of_;    // expert -> slot or -1
  std::vector<int32_t> expert_in_;  // slot -> expert or -1
  std::vector<int64_t> last_;       // expert -> clock of last use
  std::vector<int64_t> count_;      // expert -> calls that named it
  std::vector<double> sfreq_;       // slot -> LRU-FREQ frequency
  std::vector<moe_cache_event> log_;
};

}  // namespace moe
