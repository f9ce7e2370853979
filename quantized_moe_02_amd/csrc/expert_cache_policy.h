// Slot policy of the expert cache (host code only, no HIP): which routed
// experts sit in the n device slots of one layer, and which to evict.
//
// Page "Show HN: Menjalankan GLM 5.2 di komputer lambat", section "Cara kerja
// eksekusi MoE berbasis streaming disk": routed experts live outside fast
// memory and are loaded through a least-recently-used cache per layer, with
// an optional pinned hot store.  Here the slow tier is host RAM and the fast
// one HBM; the policy is the same.
//
// Rules (deterministic, so that tests can predict every load):
//   - a request names a set of distinct experts; those already resident are
//     hits, the others misses;
//   - misses are placed in ascending expert order, each into the free slot
//     of lowest index, else into the evictable slot least recently used
//     (smallest stamp, then lowest index);
//   - a slot is evictable unless it is pinned, holds an expert of the same
//     request, or is protected (stamp >= the request's protect_from);
//   - a request that cannot place all its misses changes nothing;
//   - afterwards every slot of the request gets one new stamp (the clock
//     advances once per request).
#pragma once

#include <stdint.h>

#include <algorithm>
#include <utility>
#include <vector>

namespace qmoe {

class SlotPolicy {
 public:
  SlotPolicy(int n_experts, int n_slots)
      : slot_of_(n_experts, -1), expert_in_(n_slots, -1), stamp_(n_slots, 0), pinned_(n_slots, 0) {}

  int n_experts() const { return (int)slot_of_.size(); }
  int n_slots() const { return (int)expert_in_.size(); }
  int slot_of(int e) const { return slot_of_[e]; }
  int expert_in(int s) const { return expert_in_[s]; }
  bool pinned(int s) const { return pinned_[s] != 0; }
  uint64_t stamp(int s) const { return stamp_[s]; }
  uint64_t clock() const { return clock_; }

  // Makes the distinct experts `need` (ids in [0, n_experts)) resident.
  // loads: the (expert, slot) copies to perform; hits: how many were
  // resident.  Returns false, changing nothing, if the misses do not fit.
  bool acquire(std::vector<int> need, uint64_t protect_from,
               std::vector<std::pair<int, int>>& loads, int& hits) {
    std::sort(need.begin(), need.end());
    need.erase(std::unique(need.begin(), need.end()), need.end());
    loads.clear();
    hits = 0;
    std::vector<uint8_t> taken(expert_in_.size(), 0);   // slots this request keeps
    std::vector<int> misses;
    for (int e : need) {
      if (slot_of_[e] >= 0) {
        ++hits;
        taken[slot_of_[e]] = 1;
      } else {
        misses.push_back(e);
      }
    }
    for (int e : misses) {
      int best = -1;
      for (int s = 0; s < n_slots(); ++s) {
        if (taken[s] || pinned_[s]) continue;
        if (expert_in_[s] < 0) {   // free
          best = s;
          break;
        }
        if (stamp_[s] >= protect_from) continue;
        if (best < 0 || stamp_[s] < stamp_[best]) best = s;
      }
      if (best < 0) {
        loads.clear();
        return false;
      }
      taken[best] = 1;
      loads.emplace_back(e, best);
    }
    // commit
    ++clock_;
    for (const auto& l : loads) {
      const int old = expert_in_[l.second];
      if (old >= 0) {
        slot_of_[old] = -1;
        ++evictions_;
      }
      expert_in_[l.second] = l.first;
      slot_of_[l.first] = l.second;
    }
    for (int e : need) stamp_[slot_of_[e]] = clock_;
    return true;
  }

  // Pins the slots of resident experts (they are never evicted).
  void pin(const std::vector<int>& experts) {
    for (int e : experts)
      if (slot_of_[e] >= 0) pinned_[slot_of_[e]] = 1;
  }
  void unpin_all() { std::fill(pinned_.begin(), pinned_.end(), 0); }
  int n_pinned() const { return (int)std::count(pinned_.begin(), pinned_.end(), 1); }
  uint64_t evictions() const { return evictions_; }

 private:
  std::vector<int> slot_of_;     // [experts] slot or -1
  std::vector<int> expert_in_;   // [slots] expert or -1 (free)
  std::vector<uint64_t> stamp_;  // [slots] clock of the last request that used it
  std::vector<uint8_t> pinned_;  // [slots]
  uint64_t clock_ = 0;
  uint64_t evictions_ = 0;
};

}  // namespace qmoe
