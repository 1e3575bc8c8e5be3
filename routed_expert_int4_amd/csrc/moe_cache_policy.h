// Slot bookkeeping of the per-layer expert cache: which expert sits in
// which slot and which slot to reuse.  Pure host logic with no HIP calls, so
// it can be exercised on the CPU; the HIP side (copies, events) lives in
// moe_cache.cpp.
#pragma once

#include <cstdint>
#include <vector>

namespace moe {

class SlotPolicy {
public:
    SlotPolicy(int n_experts, int n_slots)
        : slot_of_(n_experts, -1), expert_in_(n_slots, -1), last_use_(n_slots, 0), pinned_(n_slots, 0) {}

    int n_slots() const { return (int)expert_in_.size(); }
    int n_experts() const { return (int)slot_of_.size(); }
    int slot_of(int e) const { return slot_of_[e]; }
    int expert_in(int s) const { return expert_in_[s]; }
    int n_pinned() const { return n_pinned_; }
    bool is_pinned(int e) const { return slot_of_[e] >= 0 && pinned_[slot_of_[e]]; }

    // Marks a resident expert as used now (LRU order).
    void touch(int e) { last_use_[slot_of_[e]] = ++clock_; }

    // Pins / unpins a resident expert: a pinned slot is never chosen for
    // eviction (the hot store of the learning cache).
    void pin(int e) {
        const int s = slot_of_[e];
        if (s >= 0 && !pinned_[s]) {
            pinned_[s] = 1;
            ++n_pinned_;
        }
    }
    void unpin(int e) {
        const int s = slot_of_[e];
        if (s >= 0 && pinned_[s]) {
            pinned_[s] = 0;
            --n_pinned_;
        }
    }

    // Chooses the slot for a missing expert: a free slot if there is one,
    // else the least recently used unpinned slot whose expert is not in
    // `protect` (the experts the current token needs).  Returns -1 if none
    // qualifies.  On success the previous occupant (if any) is returned in
    // *evicted.
    int assign(int e, const std::vector<int>& protect, int* evicted) {
        int best = -1;
        for (int s = 0; s < n_slots(); ++s) {
            if (expert_in_[s] < 0) {
                best = s;
                break;
            }
            if (pinned_[s]) continue;
            bool held = false;
            for (int p : protect) held = held || (expert_in_[s] == p);
            if (held) continue;
            if (best < 0 || last_use_[s] < last_use_[best]) best = s;
        }
        *evicted = -1;
        if (best < 0) return -1;
        if (expert_in_[best] >= 0) {
            *evicted = expert_in_[best];
            slot_of_[expert_in_[best]] = -1;
        }
        expert_in_[best] = e;
        slot_of_[e] = best;
        last_use_[best] = ++clock_;
        return best;
    }

    // Frees the slot of e (no-op if e is not resident).  Returns the slot or -1.
    int release(int e) {
        const int s = slot_of_[e];
        if (s < 0) return -1;
        unpin(e);
        slot_of_[e] = -1;
        expert_in_[s] = -1;
        last_use_[s] = 0;
        return s;
    }

private:
    std::vector<int> slot_of_;
    std::vector<int> expert_in_;
    std::vector<uint64_t> last_use_;
    std::vector<char> pinned_;
    int n_pinned_ = 0;
    uint64_t clock_ = 0;
};

}  // namespace moe
