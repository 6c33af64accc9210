// Which plan's tables each workspace region holds. A link call reads the plan tables from the
// workspace and writes its split partials and rotated keys there, so it may only run with the
// plan that was last copied into that region. An upload into any byte of a region ends the claim
// of every plan whose region it overlaps; a plan holds one region at a time.
#pragma once

#include <stdint.h>

#include <algorithm>
#include <vector>

namespace piclink {

template <typename Plan>
class WorkspaceLedger {
public:
    // `plan`'s tables are now in [base, base + bytes)
    void claim(const Plan *plan, const void *base, int64_t bytes) {
        const uintptr_t lo = reinterpret_cast<uintptr_t>(base), hi = lo + static_cast<uintptr_t>(bytes);
        entries_.erase(std::remove_if(entries_.begin(), entries_.end(),
                                      [&](const Entry &e) { return e.plan == plan || (e.lo < hi && lo < e.hi); }),
                       entries_.end());
        entries_.push_back({plan, lo, hi});
    }
    // true when the region starting at `base` still holds `plan`'s tables
    bool holds(const Plan *plan, const void *base) const {
        const uintptr_t lo = reinterpret_cast<uintptr_t>(base);
        for (const Entry &e : entries_)
            if (e.plan == plan) return e.lo == lo;
        return false;
    }
    // the plan is freed: its claim ends
    void drop(const Plan *plan) {
        entries_.erase(std::remove_if(entries_.begin(), entries_.end(), [&](const Entry &e) { return e.plan == plan; }),
                       entries_.end());
    }
    size_t size() const { return entries_.size(); }

private:
    struct Entry {
        const Plan *plan;
        uintptr_t lo, hi;
    };
    std::vector<Entry> entries_;
};

}  // namespace piclink
