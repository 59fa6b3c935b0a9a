// Least-recently-used cache of launch plans, with pinning.  Plain C++ (no HIP):
// the policy is tested on the host on its own.
//
// A pinned entry is never evicted: a HIP graph captured from a step keeps raw
// device pointers into its plan's tables, so a plan used while its stream is
// being captured must outlive every replay.  Eviction removes the least
// recently used unpinned entries once more than `capacity` entries are held;
// pinned entries do not count against the capacity.  Evicted values are handed
// back to the caller, who drops them after releasing its own lock (a plan's
// destructor waits for the device).
#pragma once

#include <cstddef>
#include <list>
#include <memory>
#include <string>
#include <utility>
#include <vector>

namespace muon {

template <typename V>
class PlanCache {
  public:
    explicit PlanCache(size_t capacity) : capacity_(capacity) {}

    // The value cached under key, moved to the front (most recent), or null.
    // pin == true pins the entry.
    std::shared_ptr<V> find(const std::string& key, bool pin) {
        for (auto it = entries_.begin(); it != entries_.end(); ++it) {
            if (it->key == key) {
                entries_.splice(entries_.begin(), entries_, it);
                Entry& e = entries_.front();
                if (pin && !e.pinned) {
                    e.pinned = true;
                    ++pinned_;
                }
                return e.value;
            }
        }
        return nullptr;
    }

    // Inserts value under key at the front; returns the evicted values.
    std::vector<std::shared_ptr<V>> insert(std::string key, std::shared_ptr<V> value, bool pin) {
        entries_.push_front(Entry{std::move(key), std::move(value), pin});
        if (pin) ++pinned_;
        std::vector<std::shared_ptr<V>> evicted;
        while (entries_.size() - pinned_ > capacity_) {
            // least recently used unpinned entry
            auto victim = entries_.end();
            for (auto it = entries_.end(); it != entries_.begin();) {
                --it;
                if (!it->pinned) {
                    victim = it;
                    break;
                }
            }
            if (victim == entries_.end()) break;
            evicted.push_back(std::move(victim->value));
            entries_.erase(victim);
        }
        return evicted;
    }

    size_t size() const { return entries_.size(); }
    size_t pinned() const { return pinned_; }
    // Keys from most to least recently used.
    std::vector<std::string> keys() const {
        std::vector<std::string> out;
        for (const Entry& e : entries_) out.push_back(e.key);
        return out;
    }

  private:
    struct Entry {
        std::string key;
        std::shared_ptr<V> value;
        bool pinned;
    };
    size_t capacity_;
    size_t pinned_ = 0;
    std::list<Entry> entries_;
};

}  // namespace muon
