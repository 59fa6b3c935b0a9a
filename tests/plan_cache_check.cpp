// Host-only checks of the launch-plan cache policy (least recently used
// eviction; pinned plans, the ones a captured graph refers to, are never
// evicted).  Built with g++ by tests/test_plan_cache.py; prints "ok" on success.
#include <cstdio>
#include <cstdlib>
#include <memory>
#include <string>
#include <vector>

#include "plan_cache.h"

namespace {

int g_alive = 0;
struct Plan {
    int id;
    explicit Plan(int i) : id(i) { ++g_alive; }
    ~Plan() { --g_alive; }
};

#define CHECK(cond)                                                    \
    do {                                                               \
        if (!(cond)) {                                                 \
            std::printf("check failed at line %d: %s\n", __LINE__, #cond); \
            std::exit(1);                                              \
        }                                                              \
    } while (0)

std::string key(int i) { return "set" + std::to_string(i); }

}  // namespace

int main() {
    using muon::PlanCache;
    {
        // plain LRU: capacity 3, the least recently used goes first
        PlanCache<Plan> c(3);
        for (int i = 0; i < 3; ++i) CHECK(c.insert(key(i), std::make_shared<Plan>(i), false).empty());
        CHECK(c.find(key(0), false) != nullptr);  // 0 becomes most recent
        auto ev = c.insert(key(3), std::make_shared<Plan>(3), false);
        CHECK(ev.size() == 1 && ev[0]->id == 1);
        CHECK(c.find(key(1), false) == nullptr);
        CHECK(c.size() == 3);
        ev.clear();
        CHECK(g_alive == 3);
    }
    CHECK(g_alive == 0);
    {
        // a pinned plan survives any number of later sets
        PlanCache<Plan> c(2);
        c.insert(key(0), std::make_shared<Plan>(0), false);
        CHECK(c.find(key(0), true) != nullptr);  // used under capture: pinned
        std::weak_ptr<Plan> pinned = c.find(key(0), false);
        for (int i = 1; i <= 100; ++i) {
            auto ev = c.insert(key(i), std::make_shared<Plan>(i), false);
            for (auto& p : ev) CHECK(p->id != 0);
        }
        CHECK(!pinned.expired());
        CHECK(c.find(key(0), false) != nullptr);
        CHECK(c.pinned() == 1);
        CHECK(c.size() == 3);  // the pinned plan does not count against the capacity
        CHECK(g_alive == 3);
    }
    CHECK(g_alive == 0);
    {
        // inserting pinned; every entry pinned: nothing is evicted
        PlanCache<Plan> c(1);
        for (int i = 0; i < 5; ++i) CHECK(c.insert(key(i), std::make_shared<Plan>(i), true).empty());
        CHECK(c.size() == 5 && c.pinned() == 5);
        // one unpinned on top of capacity 1: kept; a second one evicts the first unpinned
        CHECK(c.insert(key(5), std::make_shared<Plan>(5), false).empty());
        auto ev = c.insert(key(6), std::make_shared<Plan>(6), false);
        CHECK(ev.size() == 1 && ev[0]->id == 5);
        for (int i = 0; i < 5; ++i) CHECK(c.find(key(i), false) != nullptr);
    }
    {
        // an evicted plan still held by a caller stays alive until released
        PlanCache<Plan> c(1);
        std::shared_ptr<Plan> held = std::make_shared<Plan>(0);
        c.insert(key(0), held, false);
        auto ev = c.insert(key(1), std::make_shared<Plan>(1), false);
        CHECK(ev.size() == 1);
        ev.clear();
        CHECK(held->id == 0 && held.use_count() == 1);
        // pinning an entry twice counts it once
        c.find(key(1), true);
        c.find(key(1), true);
        CHECK(c.pinned() == 1);
        std::vector<std::string> k = c.keys();
        CHECK(k.size() == 1 && k[0] == key(1));
    }
    std::printf("ok\n");
    return 0;
}
