// Device allocations with a byte budget (see alloc.h).
#include "alloc.h"

#include <climits>
#include <mutex>
#include <unordered_map>

namespace gspmm {

namespace {

std::mutex g_mu;
std::unordered_map<void *, int64_t> g_sizes;   // live allocations
int64_t g_in_use = 0;

struct Budget {
    bool active = false;
    int64_t used = 0;          // bytes allocated minus bytes freed in this call
    int64_t peak = 0;
    int64_t allocs = 0;
    int64_t call_limit = INT64_MAX;
    int64_t plan_base = 0;
    int64_t plan_limit = INT64_MAX;
};

thread_local Budget t_budget;
thread_local int64_t t_limit = 0;
thread_local OomInfo t_oom = {"", 0, 0, false};
thread_local int64_t t_last_peak = 0, t_last_allocs = 0;

}  // namespace

hipError_t dmalloc(void **p, size_t bytes, const char *what) {
    *p = nullptr;
    const int64_t b = (int64_t)bytes;
    Budget &bu = t_budget;
    if (bu.active) {
        const bool over_call = bu.used + b > bu.call_limit;
        const bool over_plan = bu.plan_base + bu.used + b > bu.plan_limit;
        if (over_call || over_plan) {
            t_oom = {what, b, over_call ? bu.call_limit : bu.plan_limit, true};
            return hipErrorOutOfMemory;
        }
    }
    const hipError_t e = hipMalloc(p, bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        *p = nullptr;
        t_oom = {what, b, 0, false};
        return e;
    }
    {
        std::lock_guard<std::mutex> lk(g_mu);
        g_sizes[*p] = b;
        g_in_use += b;
    }
    if (bu.active) {
        bu.used += b;
        bu.allocs += 1;
        if (bu.used > bu.peak) bu.peak = bu.used;
    }
    return hipSuccess;
}

void dfree(void *p) {
    if (!p) return;
    int64_t b = 0;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        auto it = g_sizes.find(p);
        if (it != g_sizes.end()) {
            b = it->second;
            g_in_use -= b;
            g_sizes.erase(it);
        }
    }
    (void)hipFree(p);
    if (t_budget.active) t_budget.used -= b;
}

int64_t dbytes(const void *p) {
    if (!p) return 0;
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_sizes.find(const_cast<void *>(p));
    return it == g_sizes.end() ? 0 : it->second;
}

int64_t dbytes_in_use() {
    std::lock_guard<std::mutex> lk(g_mu);
    return g_in_use;
}

void set_thread_limit(int64_t bytes) { t_limit = bytes > 0 ? bytes : 0; }
int64_t thread_limit() { return t_limit; }

CallScope::CallScope(int64_t plan_base, int64_t plan_limit) : outer_(!t_budget.active) {
    if (!outer_) return;
    Budget &bu = t_budget;
    bu.active = true;
    bu.used = bu.peak = bu.allocs = 0;
    bu.call_limit = t_limit > 0 ? t_limit : INT64_MAX;
    bu.plan_base = plan_base;
    bu.plan_limit = plan_limit > 0 ? plan_limit : INT64_MAX;
}

CallScope::~CallScope() {
    if (!outer_) return;
    t_last_peak = t_budget.peak;
    t_last_allocs = t_budget.allocs;
    t_budget = Budget();
}

BudgetPause::BudgetPause() : was_active_(t_budget.active) { t_budget.active = false; }
BudgetPause::~BudgetPause() { t_budget.active = was_active_; }

OomInfo last_oom() { return t_oom; }
int64_t last_call_peak() { return t_last_peak; }
int64_t last_call_allocs() { return t_last_allocs; }

}  // namespace gspmm
