// Device memory of the library: every buffer, whether a plan keeps it or a
// call frees it before returning, is allocated here, so that a byte budget can
// be enforced and the library's holdings counted.
//
// Budget: while a call scope is open on a thread (CallScope), an allocation
// fails with hipErrorOutOfMemory, without touching the device, when it would
// take the bytes the call holds above the thread's per-call limit, or the
// bytes the call's plan holds above the plan's limit.  The name of the buffer
// that did not fit is kept for the error message.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace gspmm {

hipError_t dmalloc(void **p, size_t bytes, const char *what);
void dfree(void *p);
template <typename T>
hipError_t dmalloc(T **p, size_t bytes, const char *what) {
    return dmalloc(reinterpret_cast<void **>(p), bytes, what);
}
template <typename T>
hipError_t dmalloc_n(T **p, int64_t count, const char *what) {
    return dmalloc(reinterpret_cast<void **>(p), sizeof(T) * (size_t)(count > 0 ? count : 1), what);
}

// Bytes of one live allocation (0 for nullptr or a pointer not from dmalloc).
int64_t dbytes(const void *p);

// Process-wide bytes currently held by the library's allocations.
int64_t dbytes_in_use();

// Limit of the calling thread (<= 0: none) on the bytes one call may hold.
void set_thread_limit(int64_t bytes);
int64_t thread_limit();

// Opens the budget of one library call; nested scopes leave the outer one in
// force.  plan_base and plan_limit describe the plan the call works on (its
// current holdings and its limit, <= 0 meaning none).
class CallScope {
public:
    CallScope(int64_t plan_base, int64_t plan_limit);
    ~CallScope();
    CallScope(const CallScope &) = delete;
    CallScope &operator=(const CallScope &) = delete;

private:
    bool outer_;
};

// Suspends the calling thread's budget (used to put back buffers a plan
// held before a failed call, whose temporaries may briefly pass the limit).
class BudgetPause {
public:
    BudgetPause();
    ~BudgetPause();
    BudgetPause(const BudgetPause &) = delete;
    BudgetPause &operator=(const BudgetPause &) = delete;

private:
    bool was_active_;
};

// The failed allocation of the calling thread's last OOM: name, size, and
// whether the budget (rather than the device) refused it.
struct OomInfo {
    const char *what;
    int64_t bytes;
    int64_t limit;       // the limit that refused it (0 when the device did)
    bool simulated;
};
OomInfo last_oom();

// Peak bytes held and number of allocations of the calling thread's last
// completed call scope.
int64_t last_call_peak();
int64_t last_call_allocs();

}  // namespace gspmm
