// gdr_prof.cpp -- optional per-launch HIP event timing (gdr_profile_begin/end).
//
// When enabled, the ABI layer brackets each kernel launch with an event pair
// recorded on the launch stream; gdr_profile_end() waits for the events and
// sums the elapsed times per kernel name.  Disabled, both hooks are a single
// load and branch.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/gdr.h"
#include "gdr_launch.hpp"

namespace {

constexpr size_t kMaxLaunches = 65536;

struct Rec {
    const char* name;
    hipEvent_t start, stop;
};

bool g_on = false;
std::vector<hipEvent_t> g_pool;  // reusable events, never destroyed
std::vector<Rec> g_recs;
size_t g_next = 0;  // next free pool slot
bool g_pending = false;

hipEvent_t take_event() {
    if (g_next == g_pool.size()) {
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        g_pool.push_back(e);
    }
    return g_pool[g_next++];
}

hipEvent_t g_start = nullptr;

}  // namespace

namespace gdr {

void prof_before(hipStream_t stream) {
    g_pending = false;
    if (!g_on || g_recs.size() >= kMaxLaunches) return;
    g_start = take_event();
    if (g_start && hipEventRecord(g_start, stream) == hipSuccess) g_pending = true;
}

void prof_after(const char* name, hipStream_t stream) {
    if (!g_pending) return;
    g_pending = false;
    hipEvent_t stop = take_event();
    if (!stop || hipEventRecord(stop, stream) != hipSuccess) return;
    g_recs.push_back(Rec{name, g_start, stop});
}

}  // namespace gdr

extern "C" {

int32_t gdr_profile_begin(void) {
    g_recs.clear();
    g_next = 0;
    g_on = true;
    return 0;
}

int32_t gdr_profile_end(gdr_kernel_time* out, int32_t max) {
    g_on = false;
    std::vector<gdr_kernel_time> agg;
    for (const Rec& r : g_recs) {
        if (hipEventSynchronize(r.stop) != hipSuccess) return -1;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return -1;
        size_t i = 0;
        for (; i < agg.size(); ++i)
            if (std::strncmp(agg[i].name, r.name, sizeof agg[i].name) == 0) break;
        if (i == agg.size()) {
            gdr_kernel_time t;
            std::memset(&t, 0, sizeof t);
            std::snprintf(t.name, sizeof t.name, "%s", r.name);
            agg.push_back(t);
        }
        agg[i].launches += 1;
        agg[i].total_ms += ms;
    }
    g_recs.clear();
    g_next = 0;
    int32_t n = 0;
    for (; n < int32_t(agg.size()) && n < max; ++n)
        if (out) out[n] = agg[n];
    return n;
}

}  // extern "C"
