// dn_profile.cpp -- optional per-kernel timing with HIP events.
//
// When enabled (dn_profile_enable(1)) every kernel launch of the library is
// bracketed by two hipEvents recorded on the launch stream.  dn_profile_collect
// waits for those events, sums the elapsed time per kernel name and releases
// the events.  Disabled (the default) it costs one relaxed atomic load per launch.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "dn.h"
#include "dn_internal.h"

namespace dn {

namespace {

struct Mark {
    std::string name;
    hipEvent_t start, stop;
};

std::atomic<int> g_on{0};
std::mutex g_mu;
std::vector<Mark> g_marks;
thread_local int g_open = -1;  // index of the mark opened by prof_begin on this thread

}  // namespace

void prof_begin(hipStream_t stream, const char* name) {
    g_open = -1;
    if (!g_on.load(std::memory_order_relaxed)) return;
    Mark m{name, nullptr, nullptr};
    if (hipEventCreate(&m.start) != hipSuccess) return;
    if (hipEventCreate(&m.stop) != hipSuccess) {
        (void)hipEventDestroy(m.start);
        return;
    }
    (void)hipEventRecord(m.start, stream);
    std::lock_guard<std::mutex> lk(g_mu);
    g_marks.push_back(m);
    g_open = (int)g_marks.size() - 1;
}

void prof_end(hipStream_t stream) {
    if (g_open < 0) return;
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_open < (int)g_marks.size()) (void)hipEventRecord(g_marks[g_open].stop, stream);
    g_open = -1;
}

}  // namespace dn

extern "C" {

dn_status dn_profile_enable(int on) {
    dn::g_on.store(on ? 1 : 0);
    return DN_OK;
}

int dn_profile_collect(char* names, double* total_ms, int* launches, int max_kernels) {
    std::lock_guard<std::mutex> lk(dn::g_mu);
    std::vector<std::string> keys;
    std::vector<double> ms;
    std::vector<int> cnt;
    for (auto& m : dn::g_marks) {
        float t = 0.f;
        if (hipEventSynchronize(m.stop) == hipSuccess && hipEventElapsedTime(&t, m.start, m.stop) == hipSuccess) {
            size_t i = 0;
            while (i < keys.size() && keys[i] != m.name) ++i;
            if (i == keys.size()) {
                keys.push_back(m.name);
                ms.push_back(0.0);
                cnt.push_back(0);
            }
            ms[i] += t;
            cnt[i] += 1;
        }
        (void)hipEventDestroy(m.start);
        (void)hipEventDestroy(m.stop);
    }
    dn::g_marks.clear();
    const int n = (int)keys.size() < max_kernels ? (int)keys.size() : max_kernels;
    for (int i = 0; i < n; ++i) {
        if (names) {
            std::strncpy(names + 32 * i, keys[i].c_str(), 31);
            names[32 * i + 31] = '\0';
        }
        if (total_ms) total_ms[i] = ms[i];
        if (launches) launches[i] = cnt[i];
    }
    return n;
}

}  // extern "C"
