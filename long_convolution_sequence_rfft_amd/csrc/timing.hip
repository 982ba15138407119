// timing.hip -- host side of the per-launch timing (hyena_timing_* entry
// points).  State is per host thread: the events, the labels of the recorded
// launches and, after hyena_timing_end, the per-kernel totals.
#include <algorithm>
#include <map>
#include <string>
#include <vector>

#include "plan.h"
#include "timing.h"

namespace hy {
namespace {

struct KernelTotals {
    std::string name;
    int64_t launches = 0;
    double total_ms = 0.0, min_ms = 0.0, max_ms = 0.0;
};

struct TimingState {
    bool on = false;
    int32_t cap = 0;    // launches that can be recorded
    int32_t used = 0;   // launches recorded
    int64_t dropped = 0;
    std::vector<hipEvent_t> ev;  // 2 per launch
    std::vector<std::string> label;
    std::vector<KernelTotals> totals;
    // a begin event was recorded for the launch in flight
    bool open = false;
};

thread_local TimingState g_timing;

void destroy_events(TimingState& t)
{
    for (hipEvent_t e : t.ev)
        if (e) (void)hipEventDestroy(e);
    t.ev.clear();
    t.label.clear();
    t.cap = t.used = 0;
    t.dropped = 0;
    t.open = false;
}

}  // namespace

bool timing_on() { return g_timing.on; }

void timing_mark_begin(hipStream_t s)
{
    TimingState& t = g_timing;
    t.open = false;
    if (t.used >= t.cap) {
        ++t.dropped;
        return;
    }
    if (hipEventRecord(t.ev[2 * t.used], s) == hipSuccess) t.open = true;
}

void timing_mark_end(hipStream_t s, const std::string& label)
{
    TimingState& t = g_timing;
    if (!t.open) return;
    t.open = false;
    if (hipEventRecord(t.ev[2 * t.used + 1], s) != hipSuccess) return;
    t.label[t.used] = label;
    ++t.used;
}

}  // namespace hy

using hy::fail;

extern "C" {

hyena_status hyena_timing_begin(int32_t max_launches)
{
    if (max_launches < 1 || max_launches > (1 << 20))
        return fail(HYENA_ERR_INVALID_ARGUMENT, "max_launches must be in [1, 2^20]");
    hy::TimingState& t = hy::g_timing;
    t.on = false;
    hy::destroy_events(t);
    t.totals.clear();
    t.ev.assign(2 * (size_t)max_launches, nullptr);
    for (auto& e : t.ev) {
        const hipError_t r = hipEventCreate(&e);
        if (r != hipSuccess) {
            e = nullptr;
            hy::destroy_events(t);
            return fail(HYENA_ERR_DEVICE, std::string("hipEventCreate: ") + hipGetErrorString(r));
        }
    }
    t.label.assign((size_t)max_launches, std::string());
    t.cap = max_launches;
    t.on = true;
    return HYENA_OK;
}

hyena_status hyena_timing_end(int32_t* n_kernels, int64_t* dropped)
{
    hy::TimingState& t = hy::g_timing;
    t.on = false;
    t.totals.clear();
    std::map<std::string, size_t> slot;
    for (int32_t i = 0; i < t.used; ++i) {
        hipError_t r = hipEventSynchronize(t.ev[2 * i + 1]);
        float ms = 0.0f;
        if (r == hipSuccess) r = hipEventElapsedTime(&ms, t.ev[2 * i], t.ev[2 * i + 1]);
        if (r != hipSuccess)
            return fail(HYENA_ERR_DEVICE, std::string("timing events: ") + hipGetErrorString(r));
        auto it = slot.find(t.label[i]);
        if (it == slot.end()) {
            it = slot.emplace(t.label[i], t.totals.size()).first;
            hy::KernelTotals k;
            k.name = t.label[i];
            k.min_ms = k.max_ms = ms;
            t.totals.push_back(k);
        }
        hy::KernelTotals& k = t.totals[it->second];
        ++k.launches;
        k.total_ms += ms;
        k.min_ms = std::min(k.min_ms, (double)ms);
        k.max_ms = std::max(k.max_ms, (double)ms);
    }
    if (n_kernels) *n_kernels = (int32_t)t.totals.size();
    if (dropped) *dropped = t.dropped;
    return HYENA_OK;
}

hyena_status hyena_timing_kernel(int32_t i, const char** name, int64_t* launches,
                                 double* total_ms, double* min_ms, double* max_ms)
{
    const hy::TimingState& t = hy::g_timing;
    if (i < 0 || (size_t)i >= t.totals.size())
        return fail(HYENA_ERR_INVALID_ARGUMENT, "kernel index out of range (call hyena_timing_end first)");
    const hy::KernelTotals& k = t.totals[(size_t)i];
    if (name) *name = k.name.c_str();
    if (launches) *launches = k.launches;
    if (total_ms) *total_ms = k.total_ms;
    if (min_ms) *min_ms = k.min_ms;
    if (max_ms) *max_ms = k.max_ms;
    return HYENA_OK;
}

hyena_status hyena_timing_release(void)
{
    hy::TimingState& t = hy::g_timing;
    t.on = false;
    hy::destroy_events(t);
    t.totals.clear();
    return HYENA_OK;
}

}  // extern "C"
