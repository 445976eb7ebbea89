// Opt-in kernel timing: while enabled, the launchers bracket each launch of
// the selected kernels with a pair of HIP events recorded on the launch's own
// stream, so a measurement tool can read per-kernel device time of the work it
// enqueued without a profiler.  Disabled (the default), a bracket costs one
// relaxed atomic load.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "internal.h"

namespace {

constexpr int POOL = 16384;  // event pairs, created at the first enable

std::mutex mu;
std::atomic<unsigned> mask{0};
std::vector<hipEvent_t> ev;               // 2 * POOL events
int used = 0;                             // pairs handed out since the last enable
std::vector<int> pairs[SPEC_KT_COUNT];    // pair indices per kernel
int64_t dropped[SPEC_KT_COUNT];

}  // namespace

int ktimer_begin(hipStream_t stream, int id)
{
    if (!(mask.load(std::memory_order_relaxed) & (1u << id))) return -1;
    std::lock_guard<std::mutex> g(mu);
    if (used >= POOL) {
        ++dropped[id];
        return -1;
    }
    const int p = used++;
    if (hipEventRecord(ev[2 * p], stream) != hipSuccess) return -1;
    pairs[id].push_back(p);
    return p;
}

void ktimer_end(hipStream_t stream, int p)
{
    if (p >= 0) (void)hipEventRecord(ev[2 * p + 1], stream);
}

extern "C" {

int spec_timing_enable(unsigned kernels)
{
    std::lock_guard<std::mutex> g(mu);
    if (kernels != 0 && ev.empty()) {
        ev.resize(2 * POOL);
        for (auto &e : ev)
            if (hipEventCreate(&e) != hipSuccess) {
                ev.clear();
                return SPEC_EHIP;
            }
    }
    used = 0;
    for (int k = 0; k < SPEC_KT_COUNT; ++k) {
        pairs[k].clear();
        dropped[k] = 0;
    }
    mask.store(kernels & ((1u << SPEC_KT_COUNT) - 1), std::memory_order_relaxed);
    return SPEC_OK;
}

int spec_timing_read(int kernel, double *total_ms, int64_t *launches)
{
    if (kernel < 0 || kernel >= SPEC_KT_COUNT || total_ms == nullptr || launches == nullptr) return SPEC_EINVAL;
    std::lock_guard<std::mutex> g(mu);
    double sum = 0.0;
    for (int p : pairs[kernel]) {
        if (hipEventSynchronize(ev[2 * p + 1]) != hipSuccess) return SPEC_EHIP;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, ev[2 * p], ev[2 * p + 1]) != hipSuccess) return SPEC_EHIP;
        sum += ms;
    }
    *total_ms = sum;
    *launches = (int64_t)pairs[kernel].size();
    return dropped[kernel] ? SPEC_EWORKSPACE : SPEC_OK;
}

}  // extern "C"
