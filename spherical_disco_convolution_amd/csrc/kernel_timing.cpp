// Opt-in per-kernel timing: while enabled, every kernel the library launches
// is bracketed by a pair of HIP events recorded on its launch stream; a read
// drains them into per-kernel totals.  Off by default, and then a launch costs
// one relaxed atomic load.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "disco.h"
#include "disco_internal.h"

namespace disco {

namespace {

struct Pending {
    const char* name;
    hipEvent_t start, stop;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Pending> g_pending;

}  // namespace

KernelTimer::KernelTimer(const char* name, hipStream_t st) : name_(name), st_(st) {
    if (!g_on.load(std::memory_order_relaxed)) return;
    if (hipEventCreate(&start_) != hipSuccess || hipEventCreate(&stop_) != hipSuccess ||
        hipEventRecord(start_, st_) != hipSuccess) {
        (void)hipGetLastError();
        if (start_) (void)hipEventDestroy(start_);
        if (stop_) (void)hipEventDestroy(stop_);
        start_ = stop_ = nullptr;
        return;
    }
    armed_ = true;
}

KernelTimer::~KernelTimer() {
    if (!armed_) return;
    if (hipEventRecord(stop_, st_) != hipSuccess) {
        (void)hipGetLastError();
        (void)hipEventDestroy(start_);
        (void)hipEventDestroy(stop_);
        return;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    g_pending.push_back({name_, start_, stop_});
}

}  // namespace disco

extern "C" {

int disco_kernel_timing(int enable) {
    disco::g_on.store(enable != 0, std::memory_order_relaxed);
    return DISCO_OK;
}

int disco_kernel_timing_read(char* names, int32_t names_len, double* total_ms,
                             int64_t* launches, int32_t max_kernels) {
    using namespace disco;
    if (max_kernels < 0 || names_len < 0 || (max_kernels > 0 && (!total_ms || !launches)) ||
        (names_len > 0 && !names))
        return set_error(DISCO_EINVAL, "invalid output buffers for the kernel timings");
    std::vector<Pending> pend;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        pend.swap(g_pending);
    }
    std::vector<std::string> order;
    std::vector<double> tot;
    std::vector<int64_t> cnt;
    int rc = DISCO_OK;
    for (const Pending& p : pend) {
        float ms = 0.0f;
        if (rc == DISCO_OK) {
            hipError_t e = hipEventSynchronize(p.stop);
            if (e == hipSuccess) e = hipEventElapsedTime(&ms, p.start, p.stop);
            if (e != hipSuccess) {
                (void)hipGetLastError();
                rc = set_error(DISCO_EHIP, "reading a kernel timing event failed: %s",
                               hipGetErrorString(e));
            }
        }
        if (rc == DISCO_OK) {
            size_t i = 0;
            while (i < order.size() && order[i] != p.name) ++i;
            if (i == order.size()) {
                order.emplace_back(p.name);
                tot.push_back(0.0);
                cnt.push_back(0);
            }
            tot[i] += ms;
            cnt[i] += 1;
        }
        (void)hipEventDestroy(p.start);
        (void)hipEventDestroy(p.stop);
    }
    if (rc != DISCO_OK) return rc;
    if ((int64_t)order.size() > max_kernels)
        return set_error(DISCO_EINVAL, "%d kernels timed, room for %d", (int)order.size(),
                         max_kernels);
    size_t need = 0;
    for (const std::string& s : order) need += s.size() + 1;
    if (need > (size_t)names_len)
        return set_error(DISCO_EINVAL, "kernel names need %zu bytes, room for %d", need,
                         names_len);
    size_t off = 0;
    for (size_t i = 0; i < order.size(); ++i) {
        std::memcpy(names + off, order[i].c_str(), order[i].size() + 1);
        off += order[i].size() + 1;
        total_ms[i] = tot[i];
        launches[i] = cnt[i];
    }
    return (int)order.size();
}

}  // extern "C"
