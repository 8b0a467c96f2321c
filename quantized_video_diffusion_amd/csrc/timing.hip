// Opt-in per-kernel timing with HIP events.  When enabled, every launch the library makes records an
// event pair on its own stream, keyed by the kernel's class (and the GEMM's shape); the report sums
// the elapsed times after the recorded work has finished.  Disabled, the hooks cost one branch.
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"
#include "timing.h"

namespace qvd {

namespace {

struct Rec {
    std::string key;
    hipEvent_t start, stop;
};

std::mutex g_mu;
bool g_on = false;
std::vector<hipEvent_t> g_pool;     // free events
std::vector<Rec> g_recs;            // pending records

hipEvent_t take_event() {
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

}  // namespace

bool timing_enabled() { return g_on; }

namespace {
thread_local int t_off = 0;
}

TimingOff::TimingOff() { ++t_off; }
TimingOff::~TimingOff() { --t_off; }

TimingScope::TimingScope(const char* key, hipStream_t st) : st_(st) {
    if (!g_on || t_off > 0) return;
    std::lock_guard<std::mutex> lk(g_mu);
    start_ = take_event();
    stop_ = take_event();
    if (!start_ || !stop_) return;
    key_ = key;
    (void)hipEventRecord(start_, st_);
}

TimingScope::~TimingScope() {
    if (!start_ || !stop_) return;
    (void)hipEventRecord(stop_, st_);
    std::lock_guard<std::mutex> lk(g_mu);
    g_recs.push_back(Rec{key_, start_, stop_});
}

}  // namespace qvd

using namespace qvd;

extern "C" {

int qvd_timing_enable(int on) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (on && g_pool.empty() && g_recs.empty()) {
        QVD_DEVICE_OK();
        g_pool.reserve(4096);
        for (int i = 0; i < 4096; ++i) {
            hipEvent_t e;
            if (hipEventCreate(&e) != hipSuccess) return fail(QVD_EHIP, "qvd_timing_enable: hipEventCreate");
            g_pool.push_back(e);
        }
    }
    g_on = on != 0;
    return QVD_OK;
}

int qvd_timing_report(char* buf, size_t len) {
    QVD_PTR(buf);
    QVD_REQUIRE(len >= 16, QVD_EINVAL, "qvd_timing_report: buffer too small");
    std::vector<Rec> recs;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        recs.swap(g_recs);
    }
    struct Agg {
        std::string key;
        int n;
        double ms;
    };
    std::vector<Agg> agg;
    int status = QVD_OK;
    for (auto& r : recs) {
        if (hipEventSynchronize(r.stop) != hipSuccess) status = QVD_EHIP;
        float ms = 0.0f;
        if (status == QVD_OK && hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) status = QVD_EHIP;
        bool found = false;
        for (auto& a : agg)
            if (a.key == r.key) {
                a.n += 1;
                a.ms += ms;
                found = true;
                break;
            }
        if (!found) agg.push_back(Agg{r.key, 1, (double)ms});
    }
    {
        std::lock_guard<std::mutex> lk(g_mu);
        for (auto& r : recs) {
            g_pool.push_back(r.start);
            g_pool.push_back(r.stop);
        }
    }
    std::string out = "{";
    for (size_t i = 0; i < agg.size(); ++i) {
        char tmp[256];
        snprintf(tmp, sizeof(tmp), "%s\"%s\": {\"count\": %d, \"total_ms\": %.6f}", i ? ", " : "",
                 agg[i].key.c_str(), agg[i].n, agg[i].ms);
        out += tmp;
    }
    out += "}";
    QVD_REQUIRE(out.size() + 1 <= len, QVD_EINVAL, "qvd_timing_report: needs %zu bytes", out.size() + 1);
    std::memcpy(buf, out.c_str(), out.size() + 1);
    if (status != QVD_OK) return fail(status, "qvd_timing_report: event query failed");
    return QVD_OK;
}

}  // extern "C"
