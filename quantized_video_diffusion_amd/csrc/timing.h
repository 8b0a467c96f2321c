// Per-kernel event timing hooks (see timing.hip).
#pragma once

#include <string>

#include <hip/hip_runtime.h>

namespace qvd {

bool timing_enabled();

// While one of these lives on a thread, that thread's launches record no events (the timer creates
// events on demand, which an allocation-free entry point must not do).
class TimingOff {
public:
    TimingOff();
    ~TimingOff();
    TimingOff(const TimingOff&) = delete;
    TimingOff& operator=(const TimingOff&) = delete;
};

// Records an event pair around the launches made during its lifetime, when timing is enabled.
class TimingScope {
public:
    TimingScope(const char* key, hipStream_t st);
    ~TimingScope();
    TimingScope(const TimingScope&) = delete;
    TimingScope& operator=(const TimingScope&) = delete;

private:
    hipStream_t st_;
    hipEvent_t start_ = nullptr, stop_ = nullptr;
    std::string key_;
};

}  // namespace qvd
