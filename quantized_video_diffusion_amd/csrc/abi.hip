// Status reporting and device checks shared by every entry point of the C ABI.
#include <cstring>
#include <mutex>

#include "common.h"

namespace qvd {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
}

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

static std::mutex g_dev_mu;
static int g_dev_state[64];   // 0 unknown, 1 gfx950, -1 other

int check_device() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(QVD_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(QVD_EUNSUPPORTED, "device index %d out of range", dev);
    {
        std::lock_guard<std::mutex> lk(g_dev_mu);
        if (g_dev_state[dev] == 1) return QVD_OK;
        if (g_dev_state[dev] == -1)
            return fail(QVD_EUNSUPPORTED, "device %d is not gfx950", dev);
    }
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(QVD_EHIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    std::lock_guard<std::mutex> lk(g_dev_mu);
    g_dev_state[dev] = ok ? 1 : -1;
    if (!ok) return fail(QVD_EUNSUPPORTED, "device %d is %s, this library is built for gfx950", dev,
                         prop.gcnArchName);
    return QVD_OK;
}

// Launches left before an injected failure on this thread (-1: none pending).
static thread_local int64_t t_fail_after = -1;

int launch_status(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QVD_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    if (t_fail_after >= 0 && t_fail_after-- == 0)
        return fail(QVD_EHIP, "%s: launch failed: injected failure", what);
    return QVD_OK;
}

}  // namespace qvd

extern "C" {

int qvd_abi_version(void) { return QVD_ABI_VERSION; }

const char* qvd_last_error(void) { return qvd::g_err; }

int qvd_init(void) { return qvd::check_device(); }

int qvd_inject_launch_failure(int32_t after) {
    if (after < -1) return qvd::fail(QVD_EINVAL, "qvd_inject_launch_failure: after = %d (-1 or more)", after);
    qvd::t_fail_after = after;
    return QVD_OK;
}

}  // extern "C"
