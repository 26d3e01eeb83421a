// Library-wide plumbing: thread-local error text, HIP error mapping, ABI version.
#include <stdarg.h>
#include <stdio.h>

#include "common.h"

namespace moe {

static thread_local char g_err[512] = "";

void set_error(const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
}

void clear_error() { g_err[0] = '\0'; }

moe_status hip_check(hipError_t e, const char *what) {
    if (e == hipSuccess) return MOE_OK;
    set_error("%s: %s", what, hipGetErrorString(e));
    return MOE_ERR_HIP;
}

moe_status launch_check(const char *what) { return hip_check(hipGetLastError(), what); }

int device_cu_count() {
    constexpr int kMaxDev = 64;
    static int cache[kMaxDev] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 256;
    if (cache[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
        cache[dev] = cus;
    }
    return cache[dev];
}

}  // namespace moe

extern "C" const char *moe_last_error(void) { return moe::g_err; }
extern "C" int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }
