// Host-side plumbing of the C ABI: thread-local error text, per-device
// compute-unit count, row capacity.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "common.hpp"

namespace moe {

static thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_err[0] = 0; }

int num_cus() {
    constexpr int MAXDEV = 64;
    static int cache[MAXDEV] = {0};
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAXDEV) return 256;
    std::lock_guard<std::mutex> lk(mu);
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

}  // namespace moe

extern "C" const char* moe_last_error(void) { return moe::g_err; }

extern "C" int64_t moe_row_cap(int64_t T, int32_t k, int32_t L) {
    if (T < 0 || k < 0 || L < 0) return -1;
    int64_t per_tok = k < L ? k : L;
    int64_t rows = T * per_tok + (int64_t)L * (MOE_ROW_ALIGN - 1);
    return (rows + MOE_ROW_ALIGN - 1) / MOE_ROW_ALIGN * MOE_ROW_ALIGN;
}
