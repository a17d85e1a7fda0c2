// Error reporting and version of the C ABI (declared in exactverify.h).
#include <stdarg.h>
#include <stdio.h>

#include "ev_internal.h"

namespace {
thread_local char g_err[512] = "";
}

namespace ev {

int32_t fail(int32_t code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_err[0] = '\0'; }

int32_t check_hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return EV_OK;
    return fail(EV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace ev

extern "C" const char* ev_last_error(void) { return g_err; }
extern "C" int32_t ev_version(void) { return 100; }  // 0.1.0
