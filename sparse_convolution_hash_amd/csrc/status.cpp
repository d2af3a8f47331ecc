// Thread-local error string and version of libspc.
#include <stdarg.h>
#include <stdio.h>

#include "common.h"

namespace spc {

namespace {
thread_local char g_err[512] = "";
}

spc_status fail(spc_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

void clear_error() { g_err[0] = '\0'; }

}  // namespace spc

extern "C" const char* spc_last_error(void) { return spc::g_err; }

extern "C" const char* spc_version(void) { return "libspc 0.1 gfx950"; }
