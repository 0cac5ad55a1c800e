// errors.cpp -- per-thread message of the latest failed call.
#include <stdarg.h>
#include <stdio.h>

#include "skv_host.h"

namespace {
thread_local char g_msg[512] = "";
}

namespace skv {

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof g_msg, fmt, ap);
  va_end(ap);
}

void clear_error() { g_msg[0] = '\0'; }

}  // namespace skv

extern "C" const char* sparsekv_last_error(void) { return g_msg; }
