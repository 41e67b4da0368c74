// Thread-local error message behind pa_last_error().
#include <stdarg.h>
#include <stdio.h>

#include "pa_internal.h"

namespace {
thread_local char g_msg[512];
}

pa_status pa_fail(pa_status code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof g_msg, fmt, ap);
  va_end(ap);
  return code;
}

void pa_clear_error() { g_msg[0] = '\0'; }

extern "C" const char *pa_last_error(void) { return g_msg; }

extern "C" int32_t pa_version(void) { return 104; }
