// Thread-local error message behind pa_last_error().
#include <cstdarg>
#include <cstdio>

#include "pa_internal.h"

namespace {
thread_local char g_msg[512] = "";
}

namespace pa {

pa_status_t fail(pa_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() { g_msg[0] = '\0'; }

}  // namespace pa

extern "C" const char* pa_last_error(void) { return g_msg; }

extern "C" int pa_abi_version(void) { return 1; }
