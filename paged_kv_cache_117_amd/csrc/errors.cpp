// Thread-local error message behind pa_last_error(), and the pending
// request of pa_time_next_main_kernel.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "pa_internal.h"

namespace {
thread_local char g_msg[512] = "";
std::mutex g_ev_mu;
void* g_ev_start = nullptr;
void* g_ev_stop = nullptr;
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

void take_main_kernel_events(void** start_event, void** stop_event) {
  std::lock_guard<std::mutex> lk(g_ev_mu);
  *start_event = g_ev_start;
  *stop_event = g_ev_stop;
  g_ev_start = g_ev_stop = nullptr;
}

}  // namespace pa

extern "C" const char* pa_last_error(void) { return g_msg; }

extern "C" int pa_abi_version(void) { return 1; }

extern "C" pa_status_t pa_time_next_main_kernel(void* start_event, void* stop_event) {
  pa::clear_error();
  if ((start_event == nullptr) != (stop_event == nullptr))
    return pa::fail(PA_ERR_NULL, "pa_time_next_main_kernel: give both events or neither");
  std::lock_guard<std::mutex> lk(g_ev_mu);
  g_ev_start = start_event;
  g_ev_stop = stop_event;
  return PA_OK;
}
