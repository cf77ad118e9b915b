// Internal helpers shared by the library's translation units (host side).
#pragma once

#include "pa.h"

namespace pa {

// Records a printf-style message for pa_last_error() and returns `st`.
pa_status_t fail(pa_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Takes (and clears) the event pair of a pending pa_time_next_main_kernel
// request; both NULL when there is none.
void take_main_kernel_events(void** start_event, void** stop_event);

}  // namespace pa
