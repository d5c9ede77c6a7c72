// Internal declarations shared by the host translation units of libpagedattn.
#pragma once
#include <cstdarg>
#include <cstdint>

#include "pa.h"

namespace pa {

// Record a detail message for pa_last_error() and return the status.
pa_status fail(pa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the detail message and return PA_OK.
pa_status ok();

}  // namespace pa
