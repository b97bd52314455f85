// Internal helpers shared by the translation units of libpagedkv.
#pragma once

#include "pagedkv.h"

namespace pagedkv {

// Record a printf-style message for pa_last_error() and return `st`.
pa_status fail(pa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace pagedkv
