// Error reporting shared by the host-side translation units.
#pragma once

#include <cstdarg>
#include <cstdio>

#include "pagedkv.h"

namespace pa {

// Records a message for pa_last_error() on this thread and returns `s`.
pa_status fail(pa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

}  // namespace pa
