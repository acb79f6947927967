// Host-side error reporting shared by the library's host code.
#pragma once

#include "../../include/ess.h"

namespace ess {

// Records the formatted message as the calling thread's last error (what
// ess_last_error returns) and returns s.
ess_status host_fail(ess_status s, const char* fmt, ...)
    __attribute__((format(printf, 2, 3)));

}  // namespace ess
