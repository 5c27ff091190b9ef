// Shared host-side helpers: thread-local error detail for pa_last_error().
#pragma once

#include <string>

#include "pa.h"

namespace pa {

// Records `detail` as the calling thread's last error and returns `s`.
pa_status fail(pa_status s, const std::string& detail);

}  // namespace pa
