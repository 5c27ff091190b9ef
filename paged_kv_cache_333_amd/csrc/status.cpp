// Status strings, per-thread error detail and the ABI version.
#include "status.hpp"

namespace {
thread_local std::string g_last_error;
}

namespace pa {
pa_status fail(pa_status s, const std::string& detail) {
  g_last_error = detail;
  return s;
}
}  // namespace pa

extern "C" {

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_NO_FREE_BLOCKS: return "no free blocks";
    case PA_ERR_UNKNOWN_SEQ: return "unknown sequence";
    case PA_ERR_SEQ_EXISTS: return "sequence exists";
    case PA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case PA_ERR_BAD_TABLE: return "index outside its range";
    case PA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case PA_ERR_HIP: return "HIP error";
    case PA_ERR_UNKNOWN_PREFIX: return "unknown prefix";
  }
  return "unknown status";
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

}  // extern "C"
