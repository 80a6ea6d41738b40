// Thread-local last-error storage and the meta entry points of the ABI.
#include "status.h"

#include <string>

#include "pagedkv.h"

namespace {
thread_local std::string g_last_error;
}

namespace pa {
int32_t fail(int32_t status, const char* msg) {
  g_last_error = msg ? msg : "";
  return status;
}
}  // namespace pa

extern "C" {

const char* pa_version(void) { return "0.1.0"; }

const char* pa_status_string(int32_t status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_EINVAL: return "PA_EINVAL";
    case PA_ENOMEM: return "PA_ENOMEM";
    case PA_ELAUNCH: return "PA_ELAUNCH";
    default: return "PA_UNKNOWN";
  }
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
