#include "status.hpp"

namespace {
thread_local std::string g_last_error;
}

namespace pkv {

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

void clear_error() { g_last_error.clear(); }

}  // namespace pkv

extern "C" const char* pa_status_str(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_OUT_OF_BLOCKS: return "PA_ERR_OUT_OF_BLOCKS";
    case PA_ERR_INVALID: return "PA_ERR_INVALID";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_DEVICE: return "PA_ERR_DEVICE";
    default: return "PA_ERR_UNKNOWN";
  }
}

extern "C" const char* pa_last_error(void) { return g_last_error.c_str(); }
