// Status strings, last-error text and version of libll.
#include "api.h"

namespace ll {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

}  // namespace ll

extern "C" {

const char* ll_status_string(int status) {
  switch (status) {
    case LL_OK: return "LL_OK";
    case LL_ERR_INVALID_ARG: return "LL_ERR_INVALID_ARG";
    case LL_ERR_UNSUPPORTED: return "LL_ERR_UNSUPPORTED";
    case LL_ERR_WORKSPACE: return "LL_ERR_WORKSPACE";
    case LL_ERR_HIP: return "LL_ERR_HIP";
    default: return "LL_ERR_UNKNOWN";
  }
}

const char* ll_last_error(void) { return ll::g_last_error.c_str(); }

int ll_version(void) { return 100; }

}  // extern "C"
