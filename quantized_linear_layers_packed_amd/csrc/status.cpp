// Status codes, the thread-local error message and launch-error capture.

#include <string>

#include "common.hpp"

namespace qlin {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }
void clear_error() { g_last_error.clear(); }

qlin_status fail(qlin_status s, const std::string& msg) {
  set_error(msg);
  return s;
}

qlin_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    return fail(QLIN_EHIP, std::string(what) + ": " + hipGetErrorString(e));
  }
  return QLIN_OK;
}

}  // namespace qlin

extern "C" {

int qlin_version(void) { return 100; }

const char* qlin_status_str(int s) {
  switch (s) {
    case QLIN_OK: return "QLIN_OK";
    case QLIN_EINVAL: return "QLIN_EINVAL";
    case QLIN_EALIGN: return "QLIN_EALIGN";
    case QLIN_EUNSUPPORTED: return "QLIN_EUNSUPPORTED";
    case QLIN_EHIP: return "QLIN_EHIP";
    default: return "QLIN_UNKNOWN";
  }
}

const char* qlin_last_error(void) { return qlin::g_last_error.c_str(); }

}  // extern "C"
