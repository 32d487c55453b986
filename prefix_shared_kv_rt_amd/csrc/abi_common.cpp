// Error reporting and version query of the C ABI.
#include <string>

#include "radixrt.h"
#include "rt_internal.h"

namespace {
thread_local std::string g_last_error;
}

namespace rt {
int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}
}  // namespace rt

extern "C" {
const char* rt_last_error(void) { return g_last_error.c_str(); }
int rt_abi_version(void) { return 1; }
}
