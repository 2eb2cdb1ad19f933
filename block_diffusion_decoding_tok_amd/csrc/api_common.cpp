// C ABI: version and error reporting.
#include "common.h"

namespace dg {
static thread_local std::string g_last_error;
void set_error(const std::string& msg) { g_last_error = msg; }
dg_status fail(dg_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}
}  // namespace dg

extern "C" {
int dg_version(void) { return 100; }
const char* dg_last_error(void) { return dg::g_last_error.c_str(); }
}
