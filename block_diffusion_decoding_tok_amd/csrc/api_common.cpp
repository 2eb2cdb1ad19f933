// C ABI: version and error reporting; per-device kernel attributes.
#include <mutex>
#include <set>
#include <tuple>

#include "common.h"

namespace dg {
static thread_local std::string g_last_error;
void set_error(const std::string& msg) { g_last_error = msg; }
dg_status fail(dg_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

dg_status ensure_lds_limit(const void* kernel, int bytes) {
  static std::mutex mu;
  static std::set<std::tuple<const void*, int, int>> done;   // (kernel, device, bytes)
  int dev = 0;
  DG_HIP(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({kernel, dev, bytes})) return DG_OK;
  DG_HIP(hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes));
  done.insert({kernel, dev, bytes});
  return DG_OK;
}
}  // namespace dg

extern "C" {
int dg_version(void) { return 100; }
const char* dg_last_error(void) { return dg::g_last_error.c_str(); }
}
