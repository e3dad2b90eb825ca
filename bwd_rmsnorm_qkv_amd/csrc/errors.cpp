// Thread-local error message behind qblk_last_error().
#include <stdarg.h>
#include <stdio.h>

#include "common.h"
#include "../../include/qblk.h"

namespace qblk {

static thread_local char g_msg[1024] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return code;
}

int check_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return QBLK_OK;
  return fail(QBLK_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int check_launch(const char* what) { return check_hip(hipGetLastError(), what); }

}  // namespace qblk

extern "C" const char* qblk_last_error(void) { return qblk::g_msg; }

extern "C" void qblk_clear_error(void) { qblk::g_msg[0] = 0; }
