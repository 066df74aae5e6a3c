// Thread-local error message of the gdnrt C ABI.
#include <stdarg.h>
#include <stdio.h>

#include "../../include/gdnrt.h"

namespace gdnrt {

static thread_local char g_msg[512] = "";

int set_error(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return status;
}

int clear_error() {
  g_msg[0] = '\0';
  return GDNRT_OK;
}

}  // namespace gdnrt

extern "C" const char* gdnrt_last_error(void) { return gdnrt::g_msg; }
