// Status strings and the thread-local error detail of the C ABI.
#include <stdio.h>

#include "bitsmoe.h"
#include "common.h"

namespace bitsmoe {
namespace {
thread_local char g_detail[512] = "";
}

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
  va_end(ap);
  return status;
}
}  // namespace bitsmoe

extern "C" {

int bitsmoe_version(void) { return 10000; }

const char* bitsmoe_strerror(int status) {
  switch (status) {
    case BITSMOE_OK: return "ok";
    case BITSMOE_EINVAL: return "invalid argument (null or misaligned pointer, bad count)";
    case BITSMOE_ESHAPE: return "invalid or inconsistent shape";
    case BITSMOE_EBITS: return "invalid width or non-finite input";
    case BITSMOE_ENOSPC: return "buffer too small";
    case BITSMOE_EFORMAT: return "invalid packed blob";
    case BITSMOE_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* bitsmoe_last_error_detail(void) { return bitsmoe::g_detail; }

}  // extern "C"
