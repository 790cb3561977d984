// Status handling shared by the host-side translation units.
#pragma once
#include <stdarg.h>

namespace bitsmoe {
// Records a thread-local detail message for `status` and returns it.
int fail(int status, const char* fmt, ...);
}  // namespace bitsmoe
