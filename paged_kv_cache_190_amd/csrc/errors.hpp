// Error reporting shared by the C ABI's translation units: record a message for pkv_last_error
// (per thread) and return the status code.
#pragma once

#include "../../include/pkv.h"

namespace pkv {
pkv_status fail(pkv_status status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
}  // namespace pkv
