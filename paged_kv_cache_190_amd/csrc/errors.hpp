// Error reporting shared by the C ABI's translation units: record a message for pkv_last_error
// (per thread) and return the status code.
#pragma once

namespace pkv {
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
}  // namespace pkv
