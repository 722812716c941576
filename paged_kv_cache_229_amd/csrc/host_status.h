// Status reporting shared by the library's host sources: a failed call records its message for
// paged_kv_last_error() and returns the status; a successful one clears it.
#pragma once

#include <string>

namespace pkv {
int host_fail(int status, const std::string& msg);
int host_ok();
}  // namespace pkv
