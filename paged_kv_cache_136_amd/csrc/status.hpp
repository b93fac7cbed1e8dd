// Status codes and per-thread error detail shared by every C entry point.
#pragma once

#include <string>

#include "pagedkv.h"

namespace pkv {

// Records `msg` as the calling thread's last error and returns `status`.
int fail(int status, const std::string& msg);
// Clears the calling thread's last error (start of each successful call).
void clear_error();

}  // namespace pkv
