// Internal helpers shared by the library's translation units.
#pragma once

#include <string>

namespace rt {
// Records `msg` as the calling thread's last error and returns `code`.
int fail(int code, const std::string& msg);
}  // namespace rt
