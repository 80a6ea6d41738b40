// Status reporting shared by the ABI entry points: a failing call records a
// message in a thread-local buffer and returns its status code.
#pragma once

#include <cstdint>

namespace pa {

// Record `msg` as the calling thread's last error and return `status`.
int32_t fail(int32_t status, const char* msg);

}  // namespace pa
