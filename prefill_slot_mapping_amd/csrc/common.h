// Internal helpers shared by the host-side translation units of the library.
#pragma once

#include <cstdint>
#include <string>

#include "../../include/pkv.h"

namespace pkv {

// Records msg as the calling thread's last error and returns status.
int32_t fail(int32_t status, const std::string& msg);

// Clears the calling thread's last error and returns PKV_OK.
int32_t ok();

}  // namespace pkv
