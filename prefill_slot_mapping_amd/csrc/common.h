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

// Host check of a slot array: each slot negative (skipped) or in [0, num_slots), and no
// non-negative slot twice. PKV_OK, or PKV_ERR_INVALID with a message prefixed by `what`.
int32_t check_slots(const int32_t* slots, int32_t n, int64_t num_slots, const char* what);

}  // namespace pkv
