// Error state and format checks shared by the host files of the C ABI
// (the codec in host_codec.cpp and the device entry points in moe_capi.hip).
#pragma once

#include <stdint.h>

namespace moe {

// Sets the calling thread's message (printf-style) and returns `code`.
int32_t fail(int32_t code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the calling thread's message and returns MOE_OK.
int32_t ok();
// The two container ids, 142 (PQ2_0) and 143 (PTQ1_0).
bool known_fmt(int32_t fmt);
// MOE_E_FORMAT with a message naming the id and the valid ones.
int32_t bad_fmt(int32_t fmt);

}  // namespace moe
