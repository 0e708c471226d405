// Internal declarations shared by the host and device halves of libzero_shard.
#pragma once

#include <cstdarg>
#include <cstdint>

#include "../../include/zero_shard.h"

namespace zs {

// Record a message for zero_last_error() and return `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Start a call: clear the thread's message.
void clear_error();

}  // namespace zs
