// Shared declarations of the library's translation units (not part of the ABI).
#pragma once

#include <stdint.h>

#include "../../include/tree_attn.h"

namespace treeattn {

// Record a thread-local message for tree_last_error() and return `s`.
tree_status fail(tree_status s, const char* fmt, ...);
void clear_error();

}  // namespace treeattn
