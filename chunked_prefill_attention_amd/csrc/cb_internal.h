// Internal declarations shared by the host files of the library.
#pragma once

#include <cstdarg>
#include <cstddef>
#include <cstdint>

#include "cb.h"

namespace cb {

// Record a thread-local error message and return `status`.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace cb

namespace cb {
// Largest number of pages any live request of the builder holds.
int32_t builder_max_pages_held(const cb_builder* b);
// Deep copy of src's state into dst (dst keeps its address).
int builder_assign(cb_builder* dst, const cb_builder* src);
}  // namespace cb
