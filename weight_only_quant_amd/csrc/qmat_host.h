// Host-side helpers shared by the library's C ABI sources (qmat_api.cpp, qmat_encode.cpp).
#pragma once

#include <stdint.h>

namespace qmath {

// Record a message for qmat_last_error() (thread-local) and return status.
int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the calling thread's message and return QMAT_OK.
int ok();
// Worker threads for host loops over n independent items (1..16).
unsigned host_threads(int64_t n);

}  // namespace qmath
