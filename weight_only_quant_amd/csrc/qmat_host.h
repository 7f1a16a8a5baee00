// Host-side helpers shared by the library's C ABI sources (qmat_api.cpp, qmat_pack.cpp,
// qmat_encode.cpp); defined in qmat_host.cpp.
#pragma once

#include <stdint.h>

namespace qmath {

// Record a message for qmat_last_error() (thread-local) and return status.
int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the calling thread's message and return QMAT_OK.
int ok();
// Worker threads for host loops over n independent items (1..16).
unsigned host_threads(int64_t n);
// The calling thread's message (the storage behind qmat_last_error()).
const char *last_error();
// M >= 1, K a positive multiple of 64, and the size limits of include/qmat.h.
bool shape_ok(int64_t M, int64_t K);

}  // namespace qmath
