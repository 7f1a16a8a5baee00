// Host helpers of the qmat C ABI shared by its sources: the thread-local error message behind
// qmat_last_error(), the worker-thread count of host loops and the shape rule.  No HIP here.
#include <cstdarg>
#include <cstdio>
#include <thread>

#include "../../include/qmat.h"
#include "qmat_host.h"
#include "qmat_layout.h"

namespace qmath {

namespace {
thread_local char g_err[512] = "";
}

int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

int ok()
{
    g_err[0] = '\0';
    return QMAT_OK;
}

const char *last_error() { return g_err; }

// M and K limits keep every kernel index inside 32-bit tile/unit counts and 64-bit offsets.
bool shape_ok(int64_t M, int64_t K)
{
    return M >= 1 && K >= 64 && K % qmatk::kGroup == 0 && M <= (1LL << 30) && K <= (1LL << 20) &&
           M * K <= (1LL << 40);
}

unsigned host_threads(int64_t n)
{
    unsigned nth = std::thread::hardware_concurrency();
    if (nth == 0) nth = 1;
    if (nth > 16) nth = 16;
    if ((int64_t)nth > n) nth = n > 0 ? (unsigned)n : 1u;
    return nth;
}

}  // namespace qmath

extern "C" const char *qmat_last_error(void) { return qmath::last_error(); }
