// Error state, version and the proposal-weight table of libisg.
#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "isg_internal.h"

static thread_local char g_err[1024] = "";

isg_status isg_fail(isg_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

isg_status isg_check_launch(const char *what)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return isg_fail(ISG_E_HIP, "%s: %s", what, hipGetErrorString(e));
    return ISG_OK;
}

extern "C" const char *isg_last_error(void) { return g_err; }

extern "C" int isg_version(void) { return 4; }

// Importance weights live on a grid of ratio 2^(-1/256): entry k is 2^31 scaled
// down by k grid steps, rounded to the nearest integer.
extern "C" void isg_proposal_table(uint32_t out[256])
{
    for (int k = 0; k < 256; ++k)
        out[k] = (uint32_t)std::nearbyint(std::ldexp(std::exp2(-k / 256.0), 31));
}
