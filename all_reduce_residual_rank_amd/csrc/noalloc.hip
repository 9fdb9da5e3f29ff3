// noalloc.hip -- arrms_fused_noalloc (include/arrms.h): arrms_fused for callers
// that cannot allocate device memory. The two-stage path's staging lives in a
// fixed region of device memory that belongs to this library's code object
// (one copy per GPU, held until the process ends), so no call ever allocates.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "arrms.h"
#include "launch.hpp"

namespace {

// The fixed staging region. In host code this name is only a stand-in for the
// device symbol: kernels must get the per-device address from
// hipGetSymbolAddress (scratch_ptr below), never the name itself.
static __device__ __align__(256) unsigned char scratch[ARRMS_NOALLOC_SCRATCH_BYTES];

using arrms::kMaxDevices;
std::mutex g_mu;
void *g_scratch_ptr[kMaxDevices];

// Device address of the current device's copy of `scratch`, looked up once per
// device (with that device current) and kept. ARRMS_OK or ARRMS_ERR_HIP.
int scratch_ptr(void **p)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return ARRMS_ERR_HIP;
    }
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch_ptr[dev]) {
        void *q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) {
            (void)hipGetLastError();
            return ARRMS_ERR_HIP;
        }
        g_scratch_ptr[dev] = q;
    }
    *p = g_scratch_ptr[dev];
    return ARRMS_OK;
}

}  // namespace

extern "C" ARRMS_API int arrms_fused_noalloc(const void *const *rank_in, int R, const void *residual,
                                             const void *weight, void *out, void *residual_out, void *fp8_out,
                                             float *fp8_scale, int M, int H, float eps, int flags,
                                             hipStream_t stream)
{
    // the argument checks first: bad arguments come back before any device call
    int rc = arrms::fused_validate(rank_in, R, residual, weight, out, residual_out, fp8_out, fp8_scale, M, H, eps,
                                   flags);
    if (rc != ARRMS_OK || M == 0)
        return rc;
    void *p = nullptr;
    rc = scratch_ptr(&p);
    if (rc != ARRMS_OK)
        return rc;
    return arrms::fused_fixed_staging(rank_in, R, residual, weight, out, residual_out, fp8_out, fp8_scale, M, H,
                                      eps, flags, p, ARRMS_NOALLOC_SCRATCH_BYTES, stream);
}
