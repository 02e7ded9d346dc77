// Host side of the batch-invariant RMSNorm: argument checks, then one launch.
// As for the GEMM, every check runs before any HIP call and a failure
// launches nothing (Detent, §5).

#include <hip/hip_runtime.h>

#include <cmath>
#include <string>

#include "../../include/bi_norm.h"
#include "bigemm_internal.h"
#include "norm_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

extern "C" {

bi_status_t bi_rmsnorm(const void* x, const void* gain, int T, int H, float eps, void* y, void* stream)
{
    using bigemm::api_fail;
    if (T < 0 || H < 8 || H > 65536 || H % 8 != 0)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "need T >= 0 and 8 <= H <= 65536, H a multiple of 8");
    if ((long long)T * H >= (1LL << 31))
        return api_fail(BI_ERR_INVALID_ARGUMENT, "T*H must be below 2^31");
    if (!std::isfinite(eps) || eps < 0.f)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
    if (T == 0)
        return BI_OK;
    if (!x || !gain || !y)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "a pointer is NULL");
    if (!aligned16(x) || !aligned16(gain) || !aligned16(y))
        return api_fail(BI_ERR_MISALIGNED, "x, gain and y must be 16-byte aligned");
    const char* xb = static_cast<const char*>(x);
    const char* yb = static_cast<const char*>(y);
    const size_t bytes = (size_t)T * H * 2;
    if (xb < yb + bytes && yb < xb + bytes)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "y must not overlap x");
    int dev, cus;
    bi_status_t st = bigemm::api_device(&dev, &cus);
    if (st != BI_OK)
        return st;
    const hipError_t e = binorm::launch_rmsnorm(x, gain, T, H, eps, y, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return api_fail(BI_ERR_HIP, (std::string("kernel launch: ") + hipGetErrorString(e)).c_str());
    return BI_OK;
}

}  // extern "C"
