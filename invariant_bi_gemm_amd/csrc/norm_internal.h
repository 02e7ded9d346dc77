// Internal declaration of the RMSNorm launcher shared by its host API and the
// gfx950 kernel.
#pragma once

#include <hip/hip_runtime.h>

namespace binorm {

hipError_t launch_rmsnorm(const void* x, const void* g, int T, int H, float eps, void* y,
                          hipStream_t stream);
// rstd[t] = the r of row t by the same tree, nothing else written.
hipError_t launch_rstd(const void* x, int T, int H, float eps, float* rstd, hipStream_t stream);

}  // namespace binorm
