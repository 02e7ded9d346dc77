// Internal declarations of the MoE layer's kernels (routing, grouping, row
// gather, SwiGLU, combine) shared by their host API and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bimoe {

// Most experts (the grouping kernel counts them in LDS) and most experts a
// token may use (the routing kernel keeps one per lane of a wave).
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 64;

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                       hipStream_t stream);
// Both of the above in one launch, for 1 <= T <= kRouteMaxTokens: the same
// ids, weights, offsets, rows and row_of.
constexpr int kRouteMaxTokens = 8;
hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, int32_t* offsets,
                        int32_t* tok, int32_t* row_of, hipStream_t stream);
hipError_t launch_permute(const int32_t* ids, int T, int E, int k, int32_t* offsets, int32_t* tok,
                          int32_t* row_of, hipStream_t stream);
hipError_t launch_gather(const void* src, int nsrc, const int32_t* idx, int R, int K, void* dst,
                         hipStream_t stream);
// interleaved: h's columns as the layer's gated up projection leaves them
// (16 gate columns, then their 16 up columns, and so on)
hipError_t launch_swiglu(const float* h, int R, int I, void* a, hipStream_t stream, bool interleaved = false);
hipError_t launch_combine(const float* o, int R, const int32_t* ids, const float* w,
                          const int32_t* row_of, int T, int k, int H, float* y, hipStream_t stream);

}  // namespace bimoe
