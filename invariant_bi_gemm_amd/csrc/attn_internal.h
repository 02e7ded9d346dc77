// Internal declarations of the decode-attention kernels shared by their host
// API and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace biattn {

constexpr int kHeadDim = 128;

// Split partials: o [B][Hq][splits][D] and (m, l) [B][Hq][splits][2], fp32;
// plan [max_batch + 2]: each sequence's first work item, the number of
// items, and the work queue's counter.
struct Workspace {
    float* o;
    float* ml;
    int* plan;
    int splits;  // ceil(max_seq_len / S)
    int num_cus;
};

hipError_t launch_decode(const void* q, const void* k, const void* v, const int32_t* seq_start, int B,
                         int Hq, int Hkv, int S, int max_len, int Ntok, float scale, const Workspace& ws,
                         float* out, hipStream_t stream);

}  // namespace biattn
