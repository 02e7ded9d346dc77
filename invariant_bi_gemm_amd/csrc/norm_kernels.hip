// gfx950 kernel of the batch-invariant RMSNorm (include/bi_norm.h).
//
// A stock RMSNorm splits a row's reduction over blocks when the batch is
// small, which makes a token's bits follow the batch (CoRun, §III-A Fig. 3).
// Here one block owns a row and reduces it with a tree fixed by H alone (see
// the header), whatever T is and wherever the row sits.  HBM-bound: a row is
// read once into registers and written once, in 16-byte chunks; no MFMA
// (this is not a contraction).

#include <math.h>

#include "bf16_round.h"
#include "norm_internal.h"

namespace binorm {
namespace {

constexpr int kThreads = 256;  // one block per row: four waves
constexpr int kWaves = kThreads / 64;

// CPT: chunks of 8 values per thread, enough for the row (held in registers
// between the two passes, so x is read once).
template <int CPT>
__global__ void __launch_bounds__(kThreads)
    rmsnorm_rows(const uint4* __restrict__ x, const uint4* __restrict__ g, int H, float eps,
                 uint4* __restrict__ y)
{
    __shared__ float s_wave[kWaves];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int h8 = H / 8;
    const uint4* xr = x + (size_t)blockIdx.x * h8;
    uint4* yr = y + (size_t)blockIdx.x * h8;

    uint4 v[CPT];
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
        const int c = tid + kThreads * q;
        v[q] = c < h8 ? xr[c] : uint4{0u, 0u, 0u, 0u};
    }
    // this thread's chunks in ascending order, each chunk's values in order
    // (a missing chunk adds +0 squares, which leaves the sum unchanged)
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
        const uint32_t w[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a = bi::from_bf16(w[e] & 0xffffu);
            const float b = bi::from_bf16(w[e] >> 16);
            ss = ss + a * a;
            ss = ss + b * b;
        }
    }
    // butterfly inside each wave (every lane ends with the wave's total),
    // then the four wave totals in order
#pragma unroll
    for (int d = 32; d > 0; d >>= 1)
        ss = ss + __shfl_xor(ss, d, 64);
    if (lane == 0)
        s_wave[wave] = ss;
    __syncthreads();
    float total = s_wave[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w)
        total = total + s_wave[w];
    const float r = __fdiv_rn(1.0f, __fsqrt_rn(__fdiv_rn(total, (float)H) + eps));

#pragma unroll
    for (int q = 0; q < CPT; ++q) {
        const int c = tid + kThreads * q;
        if (c >= h8)
            break;
        const uint4 gv = g[c];
        const uint32_t w[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
        const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a = (bi::from_bf16(w[e] & 0xffffu) * r) * bi::from_bf16(gw[e] & 0xffffu);
            const float b = (bi::from_bf16(w[e] >> 16) * r) * bi::from_bf16(gw[e] >> 16);
            o[e] = (uint32_t)bi::to_bf16(a) | ((uint32_t)bi::to_bf16(b) << 16);
        }
        yr[c] = uint4{o[0], o[1], o[2], o[3]};
    }
}

template <int CPT>
void launch_cpt(const void* x, const void* g, int T, int H, float eps, void* y, hipStream_t stream)
{
    hipLaunchKernelGGL(rmsnorm_rows<CPT>, dim3(T), dim3(kThreads), 0, stream, static_cast<const uint4*>(x),
                       static_cast<const uint4*>(g), H, eps, static_cast<uint4*>(y));
}

}  // namespace

hipError_t launch_rmsnorm(const void* x, const void* g, int T, int H, float eps, void* y,
                          hipStream_t stream)
{
    const int cpt = (H / 8 + kThreads - 1) / kThreads;  // H <= 65536: at most 32
    if (cpt <= 1)
        launch_cpt<1>(x, g, T, H, eps, y, stream);
    else if (cpt <= 2)
        launch_cpt<2>(x, g, T, H, eps, y, stream);
    else if (cpt <= 4)
        launch_cpt<4>(x, g, T, H, eps, y, stream);
    else if (cpt <= 8)
        launch_cpt<8>(x, g, T, H, eps, y, stream);
    else if (cpt <= 16)
        launch_cpt<16>(x, g, T, H, eps, y, stream);
    else
        launch_cpt<32>(x, g, T, H, eps, y, stream);
    return hipGetLastError();
}

}  // namespace binorm
