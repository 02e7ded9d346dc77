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

// The row's 1 / sqrt(mean(x^2) + eps) by the fixed tree: this thread's
// chunks in ascending order, each chunk's values in order (a missing chunk
// adds +0 squares, which leaves the sum unchanged); a butterfly inside each
// wave (every lane ends with the wave's total); the four wave totals in
// order.  Every thread of the block returns it.
template <int CPT>
__device__ __forceinline__ float row_rstd(const uint4 (&v)[CPT], int H, float eps, float* s_wave)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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
    return __fdiv_rn(1.0f, __fsqrt_rn(__fdiv_rn(total, (float)H) + eps));
}

// One row per block.  CPT: chunks of 8 values per thread, enough for the row
// (held in registers between the two passes, so x is read once).
template <int CPT>
__device__ __forceinline__ void load_row(const uint4* __restrict__ xr, int h8, uint4 (&v)[CPT])
{
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
        const int c = threadIdx.x + kThreads * q;
        v[q] = c < h8 ? xr[c] : uint4{0u, 0u, 0u, 0u};
    }
}

template <int CPT>
__global__ void __launch_bounds__(kThreads)
    rmsnorm_rows(const uint4* __restrict__ x, const uint4* __restrict__ g, int H, float eps,
                 uint4* __restrict__ y)
{
    __shared__ float s_wave[kWaves];
    const int h8 = H / 8;
    uint4 v[CPT], gv[CPT];
    load_row<CPT>(x + (size_t)blockIdx.x * h8, h8, v);
    load_row<CPT>(g, h8, gv);  // issued with the row, so the reduction hides its latency
    const float r = row_rstd<CPT>(v, H, eps, s_wave);
    uint4* yr = y + (size_t)blockIdx.x * h8;
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
        const int c = threadIdx.x + kThreads * q;
        if (c >= h8)
            break;
        yr[c] = bi::rms_scale_chunk(v[q], r, gv[q]);
    }
}

// The same r per row, stored instead of applied: the prologue of a
// projection that normalises its x tiles itself.
template <int CPT>
__global__ void __launch_bounds__(kThreads)
    rms_rstd_rows(const uint4* __restrict__ x, int H, float eps, float* __restrict__ rstd)
{
    __shared__ float s_wave[kWaves];
    const int h8 = H / 8;
    uint4 v[CPT];
    load_row<CPT>(x + (size_t)blockIdx.x * h8, h8, v);
    const float r = row_rstd<CPT>(v, H, eps, s_wave);
    if (threadIdx.x == 0)
        rstd[blockIdx.x] = r;
}

// g == nullptr: the rstd pass into rstd; else the full norm into y.
template <int CPT>
void launch_cpt(const void* x, const void* g, int T, int H, float eps, void* y, float* rstd, hipStream_t stream)
{
    if (g)
        hipLaunchKernelGGL(rmsnorm_rows<CPT>, dim3(T), dim3(kThreads), 0, stream, static_cast<const uint4*>(x),
                           static_cast<const uint4*>(g), H, eps, static_cast<uint4*>(y));
    else
        hipLaunchKernelGGL(rms_rstd_rows<CPT>, dim3(T), dim3(kThreads), 0, stream, static_cast<const uint4*>(x), H,
                           eps, rstd);
}

hipError_t launch_rows(const void* x, const void* g, int T, int H, float eps, void* y, float* rstd,
                       hipStream_t stream)
{
    const int cpt = (H / 8 + kThreads - 1) / kThreads;  // H <= 65536: at most 32
    if (cpt <= 1)
        launch_cpt<1>(x, g, T, H, eps, y, rstd, stream);
    else if (cpt <= 2)
        launch_cpt<2>(x, g, T, H, eps, y, rstd, stream);
    else if (cpt <= 4)
        launch_cpt<4>(x, g, T, H, eps, y, rstd, stream);
    else if (cpt <= 8)
        launch_cpt<8>(x, g, T, H, eps, y, rstd, stream);
    else if (cpt <= 16)
        launch_cpt<16>(x, g, T, H, eps, y, rstd, stream);
    else
        launch_cpt<32>(x, g, T, H, eps, y, rstd, stream);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm(const void* x, const void* g, int T, int H, float eps, void* y,
                          hipStream_t stream)
{
    return launch_rows(x, g, T, H, eps, y, nullptr, stream);
}

hipError_t launch_rstd(const void* x, int T, int H, float eps, float* rstd, hipStream_t stream)
{
    return launch_rows(x, nullptr, T, H, eps, nullptr, rstd, stream);
}

}  // namespace binorm
