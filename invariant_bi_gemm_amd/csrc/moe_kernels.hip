// gfx950 kernels of the MoE layer around the grouped GEMM: routing, grouping
// of the rows by expert, row gather, SwiGLU and the weighted combine.
//
// The fused MoE is one of the kernel families whose selection reads the batch
// (Detent, §2 Obs. 1 and Fig. 3a: the tuned configuration row nearest the
// batch's token count).  Every kernel here computes a token's values from
// that token's inputs alone, in an order fixed by the code, so a token's bits
// do not depend on the tokens beside it.  The two expert projections are the
// grouped GEMM of the library, which has the same property.
//
// All are memory-bound elementwise or gather work: coalesced 16-byte
// accesses where rows allow, no MFMA.

#include <math.h>

#include "moe_internal.h"

namespace bimoe {
namespace {

// ---------------------------------------------------------------------------
// Top-k routing: one wave per token.  Lane l holds logits l, l+64, ...; k
// rounds each take the best logit not yet taken across the wave (a larger
// logit wins, an equal one goes to the lower expert id).  A NaN logit counts
// as -inf, so every round takes an expert in 0..E-1.  Lane j keeps round j's
// choice; the weights are the softmax over the k chosen logits, summed in
// round order.
// ---------------------------------------------------------------------------
template <int PL>  // logits per lane: E <= 64 * PL
__global__ void __launch_bounds__(256)
    moe_topk(const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ ids,
             float* __restrict__ w)
{
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (t >= T)
        return;  // whole waves only: t is the same for all 64 lanes
    float v[PL];
    unsigned taken = 0;  // bit q: logit lane + 64q has been chosen
#pragma unroll
    for (int q = 0; q < PL; ++q) {
        const int e = lane + 64 * q;
        float x = e < E ? logits[(size_t)t * E + e] : -INFINITY;
        v[q] = x == x ? x : -INFINITY;
    }
    int my_e = 0;
    float my_v = 0.f;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int q = 0; q < PL; ++q) {
            const int e = lane + 64 * q;
            const bool free = e < E && !((taken >> q) & 1u);
            if (free && (v[q] > bv || (v[q] == bv && e < be))) {
                bv = v[q];
                be = e;
            }
        }
        // the best (value, id) across the wave
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const float ov = __shfl_xor(bv, d, 64);
            const int oe = __shfl_xor(be, d, 64);
            if (ov > bv || (ov == bv && oe < be)) {
                bv = ov;
                be = oe;
            }
        }
        if ((be & 63) == lane)
            taken |= 1u << (be >> 6);
        if (lane == j) {
            my_e = be;
            my_v = bv;
        }
    }
    const float top = __shfl(my_v, 0, 64);
    const float z = lane < k ? expf(my_v - top) : 0.f;
    float s = 0.f;
    for (int j = 0; j < k; ++j)
        s = s + __shfl(z, j, 64);
    if (lane < k) {
        ids[(size_t)t * k + lane] = my_e;
        w[(size_t)t * k + lane] = z / s;
    }
}

// ---------------------------------------------------------------------------
// Grouping by expert: block e places the rows of expert e.  Every block
// counts all (token, slot) pairs per expert in LDS (integer adds: the count is
// exact whatever their order), takes its base as the count of the lower
// experts, and then walks the tokens in ascending order, 256 at a time, with
// a block-wide exclusive scan giving each pair its row.  Pairs whose id is
// outside 0..E-1 get row -1 and no row.
// ---------------------------------------------------------------------------
constexpr int kPermThreads = 256;

__global__ void __launch_bounds__(kPermThreads)
    moe_permute(const int32_t* __restrict__ ids, int T, int E, int k, int32_t* __restrict__ offsets,
                int32_t* __restrict__ tok, int32_t* __restrict__ row_of)
{
    __shared__ int cnt[kMaxExperts];
    __shared__ int scan[kPermThreads];
    const int tid = threadIdx.x;
    const int e = blockIdx.x;
    const int n = T * k;
    for (int i = tid; i < E; i += kPermThreads)
        cnt[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kPermThreads) {
        const int x = ids[i];
        if (x >= 0 && x < E)
            atomicAdd(&cnt[x], 1);
    }
    __syncthreads();
    int part = 0;
    for (int i = tid; i < e; i += kPermThreads)
        part += cnt[i];
    scan[tid] = part;
    __syncthreads();
    for (int d = kPermThreads / 2; d > 0; d >>= 1) {
        if (tid < d)
            scan[tid] += scan[tid + d];
        __syncthreads();
    }
    int run = scan[0];
    if (tid == 0) {
        offsets[e + 1] = run + cnt[e];
        if (e == 0)
            offsets[0] = 0;
    }
    if (e == 0)
        for (int i = tid; i < n; i += kPermThreads) {
            const int x = ids[i];
            if (x < 0 || x >= E)
                row_of[i] = -1;
        }
    __syncthreads();
    for (int base = 0; base < T; base += kPermThreads) {
        const int t = base + tid;
        int mine = 0;
        if (t < T)
            for (int j = 0; j < k; ++j)
                mine += ids[(size_t)t * k + j] == e;
        // inclusive scan (Hillis-Steele) of the per-token counts
        scan[tid] = mine;
        __syncthreads();
        for (int d = 1; d < kPermThreads; d <<= 1) {
            const int add = tid >= d ? scan[tid - d] : 0;
            __syncthreads();
            scan[tid] += add;
            __syncthreads();
        }
        int r = run + scan[tid] - mine;
        if (t < T)
            for (int j = 0; j < k; ++j)
                if (ids[(size_t)t * k + j] == e) {
                    tok[r] = t;
                    row_of[(size_t)t * k + j] = r;
                    ++r;
                }
        run += scan[kPermThreads - 1];
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Row gather: dst[r] = src[idx[r]] (rows of `row16` 16-byte units); an index
// outside 0..nsrc-1 gives a zero row.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
    gather_rows(const uint4* __restrict__ src, int nsrc, const int32_t* __restrict__ idx, int R,
                int row16, uint4* __restrict__ dst)
{
    const long long total = (long long)R * row16;
    for (long long i = blockIdx.x * 256LL + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
        const int r = (int)(i / row16);
        const int c = (int)(i % row16);
        const int s = idx[r];
        dst[i] = (s >= 0 && s < nsrc) ? src[(size_t)s * row16 + c] : uint4{0u, 0u, 0u, 0u};
    }
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t to_bf16(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// ---------------------------------------------------------------------------
// SwiGLU: a[r][i] = bf16(g / (1 + exp(-g)) * u), g = h[r][i], u = h[r][I+i],
// four columns per thread (I is a multiple of 4).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
    swiglu(const float* __restrict__ h, int R, int I, uint16_t* __restrict__ a)
{
    const int q4 = I / 4;
    const long long total = (long long)R * q4;
    for (long long i = blockIdx.x * 256LL + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
        const int r = (int)(i / q4);
        const int c = (int)(i % q4) * 4;
        const float4 g = *reinterpret_cast<const float4*>(h + (size_t)r * 2 * I + c);
        const float4 u = *reinterpret_cast<const float4*>(h + (size_t)r * 2 * I + I + c);
        const float gg[4] = {g.x, g.y, g.z, g.w};
        const float uu[4] = {u.x, u.y, u.z, u.w};
        uint16_t out[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float sg = gg[j] / (1.0f + expf(-gg[j]));
            out[j] = to_bf16(sg * uu[j]);
        }
        uint2 packed;
        packed.x = (uint32_t)out[0] | ((uint32_t)out[1] << 16);
        packed.y = (uint32_t)out[2] | ((uint32_t)out[3] << 16);
        *reinterpret_cast<uint2*>(a + (size_t)r * I + c) = packed;
    }
}

// ---------------------------------------------------------------------------
// Weighted combine: block t computes y[t] = sum_j w[t][j] * o[row_of[t][j]]
// over the token's k slots taken in ascending expert id (a slot's position
// breaks a tie), one fp32 multiply and one fp32 add per slot, in that order.
// A row outside 0..R-1 contributes nothing.  Four columns per thread.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
    moe_combine(const float* __restrict__ o, int R, const int32_t* __restrict__ ids,
                const float* __restrict__ w, const int32_t* __restrict__ row_of, int k, int H,
                float* __restrict__ y)
{
    __shared__ int s_e[kMaxTopK];
    __shared__ int s_row[kMaxTopK];
    __shared__ float s_w[kMaxTopK];
    const int t = blockIdx.x;
    if (threadIdx.x == 0) {
        for (int j = 0; j < k; ++j) {
            const int e = ids[(size_t)t * k + j];
            const int r = row_of[(size_t)t * k + j];
            const float ww = w[(size_t)t * k + j];
            int p = j;  // insertion sort by expert id, stable
            while (p > 0 && s_e[p - 1] > e) {
                s_e[p] = s_e[p - 1];
                s_row[p] = s_row[p - 1];
                s_w[p] = s_w[p - 1];
                --p;
            }
            s_e[p] = e;
            s_row[p] = r;
            s_w[p] = ww;
        }
    }
    __syncthreads();
    for (int c = threadIdx.x * 4; c < H; c += 256 * 4) {
        float4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < k; ++j) {
            const int r = s_row[j];
            if (r < 0 || r >= R)
                continue;
            const float4 v = *reinterpret_cast<const float4*>(o + (size_t)r * H + c);
            const float ww = s_w[j];
            acc.x = acc.x + ww * v.x;
            acc.y = acc.y + ww * v.y;
            acc.z = acc.z + ww * v.z;
            acc.w = acc.w + ww * v.w;
        }
        *reinterpret_cast<float4*>(y + (size_t)t * H + c) = acc;
    }
}

int grid_for(long long work, int per_block)
{
    long long g = (work + per_block - 1) / per_block;
    const long long cap = 256LL * 64;
    return (int)(g < 1 ? 1 : (g > cap ? cap : g));
}

}  // namespace

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                       hipStream_t stream)
{
    const dim3 grid((T + 3) / 4), block(256);
    if (E <= 64)
        hipLaunchKernelGGL(moe_topk<1>, grid, block, 0, stream, logits, T, E, k, ids, w);
    else if (E <= 128)
        hipLaunchKernelGGL(moe_topk<2>, grid, block, 0, stream, logits, T, E, k, ids, w);
    else if (E <= 256)
        hipLaunchKernelGGL(moe_topk<4>, grid, block, 0, stream, logits, T, E, k, ids, w);
    else if (E <= 512)
        hipLaunchKernelGGL(moe_topk<8>, grid, block, 0, stream, logits, T, E, k, ids, w);
    else
        hipLaunchKernelGGL(moe_topk<16>, grid, block, 0, stream, logits, T, E, k, ids, w);
    return hipGetLastError();
}

hipError_t launch_permute(const int32_t* ids, int T, int E, int k, int32_t* offsets, int32_t* tok,
                          int32_t* row_of, hipStream_t stream)
{
    hipLaunchKernelGGL(moe_permute, dim3(E), dim3(kPermThreads), 0, stream, ids, T, E, k, offsets,
                       tok, row_of);
    return hipGetLastError();
}

hipError_t launch_gather(const void* src, int nsrc, const int32_t* idx, int R, int K, void* dst,
                         hipStream_t stream)
{
    const int row16 = K * 2 / 16;
    hipLaunchKernelGGL(gather_rows, dim3(grid_for((long long)R * row16, 256)), dim3(256), 0, stream,
                       static_cast<const uint4*>(src), nsrc, idx, R, row16, static_cast<uint4*>(dst));
    return hipGetLastError();
}

hipError_t launch_swiglu(const float* h, int R, int I, void* a, hipStream_t stream)
{
    hipLaunchKernelGGL(swiglu, dim3(grid_for((long long)R * (I / 4), 256)), dim3(256), 0, stream, h,
                       R, I, static_cast<uint16_t*>(a));
    return hipGetLastError();
}

hipError_t launch_combine(const float* o, int R, const int32_t* ids, const float* w,
                          const int32_t* row_of, int T, int k, int H, float* y, hipStream_t stream)
{
    hipLaunchKernelGGL(moe_combine, dim3(T), dim3(256), 0, stream, o, R, ids, w, row_of, k, H, y);
    return hipGetLastError();
}

}  // namespace bimoe
