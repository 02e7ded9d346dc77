// gfx950 kernels of batch-invariant decode attention (include/bi_attn.h).
//
// Two kernels: the split kernel computes each split's partial softmax (max,
// sum, weighted values) for the query heads that share a kv head, in one
// pass over its keys; the combine kernel rescales and sums the splits in
// ascending order.  Split
// boundaries are every S keys of the sequence (Detent, §8.1 Kernels: the
// fixed split-size principle), so nothing here depends on the batch.
//
// Every key and value is read once (512 bytes per token and kv head at
// D = 128) and reused by the Hq/Hkv query heads from registers.  The dot
// products are short (8 per lane, 16 lanes) and run on the VALU -- at most 8
// query rows share a key, too few for MFMA tiles -- with v_dot2_f32_bf16 for
// the scores (two bf16 products into the fp32 sum per instruction) and fused
// multiply-adds for the weighted values, so that the VALU keeps up with HBM
// (a wave64 VALU instruction occupies a 16-lane SIMD for four cycles).

#include <math.h>

#include "attn_internal.h"
#include "bf16_round.h"

namespace biattn {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// sum + a.lo * b.lo + a.hi * b.hi for bf16 pairs (v_dot2_f32_bf16)
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float sum)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), sum,
                                           false);
}

constexpr int kThreads = 256;  // 4 waves = 16 groups of 16 lanes
constexpr int kGroups = 16;
// keys per group in flight: 8, or 4 when 8 query heads share a kv head
template <int G>
constexpr int unroll_of() { return G <= 4 ? 8 : 4; }

// Sum over the 16 lanes of a row (DPP rotations by 8, 4, 2, 1 inside the
// row): at every level a lane adds the partner the xor butterfly would give
// it (the values are periodic in the rotation distance by then), so this is
// that butterfly's tree, every lane ending with the same total -- on the
// VALU, without LDS permutes.
__device__ __forceinline__ float row_sum16(float x)
{
    x = x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
    x = x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));
    x = x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xf, 0xf, false));
    x = x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xf, 0xf, false));
    return x;
}

__device__ __forceinline__ void widen8(const uint4& v, float* f)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = bi::from_bf16(w[e] & 0xffffu);
        f[2 * e + 1] = bi::from_bf16(w[e] >> 16);
    }
}

// A raw buffer resource over `bytes` bytes at `base`: a load whose offset
// reaches past the end returns zeros (the hardware's range check on the
// per-lane offset), which is what a key past the end of a split must read.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane, non-temporal (the cache-policy operand's nt bit): a call
// reads each key and value once, and the stream of them then does not evict
// what stays in use from the caches (the split partials the combine reads,
// the output of earlier calls).  Measured at S = 512 on the 256-sequence
// batch: 282-283 -> 264 us per call, interleaved on one box.
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voff)
{
    constexpr int kNonTemporal = 2;
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kNonTemporal));
}

// Sum over the 16 lanes of a row for n values at once: the same four DPP
// levels as row_sum16, each level applied to all n values before the next,
// so that no add waits on the one just before it.
template <int N>
__device__ __forceinline__ void row_sum16_n(float* x)
{
#pragma unroll
    for (int i = 0; i < N; ++i)
        x[i] = x[i] + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x[i]), 0x128, 0xf, 0xf, false));
#pragma unroll
    for (int i = 0; i < N; ++i)
        x[i] = x[i] + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x[i]), 0x124, 0xf, 0xf, false));
#pragma unroll
    for (int i = 0; i < N; ++i)
        x[i] = x[i] + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x[i]), 0x122, 0xf, 0xf, false));
#pragma unroll
    for (int i = 0; i < N; ++i)
        x[i] = x[i] + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x[i]), 0x121, 0xf, 0xf, false));
}

// Sequence b's length, clamped as the kernels read it.
__device__ __forceinline__ int seq_len(const int32_t* __restrict__ seq_start, int b, int Ntok, int max_len,
                                       int* t0out)
{
    int t0 = seq_start[b], t1 = seq_start[b + 1];
    t0 = t0 < 0 ? 0 : (t0 > Ntok ? Ntok : t0);
    t1 = t1 < t0 ? t0 : (t1 > Ntok ? Ntok : t1);
    *t0out = t0;
    return min(t1 - t0, max_len);
}

// The work list: plan[b] = splits of the sequences before b, plan[B] = all
// splits, and plan[B + 1] = 0, the counter the split kernel's blocks take
// work items from.  One block of 1024 threads, 1024 sequences at a time: a wave
// scan, then the 16 wave totals in order.
constexpr int kPlanThreads = 1024;

__global__ void __launch_bounds__(kPlanThreads)
    attn_plan(const int32_t* __restrict__ seq_start, int B, int S, int max_len, int Ntok, int* __restrict__ plan)
{
    __shared__ int s_w[kPlanThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int carry = 0;
    for (int base = 0; base < B; base += kPlanThreads) {
        const int b = base + tid;
        int t0;
        const int c = b < B ? (seq_len(seq_start, b, Ntok, max_len, &t0) + S - 1) / S : 0;
        int v = c;  // inclusive scan inside the wave
        for (int d = 1; d < 64; d <<= 1) {
            const int u = __shfl_up(v, d, 64);
            if (lane >= d)
                v += u;
        }
        if (lane == 63)
            s_w[wave] = v;
        __syncthreads();
        int before = carry;
        for (int w = 0; w < wave; ++w)
            before += s_w[w];
        if (b < B)
            plan[b] = before + v - c;
        for (int w = 0; w < kPlanThreads / 64; ++w)
            carry += s_w[w];
        __syncthreads();
    }
    if (tid == 0) {
        plan[B] = carry;
        plan[B + 1] = 0;
    }
}

// Persistent: the blocks take the work items (split, kv head) of all
// sequences from a counter (queue), in the order of the plan, kv heads
// fastest, so that the Hkv blocks of one split read whole token rows
// together, and a block that finishes early takes the next item: the splits
// are ragged (a sequence's last one is partial), and a fixed share per block
// would leave the kernel waiting on the blocks dealt the most keys.  Which
// block computes an item changes no bit: each item writes its own partials.  G query heads share
// the kv head.
// One pass over the split's keys: each 16-lane group keeps, per head, a
// running max m, sum l and weighted sum o of its keys (flash-decoding's
// online softmax, in log2 units: scores are scaled by scale * log2(e) and
// exponentials are exp2), loading the keys and values of kUnroll keys
// together.  Then the 16 groups are combined in a fixed order.
template <int G>
__global__ void __launch_bounds__(kThreads)
    attn_split(const uint4* __restrict__ q, const uint4* __restrict__ k, const uint4* __restrict__ v,
               const int32_t* __restrict__ seq_start, const int* __restrict__ plan, int* __restrict__ queue,
               int B, int Hkv, int S, int max_len, int Ntok, float scale_l2, float* __restrict__ ws_o,
               float* __restrict__ ws_ml, int splits)
{
    __shared__ float s_m[4][G];
    __shared__ float s_l[4][G];
    __shared__ float s_o[4][G][kHeadDim];
    __shared__ int s_item;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = wave * 4 + (lane >> 4), r = lane & 15;
    const int items = plan[B] * Hkv;
    for (;;) {
    if (tid == 0)
        s_item = atomicAdd(queue, 1);
    __syncthreads();
    // every thread reads the same value: kept uniform, so that the buffer
    // descriptors built from the item stay in scalar registers
    const int item = __builtin_amdgcn_readfirstlane(s_item);
    if (item >= items)
        break;
    const int kvh = item % Hkv, pair = item / Hkv;
    int lo = 0, hi = B;  // the sequence: the last b with plan[b] <= pair
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (plan[mid] <= pair)
            lo = mid;
        else
            hi = mid;
    }
    const int b = lo, j = pair - plan[b];
    int t0;
    const int n = seq_len(seq_start, b, Ntok, max_len, &t0);
    const int first = j * S;
    const int cnt = min(S, n - first);
    const int Hq = Hkv * G;
    const size_t row16 = (size_t)Hkv * (kHeadDim / 8);  // uint4 per token row
    // the split's keys and values of this kv head as buffers that end after
    // key cnt-1; lane r reads bytes 16r .. 16r+15 of a key's head row
    const uint32_t rowb = (uint32_t)row16 * 16;
    const __amdgpu_buffer_rsrc_t rK =
        make_rsrc(k + (size_t)(t0 + first) * row16 + (size_t)kvh * (kHeadDim / 8), (uint32_t)cnt * rowb);
    const __amdgpu_buffer_rsrc_t rV =
        make_rsrc(v + (size_t)(t0 + first) * row16 + (size_t)kvh * (kHeadDim / 8), (uint32_t)cnt * rowb);

    // query slices of the G heads, dims 8r .. 8r+7, as four bf16 pairs
    uint32_t qp[G][4];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const uint4 qq = q[((size_t)b * Hq + kvh * G + g) * (kHeadDim / 8) + r];
        qp[g][0] = qq.x;
        qp[g][1] = qq.y;
        qp[g][2] = qq.z;
        qp[g][3] = qq.w;
    }
    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[g][e] = 0.f;
    }

    // group grp takes keys grp, grp+16, ..., kUnroll at a time in ascending order
    constexpr int kUnroll = unroll_of<G>();
    // byte offset of key kidx's slice; keys past the split read as zeros
    // (the buffers end there), and an index past it is clamped to cnt so that
    // the 32-bit offset cannot wrap back into the split
    auto key_off = [&](int kidx) { return (uint32_t)min(kidx, cnt) * rowb + (uint32_t)r * 16; };
    for (int t = grp; t < cnt; t += kGroups * kUnroll) {
        uint4 kk[kUnroll], vv[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t off = key_off(t + kGroups * u);
            kk[u] = load16(rK, off);
            vv[u] = load16(rV, off);
        }
        float sc[kUnroll][G];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t kp[4] = {kk[u].x, kk[u].y, kk[u].z, kk[u].w};
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float a = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    a = dot2(kp[e], qp[g][e], a);
                sc[u][g] = a;
            }
        }
        row_sum16_n<kUnroll * G>(&sc[0][0]);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const bool live = t + kGroups * u < cnt;
#pragma unroll
            for (int g = 0; g < G; ++g)
                sc[u][g] = live ? sc[u][g] * scale_l2 : -INFINITY;
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float cm = sc[0][g];  // key t is live: cm is finite
#pragma unroll
            for (int u = 1; u < kUnroll; ++u)
                cm = fmaxf(cm, sc[u][g]);
            const float mn = fmaxf(m[g], cm);
            const float c = __builtin_amdgcn_exp2f(m[g] - mn);  // 0 on the first chunk
            l[g] = l[g] * c;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[g][e] = acc[g][e] * c;
            m[g] = mn;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float vf[8];
            widen8(vv[u], vf);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float pw = __builtin_amdgcn_exp2f(sc[u][g] - m[g]);  // 0 past the split
                l[g] = l[g] + pw;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[g][e] = __builtin_fmaf(pw, vf[e], acc[g][e]);
            }
        }
    }

    // combine the 16 groups: the block max M (exact), each group's weight
    // w = exp2(m - M), then w*l and w*o summed: the four groups of a wave in
    // order (lanes 16, 32, 48 apart), then the four waves in order.  A group
    // without keys has m = -inf, weight 0 and zero sums.
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float mx = fmaxf(fmaxf(m[g], __shfl(m[g], r + 16, 64)), fmaxf(__shfl(m[g], r + 32, 64), __shfl(m[g], r + 48, 64)));
        if (lane == 0)
            s_m[wave][g] = mx;
    }
    __syncthreads();
    float M[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
        M[g] = fmaxf(fmaxf(s_m[0][g], s_m[1][g]), fmaxf(s_m[2][g], s_m[3][g]));
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float w = m[g] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[g] - M[g]);
        const float lw = l[g] * w;
        float L = lw;
        L = L + __shfl(lw, r + 16, 64);
        L = L + __shfl(lw, r + 32, 64);
        L = L + __shfl(lw, r + 48, 64);
        if (lane == 0)
            s_l[wave][g] = L;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float ow = acc[g][e] * w;
            float o = ow;
            o = o + __shfl(ow, r + 16, 64);
            o = o + __shfl(ow, r + 32, 64);
            o = o + __shfl(ow, r + 48, 64);
            if (lane < 16)
                s_o[wave][g][8 * r + e] = o;
        }
    }
    __syncthreads();
    const size_t base = ((size_t)b * Hq + kvh * G) * splits + j;
    for (int idx = tid; idx < G * kHeadDim; idx += kThreads) {
        const int g = idx / kHeadDim, dd = idx % kHeadDim;
        const float o = ((s_o[0][g][dd] + s_o[1][g][dd]) + s_o[2][g][dd]) + s_o[3][g][dd];
        ws_o[(base + (size_t)g * splits) * kHeadDim + dd] = o;
    }
    if (tid < G) {
        const int g = tid;
        ws_ml[(base + (size_t)g * splits) * 2] = M[g];
        ws_ml[(base + (size_t)g * splits) * 2 + 1] = ((s_l[0][g] + s_l[1][g]) + s_l[2][g]) + s_l[3][g];
    }
    __syncthreads();  // the shared buffers are refilled by the next item
    }
}

// The largest of the 64 lanes' values (fmax is exact, so the order of the
// butterfly does not matter), in every lane.
__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1)
        x = fmaxf(x, __shfl_xor(x, d, 64));
    return x;
}

// One (sequence, query head) per wave, two dimensions per lane.  Lane j
// holds split j's max and sum (64 splits at a time), so the splits' maxima
// and weights come from one load and a butterfly; the rescaled sums then run
// in ascending split order, four splits' partial outputs loaded together.
constexpr int kCombineWaves = 4;

__global__ void __launch_bounds__(64 * kCombineWaves)
    attn_combine(const int32_t* __restrict__ seq_start, int BH, int Hq, int S, int max_len, int Ntok,
                 const float* __restrict__ ws_o, const float* __restrict__ ws_ml, int splits,
                 float* __restrict__ out)
{
    const int bh = (int)blockIdx.x * kCombineWaves + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    if (bh >= BH)
        return;
    const int lane = threadIdx.x & 63;
    const int b = bh / Hq;
    int t0;
    const int n = seq_len(seq_start, b, Ntok, max_len, &t0);
    const int ns = (n + S - 1) / S;
    float2* o = reinterpret_cast<float2*>(out + (size_t)bh * kHeadDim) + lane;
    if (ns == 0) {
        *o = make_float2(0.f, 0.f);
        return;
    }
    const float2* ml = reinterpret_cast<const float2*>(ws_ml + (size_t)bh * splits * 2);  // (m, l) per split
    const float2* po = reinterpret_cast<const float2*>(ws_o + (size_t)bh * splits * kHeadDim) + lane;
    float M = -INFINITY;
    for (int c = 0; c < ns; c += 64)
        M = fmaxf(M, wave_max(c + lane < ns ? ml[c + lane].x : -INFINITY));
    float ox = 0.f, oy = 0.f, L = 0.f;
    for (int c = 0; c < ns; c += 64) {
        float wj = 0.f, lj = 0.f;
        if (c + lane < ns) {
            const float2 mlj = ml[c + lane];
            wj = __builtin_amdgcn_exp2f(mlj.x - M);
            lj = mlj.y;
        }
        // split c + t: its weight and sum from lane t, its outputs from memory
        auto add = [&](int t, float2 p) {
            const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wj), t));
            const float l = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lj), t));
            ox = ox + w * p.x;
            oy = oy + w * p.y;
            L = L + w * l;
        };
        const int cn = min(64, ns - c);
        int t = 0;
        for (; t + 4 <= cn; t += 4) {
            float2 p[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                p[u] = po[(size_t)(c + t + u) * (kHeadDim / 2)];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                add(t + u, p[u]);
        }
        for (; t < cn; ++t)
            add(t, po[(size_t)(c + t) * (kHeadDim / 2)]);
    }
    *o = make_float2(__fdiv_rn(ox, L), __fdiv_rn(oy, L));
}


template <int G>
hipError_t launch_g(const void* q, const void* k, const void* v, const int32_t* seq_start, int B, int Hkv,
                    int S, int max_len, int Ntok, float scale, const Workspace& ws, float* out,
                    hipStream_t stream)
{
    hipLaunchKernelGGL(attn_plan, dim3(1), dim3(kPlanThreads), 0, stream, seq_start, B, S, max_len, Ntok,
                       ws.plan);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    // scores in log2 units, so that exponentials are exp2 (v_exp_f32)
    const float scale_l2 = scale * 1.4426950408889634f;
    // persistent grid: as many blocks as are resident on the GPU at once
    // (a host-side occupancy query, made once per kernel)
    static const int per_cu = [] {
        int nb = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, attn_split<G>, kThreads, 0) != hipSuccess || nb < 1)
            nb = 1;
        return nb;
    }();
    hipLaunchKernelGGL(attn_split<G>, dim3(ws.num_cus * per_cu), dim3(kThreads), 0, stream,
                       static_cast<const uint4*>(q), static_cast<const uint4*>(k), static_cast<const uint4*>(v),
                       seq_start, ws.plan, ws.plan + B + 1, B, Hkv, S, max_len, Ntok, scale_l2, ws.o, ws.ml,
                       ws.splits);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int BH = B * Hkv * G;
    hipLaunchKernelGGL(attn_combine, dim3((BH + kCombineWaves - 1) / kCombineWaves), dim3(64 * kCombineWaves), 0,
                       stream, seq_start, BH, Hkv * G, S, max_len, Ntok, ws.o, ws.ml, ws.splits, out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const void* q, const void* k, const void* v, const int32_t* seq_start, int B,
                         int Hq, int Hkv, int S, int max_len, int Ntok, float scale, const Workspace& ws,
                         float* out, hipStream_t stream)
{
    switch (Hq / Hkv) {
    case 1: return launch_g<1>(q, k, v, seq_start, B, Hkv, S, max_len, Ntok, scale, ws, out, stream);
    case 2: return launch_g<2>(q, k, v, seq_start, B, Hkv, S, max_len, Ntok, scale, ws, out, stream);
    case 4: return launch_g<4>(q, k, v, seq_start, B, Hkv, S, max_len, Ntok, scale, ws, out, stream);
    case 8: return launch_g<8>(q, k, v, seq_start, B, Hkv, S, max_len, Ntok, scale, ws, out, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace biattn
