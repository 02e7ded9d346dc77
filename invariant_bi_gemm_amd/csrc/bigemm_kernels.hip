// gfx950 kernels of the batch-invariant bf16 GEMM  y[M,N] = x[M,K] . W[N,K]^T.
//
// One reduction tree, two kernel families.  Every output element y[m][n] is
// the result of the same chain of v_mfma_f32_16x16x32_bf16 steps, whichever
// kernel, tile size or grid computes it:
//   * A operand = 16 rows of W, B operand = 16 rows of x (so the 16x16
//     accumulator tile holds D[n][m] = y[m][n]);
//   * step t covers k = 32t .. 32t+31; lane group g = lane/16 supplies
//     k = 32t + 8g .. 32t + 8g + 7 of its row (8 consecutive bf16);
//   * steps run in ascending t from a +0 accumulator, one chain per split
//     (only S = 1 is built).
// The result of an MFMA element depends only on its own A row, B column and
// accumulator (checked on the device by the library's invariance tests), so
// where a row sits in a tile, which tile or kernel handles it and what the
// other rows hold cannot change its bits.  This is the fixed tiling of CoRun
// (§III-A Fig. 3b) taken down to the instruction: the tree never depends on
// the batch, only the tiling of the output does.
//
// Kernel families:
//   bigemm_tiled   large M: 2-stage LDS pipeline fed by direct global->LDS
//                  loads, 256x256 or 128x128 output blocks, MFMA bound.
//   bigemm_stream  small M: a persistent, warp-specialised weight streamer.
//                  Two producer waves keep a deep LDS ring of W (and x) full
//                  with direct global->LDS loads; consumer waves run the MFMA
//                  chain of one 16-column tile.  HBM bound.
// Both have a grouped (MoE) variant whose per-expert row counts stay on the
// device.

#include "bigemm_internal.h"

namespace bigemm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ f32x4 mfma_step(const uint4& a, const uint4& b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// s_waitcnt that only bounds vmcnt (gfx9 encoding: vmcnt[3:0] and [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// 16 bytes per lane from global memory straight into LDS: lane L's bytes land
// at lds_base + 16 L (lds_base must be the same in every lane of the wave).
__device__ __forceinline__ void dma16(const void* src, const void* lds_base)
{
    __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_base, 16, 0, 0);
}

// Workgroup barrier for the pipelined loops.  __syncthreads() would add a
// release fence, and the compiler implements that by draining every
// outstanding direct-to-LDS load (vmcnt(0)) -- including the prefetch of the
// next stage.  These barriers order only what the loops need; the "memory"
// clobber keeps the compiler from moving LDS accesses across them.
__device__ __forceinline__ void barrier_only()
{
    asm volatile("s_barrier" ::: "memory");
}

// Barrier after this wave's LDS reads have returned (their buffer is about to
// be refilled by other waves).
__device__ __forceinline__ void barrier_after_lds_reads()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ void store4(float* p, const f32x4& v)
{
    *reinterpret_cast<f32x4*>(p) = v;
}

// ---------------------------------------------------------------------------
// Grouped rows.  Offsets are read clamped to 0..R and an expert's row count
// is max(0, off[e+1] - off[e]), so malformed offsets can never send a kernel
// outside rows 0..R-1.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int clamp_off(int v, int R) { return v < 0 ? 0 : (v > R ? R : v); }

// Which expert owns m-block `slot`.  Experts whose row count c satisfies
// cmin < c <= cmax each contribute ceil(c / bm) m-blocks, in ascending expert
// order.  Every thread of the block calls this; `sh` is E + 4 ints of LDS.
// Returns the expert (or -1 when slot is past the last m-block), its block
// index and its row range.
__device__ int grouped_find(const int32_t* __restrict__ off, int E, int R, int bm, int cmin,
                            int cmax, int slot, int* lb_out, int* lo_out, int* hi_out, int* sh)
{
    for (int e = threadIdx.x; e <= E; e += blockDim.x)
        sh[e] = clamp_off(off[e], R);
    if (threadIdx.x == 0) {
        sh[E + 1] = -1;
        sh[E + 2] = 0;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const int c = max(sh[e + 1] - sh[e], 0);
        const int mine = (c > cmin && c <= cmax) ? (c + bm - 1) / bm : 0;
        if (mine == 0)
            continue;
        int before = 0;
        for (int j = 0; j < e; ++j) {
            const int cj = max(sh[j + 1] - sh[j], 0);
            before += (cj > cmin && cj <= cmax) ? (cj + bm - 1) / bm : 0;
        }
        if (slot >= before && slot < before + mine) {
            sh[E + 1] = e;
            sh[E + 2] = slot - before;
        }
    }
    __syncthreads();
    const int e = sh[E + 1];
    *lb_out = sh[E + 2];
    if (e >= 0) {
        *lo_out = sh[e];
        *hi_out = sh[e] + max(sh[e + 1] - sh[e], 0);
    }
    __syncthreads();  // sh is reused by the caller
    return e;
}

// ---------------------------------------------------------------------------
// Tiled kernel (large M)
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN>
struct TiledCfg {
    static constexpr int kWaves = WM * WN;
    static constexpr int kThreads = kWaves * 64;
    static constexpr int TM = BM / WM;  // rows of x per wave
    static constexpr int TN = BN / WN;  // rows of W per wave
    static constexpr int FM = TM / 16;
    static constexpr int FN = TN / 16;
    // one stage = 64 values of k for BN rows of W then BM rows of x, as
    // 16-byte units (8 per row)
    static constexpr int kStageUnits = (BM + BN) * 8;
    static constexpr int kInstr = kStageUnits / (64 * kWaves);  // loads per wave per stage
    static constexpr int kLdsBytes = 2 * kStageUnits * 16;
    static_assert(kStageUnits % (64 * kWaves) == 0, "a stage must split evenly over the waves");
    static_assert(BN * 8 % 64 == 0, "one load instruction must not straddle W and x");
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tiles are whole MFMA tiles");
};

// XOR swizzle of the 16-byte chunk c (0..7) of row r in a 64-wide stage:
// the 16 lanes reading one fragment hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz8(int r, int c) { return c ^ ((r >> 1) & 7); }

// One BM x BN output block: rows m0 .. m0+BM-1 of x/y (rows at or past
// row_hi are clamped on load and never stored), columns n0 .. n0+BN-1 of y
// (rows of Wb past N are clamped likewise).
template <int BM, int BN, int WM, int WN>
__device__ __forceinline__ void tiled_block(uint4* lds, const uint16_t* __restrict__ x,
                                            const uint16_t* __restrict__ Wb,
                                            float* __restrict__ y, int m0, int row_hi, int n0,
                                            int N, int K)
{
    using C = TiledCfg<BM, BN, WM, WN>;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave % WM;
    const int wn = wave / WM;

    // Source of each of this lane's loads in a stage.  Unit u of the stage
    // (lane-linear in LDS) holds logical chunk swz8(r, u % 8) of row r.
    const uint16_t* src[C::kInstr];
#pragma unroll
    for (int j = 0; j < C::kInstr; ++j) {
        const int u = (wave * C::kInstr + j) * 64 + lane;
        if (u < BN * 8) {
            const int r = u >> 3;
            const int n = min(n0 + r, N - 1);
            src[j] = Wb + (size_t)n * K + swz8(r, u & 7) * 8;
        } else {
            const int r = (u - BN * 8) >> 3;
            const int m = min(m0 + r, row_hi - 1);
            src[j] = x + (size_t)m * K + swz8(r, (u - BN * 8) & 7) * 8;
        }
    }

    f32x4 acc[C::FN][C::FM];
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < C::FM; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = K / 64;
    auto issue = [&](int s, int buf) {
#pragma unroll
        for (int j = 0; j < C::kInstr; ++j)
            dma16(src[j] + (size_t)s * 64, lds + buf * C::kStageUnits + (wave * C::kInstr + j) * 64);
    };

    issue(0, 0);
    for (int s = 0; s < nk; ++s) {
        const int buf = s & 1;
        if (s + 1 < nk) {
            issue(s + 1, buf ^ 1);
            wait_vmcnt<C::kInstr>();  // this wave's loads of stage s have landed
        } else {
            wait_vmcnt<0>();
        }
        barrier_only();  // ... and every other wave's
        const uint4* sW = lds + buf * C::kStageUnits;
        const uint4* sX = sW + BN * 8;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int cl = ks * 4 + (lane >> 4);
            uint4 a[C::FN], b[C::FM];
#pragma unroll
            for (int t = 0; t < C::FN; ++t) {
                const int r = wn * C::TN + t * 16 + (lane & 15);
                a[t] = sW[r * 8 + swz8(r, cl)];
            }
#pragma unroll
            for (int t = 0; t < C::FM; ++t) {
                const int r = wm * C::TM + t * 16 + (lane & 15);
                b[t] = sX[r * 8 + swz8(r, cl)];
            }
#pragma unroll
            for (int i = 0; i < C::FN; ++i)
#pragma unroll
                for (int j = 0; j < C::FM; ++j)
                    acc[i][j] = mfma_step(a[i], b[j], acc[i][j]);
        }
        barrier_after_lds_reads();  // buffer `buf` is refilled at the next iteration
    }

#pragma unroll
    for (int j = 0; j < C::FM; ++j) {
        const int m = m0 + wm * C::TM + j * 16 + (lane & 15);
        if (m >= row_hi)
            continue;
#pragma unroll
        for (int i = 0; i < C::FN; ++i) {
            const int n = n0 + wn * C::TN + i * 16 + 4 * (lane >> 4);
            if (n < N)
                store4(y + (size_t)m * N + n, acc[i][j]);
        }
    }
}

// Block -> output tile, XCD aware.  Hardware hands block b to XCD b % 8; the
// remap gives each XCD a contiguous run of logical tiles, and logical tiles
// walk groups of `group_m` m-blocks column by column, so the blocks sharing
// an XCD's L2 share x rows and W rows.
__device__ __forceinline__ void tile_of_block(int b, int nblocks, int tiles_m, int tiles_n,
                                              int group_m, int* tm, int* tn)
{
    const int per_xcd = nblocks / 8;
    if (b < per_xcd * 8)
        b = (b % 8) * per_xcd + b / 8;
    const int span = group_m * tiles_n;
    const int g = b / span;
    const int first = g * group_m;
    const int rows = min(tiles_m - first, group_m);
    const int r = b % span;
    *tm = first + r % rows;
    *tn = r / rows;
}

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(WM * WN * 64)
    bigemm_tiled(const uint16_t* __restrict__ x, const uint16_t* __restrict__ W,
                 float* __restrict__ y, int M, int N, int K, int tiles_m, int tiles_n, int group_m)
{
    using C = TiledCfg<BM, BN, WM, WN>;
    __shared__ uint4 lds[2 * C::kStageUnits];
    int tm, tn;
    tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, &tm, &tn);
    tiled_block<BM, BN, WM, WN>(lds, x, W, y, tm * BM, M, tn * BN, N, K);
}

// Grouped: block (slot, tn) where slot enumerates the m-blocks of experts
// with more than cmin rows.
template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(WM * WN * 64)
    bigemm_tiled_grouped(const uint16_t* __restrict__ x, const uint16_t* __restrict__ W,
                         float* __restrict__ y, const int32_t* __restrict__ off, int E, int R,
                         int N, int K, int tiles_n, int cmin)
{
    using C = TiledCfg<BM, BN, WM, WN>;
    __shared__ uint4 lds[2 * C::kStageUnits];
    static_assert(C::kLdsBytes >= (kMaxExperts + 4) * 4, "offsets must fit the stage buffers");
    const int slot = blockIdx.x / tiles_n;
    const int tn = blockIdx.x % tiles_n;
    int lb, lo = 0, hi = 0;
    const int e = grouped_find(off, E, R, BM, cmin, 0x7fffffff, slot, &lb, &lo, &hi,
                               reinterpret_cast<int*>(lds));
    if (e < 0)
        return;
    tiled_block<BM, BN, WM, WN>(lds, x, W + (size_t)e * N * K, y, lo + lb * BM, hi, tn * BN, N, K);
}

// ---------------------------------------------------------------------------
// Streaming kernel (small M)
// ---------------------------------------------------------------------------
template <int MB, int NR, int BKS>
struct StreamCfg {
    static constexpr int kConsumers = MB;  // one per 16-row m-tile
    static constexpr int kProducers = 2;
    static constexpr int kThreads = (MB + kProducers) * 64;
    static constexpr int kChunks = BKS / 8;       // 16-byte units per row per stage
    static constexpr int kRows = 16 * (1 + MB);   // 16 rows of W, then 16*MB rows of x
    static constexpr int kStageUnits = kRows * kChunks;
    static constexpr int kInstr = kStageUnits / (64 * kProducers);  // per producer per stage
    static constexpr int kSteps = BKS / 32;
    static constexpr int kSwz = kChunks < 16 ? kChunks - 1 : 15;
    static constexpr int kLdsBytes = NR * kStageUnits * 16;
    static_assert(kStageUnits % (64 * kProducers) == 0, "a stage must split evenly");
    static_assert(kInstr * (NR - 1) < 64, "loads in flight must fit vmcnt");
    static_assert((16 * kChunks) % 64 == 0, "one load must not straddle W and x");
};

// Where work item `item` lives: rows m0.. of x/y (row_hi excluded), W rows
// n0 .. n0+15 of the expert weight *Wb.
struct StreamItem {
    int m0, row_hi, n0;
    const uint16_t* Wb;
};

template <int MB, int NR, int BKS>
__device__ __forceinline__ void stream_body(uint4* ring, const uint16_t* __restrict__ x,
                                            const uint16_t* __restrict__ W, float* __restrict__ y,
                                            int N, int K, int tiles_n, int nitems,
                                            // dense: M rows; grouped: expert list in LDS
                                            int M, const int* sh_off, const int* elist)
{
    using C = StreamCfg<MB, NR, BKS>;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int G = gridDim.x;
    const int mine = nitems > (int)blockIdx.x ? (nitems - 1 - (int)blockIdx.x) / G + 1 : 0;
    const int nst = K / BKS;
    const int total = mine * nst;

    auto item_at = [&](int it) {
        const int item = blockIdx.x + it * G;
        const int mb = item / tiles_n;
        StreamItem s;
        s.n0 = (item % tiles_n) * 16;
        if (elist) {
            const int e = elist[mb];
            s.m0 = sh_off[e];
            s.row_hi = max(sh_off[e + 1], s.m0);
            s.Wb = W + (size_t)e * N * K;
        } else {
            s.m0 = mb * 16 * MB;
            s.row_hi = M;
            s.Wb = W;
        }
        return s;
    };

    if (wave >= MB) {
        // ---- producer ----
        const int pw = wave - MB;
        auto issue = [&](int q) {
            const StreamItem s = item_at(q / nst);
            const int k0 = (q % nst) * BKS;
            uint4* dst = ring + (q % NR) * C::kStageUnits;
#pragma unroll
            for (int j = 0; j < C::kInstr; ++j) {
                const int u0 = (pw * C::kInstr + j) * 64;
                const int u = u0 + lane;
                const int r = u / C::kChunks;
                const int c = (u % C::kChunks) ^ (r & C::kSwz);
                const uint16_t* src;
                if (r < 16) {
                    src = s.Wb + (size_t)(s.n0 + r) * K + k0 + c * 8;
                } else {
                    const int m = min(s.m0 + (r - 16), s.row_hi - 1);
                    src = x + (size_t)m * K + k0 + c * 8;
                }
                dma16(src, dst + u0);
            }
        };
        const int pro = total < NR - 1 ? total : NR - 1;
        for (int q = 0; q < pro; ++q)
            issue(q);
        for (int q = 0; q < total; ++q) {
            if (q + NR - 2 <= total - 1)
                wait_vmcnt<C::kInstr * (NR - 2)>();
            else
                wait_vmcnt<0>();
            barrier_only();  // stage q is in LDS; slot (q-1) % NR is free
            if (q + NR - 1 < total)
                issue(q + NR - 1);
        }
    } else {
        // ---- consumer: the MFMA chain of m-tile `wave` ----
        const int ci = wave;
        const int rw = lane & 15;
        const int rx = 16 + 16 * ci + rw;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int q = 0; q < total; ++q) {
            // stage q is in LDS; this wave's reads of stage q-1 have returned
            barrier_after_lds_reads();
            const uint4* st = ring + (q % NR) * C::kStageUnits;
            uint4 a[C::kSteps], b[C::kSteps];
#pragma unroll
            for (int t = 0; t < C::kSteps; ++t) {
                const int cl = 4 * t + (lane >> 4);
                a[t] = st[rw * C::kChunks + (cl ^ (rw & C::kSwz))];
                b[t] = st[rx * C::kChunks + (cl ^ (rx & C::kSwz))];
            }
#pragma unroll
            for (int t = 0; t < C::kSteps; ++t)
                acc = mfma_step(a[t], b[t], acc);
            if ((q + 1) % nst == 0) {
                const StreamItem s = item_at(q / nst);
                const int m = s.m0 + 16 * ci + rw;
                if (m < s.row_hi)
                    store4(y + (size_t)m * N + s.n0 + 4 * (lane >> 4), acc);
                acc = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    }
}

template <int MB, int NR, int BKS>
__global__ void __launch_bounds__((MB + 2) * 64)
    bigemm_stream(const uint16_t* __restrict__ x, const uint16_t* __restrict__ W,
                  float* __restrict__ y, int M, int N, int K)
{
    using C = StreamCfg<MB, NR, BKS>;
    __shared__ uint4 ring[NR * C::kStageUnits];
    const int tiles_n = N / 16;
    const int mblocks = (M + 16 * MB - 1) / (16 * MB);
    stream_body<MB, NR, BKS>(ring, x, W, y, N, K, tiles_n, mblocks * tiles_n, M, nullptr, nullptr);
}

// Grouped: one m-block per expert whose row count c satisfies 0 < c <= cmax
// (cmax <= 16 * MB).
template <int MB, int NR, int BKS>
__global__ void __launch_bounds__((MB + 2) * 64)
    bigemm_stream_grouped(const uint16_t* __restrict__ x, const uint16_t* __restrict__ W,
                          float* __restrict__ y, const int32_t* __restrict__ off, int E, int R,
                          int N, int K, int cmax)
{
    using C = StreamCfg<MB, NR, BKS>;
    __shared__ uint4 ring[NR * C::kStageUnits];
    __shared__ int sh_off[kMaxExperts + 1];
    __shared__ int elist[kMaxExperts + 1];
    // compact, ascending list of the experts this kernel serves
    for (int e = threadIdx.x; e <= E; e += blockDim.x)
        sh_off[e] = clamp_off(off[e], R);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const int c = sh_off[e + 1] - sh_off[e];
        if (c > 0 && c <= cmax) {
            int before = 0;
            for (int j = 0; j < e; ++j) {
                const int cj = sh_off[j + 1] - sh_off[j];
                before += (cj > 0 && cj <= cmax) ? 1 : 0;
            }
            elist[before] = e;
        }
    }
    if (threadIdx.x == 0) {
        int n = 0;
        for (int j = 0; j < E; ++j) {
            const int cj = sh_off[j + 1] - sh_off[j];
            n += (cj > 0 && cj <= cmax) ? 1 : 0;
        }
        elist[kMaxExperts] = n;
    }
    __syncthreads();
    const int tiles_n = N / 16;
    const int count = elist[kMaxExperts];
    stream_body<MB, NR, BKS>(ring, x, W, y, N, K, tiles_n, count * tiles_n, 0, sh_off, elist);
}

// ---------------------------------------------------------------------------
// Launch helpers
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN>
hipError_t run_tiled(const void* W, const void* x, int M, float* y, int N, int K,
                     hipStream_t stream)
{
    using C = TiledCfg<BM, BN, WM, WN>;
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    const int nblocks = tiles_m * tiles_n;
    hipLaunchKernelGGL((bigemm_tiled<BM, BN, WM, WN>), dim3(nblocks), dim3(C::kThreads), 0, stream,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W), y, M, N, K,
                       tiles_m, tiles_n, 4);
    return hipGetLastError();
}

template <int MB, int NR, int BKS>
hipError_t run_stream(const void* W, const void* x, int M, float* y, int N, int K, int num_cus,
                      hipStream_t stream)
{
    using C = StreamCfg<MB, NR, BKS>;
    const int items = ((M + 16 * MB - 1) / (16 * MB)) * (N / 16);
    const int grid = items < num_cus ? items : num_cus;
    hipLaunchKernelGGL((bigemm_stream<MB, NR, BKS>), dim3(grid), dim3(C::kThreads), 0, stream,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W), y, M, N, K);
    return hipGetLastError();
}

template <int MB, int NR>
hipError_t run_stream_k(const void* W, const void* x, int M, float* y, int N, int K, int num_cus,
                        hipStream_t stream)
{
    if (K % 256 == 0)
        return run_stream<MB, NR, 256>(W, x, M, y, N, K, num_cus, stream);
    if (K % 128 == 0)
        return run_stream<MB, NR, 128>(W, x, M, y, N, K, num_cus, stream);
    return run_stream<MB, NR, 64>(W, x, M, y, N, K, num_cus, stream);
}

template <int MB, int NR, int BKS>
hipError_t run_stream_grouped(const void* W, const void* x, const int32_t* off, int E, int R,
                              float* y, int N, int K, int cmax, int num_cus, hipStream_t stream)
{
    using C = StreamCfg<MB, NR, BKS>;
    hipLaunchKernelGGL((bigemm_stream_grouped<MB, NR, BKS>), dim3(num_cus), dim3(C::kThreads), 0,
                       stream, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W), y,
                       off, E, R, N, K, cmax);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
hipError_t run_tiled_grouped(const void* W, const void* x, const int32_t* off, int E, int R,
                             float* y, int N, int K, int cmin, hipStream_t stream)
{
    using C = TiledCfg<BM, BN, WM, WN>;
    const int tiles_n = (N + BN - 1) / BN;
    // m-blocks of experts with more than cmin rows: at most R/BM + (number of
    // such experts), and there are at most min(E, R/(cmin+1)) of those.
    const long long big = R / (cmin + 1);
    const long long slots = (R + BM - 1) / BM + (big < E ? big : E);
    const long long nblocks = slots * tiles_n;
    if (nblocks <= 0)
        return hipSuccess;
    hipLaunchKernelGGL((bigemm_tiled_grouped<BM, BN, WM, WN>), dim3((unsigned)nblocks),
                       dim3(C::kThreads), 0, stream, static_cast<const uint16_t*>(x),
                       static_cast<const uint16_t*>(W), y, off, E, R, N, K, tiles_n, cmin);
    return hipGetLastError();
}

}  // namespace

DenseKernel choose_dense(const Plan& p, int M)
{
    if (M <= p.stream_max_m)
        return M <= 16 ? DenseKernel::kStream16 : DenseKernel::kStream32;
    return M >= 1024 ? DenseKernel::kTiled256 : DenseKernel::kTiled128;
}

const char* dense_kernel_name(DenseKernel k)
{
    switch (k) {
    case DenseKernel::kStream16: return "bigemm_stream<mb=1>";
    case DenseKernel::kStream32: return "bigemm_stream<mb=2>";
    case DenseKernel::kTiled128: return "bigemm_tiled<128x128>";
    case DenseKernel::kTiled256: return "bigemm_tiled<256x256>";
    }
    return "?";
}

hipError_t launch_dense(const Plan& p, const void* W, const void* x, int M, float* y,
                        hipStream_t stream)
{
    switch (choose_dense(p, M)) {
    case DenseKernel::kStream16:
        return run_stream_k<1, 8>(W, x, M, y, p.n, p.k, p.num_cus, stream);
    case DenseKernel::kStream32:
        return run_stream_k<2, 5>(W, x, M, y, p.n, p.k, p.num_cus, stream);
    case DenseKernel::kTiled256:
        return run_tiled<256, 256, 2, 4>(W, x, M, y, p.n, p.k, stream);
    case DenseKernel::kTiled128:
        break;
    }
    return run_tiled<128, 128, 2, 2>(W, x, M, y, p.n, p.k, stream);
}

hipError_t launch_grouped(const Plan& p, const void* W, const void* x, const int32_t* offsets,
                          int R, float* y, hipStream_t stream)
{
    // Experts with 1..smax rows go to the streaming kernel, the rest to the
    // tiled kernel; both realise the same tree, so the split point only
    // moves work, never bits.
    const int smax = p.stream_max_m < 16 ? p.stream_max_m : 16;
    hipError_t err = hipSuccess;
    if (smax > 0) {
        if (p.k % 256 == 0)
            err = run_stream_grouped<1, 8, 256>(W, x, offsets, p.experts, R, y, p.n, p.k, smax, p.num_cus, stream);
        else if (p.k % 128 == 0)
            err = run_stream_grouped<1, 8, 128>(W, x, offsets, p.experts, R, y, p.n, p.k, smax, p.num_cus, stream);
        else
            err = run_stream_grouped<1, 8, 64>(W, x, offsets, p.experts, R, y, p.n, p.k, smax, p.num_cus, stream);
        if (err != hipSuccess)
            return err;
    }
    return run_tiled_grouped<128, 128, 2, 2>(W, x, offsets, p.experts, R, y, p.n, p.k, smax, stream);
}

}  // namespace bigemm
