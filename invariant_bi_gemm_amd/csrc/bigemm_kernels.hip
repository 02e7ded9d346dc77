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
//     of S contiguous equal K ranges; the split results are added in order,
//     ((p0 + p1) + p2) + ..., in fp32 round-to-nearest-even.
// The result of an MFMA element depends only on its own A row, B column and
// accumulator (checked on the device by the library's invariance tests), so
// where a row sits in a tile, which tile or kernel handles it and what the
// other rows hold cannot change its bits.  This is the fixed tiling of CoRun
// (§III-A Fig. 3b) taken down to the instruction: the tree never depends on
// the batch, only the tiling of the output does.
//
// Kernel families:
//   bigemm_tiled   mid M: an NS-stage LDS pipeline fed by direct
//                  buffer->LDS loads, one barrier per stage, output blocks
//                  from 64x32 to 128x128 (x rows by W rows) chosen by M.
//   bigemm_tiled4  large M: 128x256 and 256x256 blocks, four waves with
//                  their accumulators in the accumulation registers.
//   bigemm_stream  small M: a persistent, warp-specialised weight streamer.
//                  Up to seven producer waves keep a deep LDS ring of W (and
//                  x) full with direct buffer->LDS loads; consumer waves run
//                  the MFMA chains of a 16-, 32- or 64-column W strip.  HBM
//                  bound; a call with one 16-row m-block reads each W line
//                  once and loads W non-temporally.
// Each has a grouped (MoE) variant whose per-expert row counts stay on the
// device.  Every kernel reads W from the handle's packed copy (slab-major,
// made at create by bigemm_pack_w); x and y are row-major.

#include <type_traits>

#include "bf16_round.h"
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

// A raw buffer resource over `bytes` bytes at `base`.  A load past the end
// returns zeros and touches no memory: the kernels aim the loads of padding
// rows (past the last row of x or W) there.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// 16 bytes per lane from the buffer at voff + soff straight into LDS: lane
// L's bytes land at lds_base + 16 L (lds_base is wave-uniform; it goes to M0).
// Cache-policy operand of a load marking it non-temporal (the nt bit).  A
// line read once then does not displace cached lines that will be read or
// written again: in particular it leaves in the Infinity Cache the output an
// earlier large call has just written, which the same stream would otherwise
// write back to HBM while these loads run.
constexpr int kCachePolicyNT = 2;
template <int kAux = 0>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                      const void* lds_base)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, voff, soff, 0, kAux);
}

// The same load, written out.  The compiler then does not see a store into
// LDS and does not wait for the load before later LDS reads; the caller
// orders them (vmcnt waits and barriers).  M0 takes the LDS address; an
// SALU write of M0 needs one wait state before the load reads it (the nop).
typedef int sgpr4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ sgpr4 rsrc_words(const void* base, uint32_t bytes)
{
    // the arguments are wave-uniform; readfirstlane makes that plain to the
    // compiler, which must keep the descriptor in scalar registers
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return sgpr4{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                 __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu)),
                 __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}
// kNt: the load carries the non-temporal bit (data read once).
template <bool kNt = false>
__device__ __forceinline__ void dma16_asm(const sgpr4& r, uint32_t voff, uint32_t soff, const void* lds_base)
{
    const uint32_t m0v = (uint32_t)(uintptr_t)((lds_void*)lds_base);
    if constexpr (kNt)
        asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen nt lds" ::"v"(voff), "s"(r), "s"(soff),
                     "{m0}"(m0v)
                     : "memory");
    else
        asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(r), "s"(soff), "{m0}"(m0v)
                     : "memory");
}

// Packed weights.  A handle holds W (per expert) slab-major: slab s is the
// k range 64s .. 64s+63 of all N rows, one contiguous [N][64] block, so
// element (n, k) sits at bf16 index (k / 64) * 64N + 64n + k % 64.  A stage
// of BN rows is then BN * 128 contiguous bytes instead of 128 bytes in each
// of BN rows 2K bytes apart, and the blocks that run together read one
// contiguous region.  The offsets below are in bytes, relative to row n0 of
// slab 0 (base W + 64 n0).
constexpr int kSlab = 64;
// 16-byte chunk c (0..7) of row n0 + r within a slab
__device__ __forceinline__ uint32_t wpk_row(int r, int c) { return (uint32_t)r * (kSlab * 2) + (uint32_t)c * 16; }
// the slab that starts at k (a multiple of 64)
__device__ __forceinline__ uint32_t wpk_slab(int k, int N) { return (uint32_t)k * (uint32_t)N * 2; }
// bytes from row n0 of slab 0 to the end of row n0 + rows - 1 of the last slab
__device__ __forceinline__ uint32_t wpk_bytes(int N, int K, int rows)
{
    return wpk_slab(K - kSlab, N) + (uint32_t)rows * (kSlab * 2);
}

// Workgroup barrier for the pipelined loops.  __syncthreads() would add a
// release fence, which the compiler implements by draining every outstanding
// direct-to-LDS load (vmcnt(0)) -- including the prefetch of later stages.
// This barrier first waits for the wave's own LDS reads (their buffer is
// refilled by other waves after it); the "memory" clobber keeps the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void barrier_after_lds_reads()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ void store4(float* p, const f32x4& v)
{
    *reinterpret_cast<f32x4*>(p) = v;
}

// One split of the reduction: values k0 .. k0+klen-1 of every row.  Split 0
// stores its chain's result; split s > 0 adds its chain's result to what
// splits 0..s-1 left in y, in fp32 round-to-nearest-even, so that y ends as
// ((p0 + p1) + p2) + ...  The splits run as consecutive launches on one
// stream, which orders them.
struct Split {
    int k0, klen, fold;
};

__device__ __forceinline__ void emit4(float* p, const f32x4& v, int fold)
{
    if (fold) {
        const f32x4 prev = *reinterpret_cast<const f32x4*>(p);
        store4(p, prev + v);
    } else {
        store4(p, v);
    }
}

// Concurrent K splits: the kernels instantiated with kMode == kCmp run split
// blockIdx.y of gridDim.y, each a chain over its own K range from +0; split 0
// stores into y and split s > 0 into partial s - 1 of `part` ([splits-1][M][N]),
// which splitk_reduce then adds to y in split order, ((p0 + p1) + p2) + ...
// Two callers: a pin whose tiling runs its S splits concurrently (the same
// tree as the splits one after another, so the same bits), and the
// non-invariant comparison path (bi_gemm_run_splitk), where the caller picks
// the split count per call.
// What a dense kernel instance does: the product GEMM, the comparison
// path's concurrent split-K, the product GEMM of RMSNorm'd rows (x raw,
// normalised in LDS before the MFMAs), or (streaming kernel) the product GEMM
// of a call whose W is read exactly once, with non-temporal W loads.
enum Mode { kPlain = 0, kCmp = 1, kNormX = 2, kStreamOnce = 3 };

template <int kMode>
__device__ __forceinline__ float* cmp_split(Split& sp, float* y, float* part, int M, int N)
{
    if constexpr (kMode == kCmp) {
        sp.k0 = (int)blockIdx.y * sp.klen;
        sp.fold = 0;
        if (blockIdx.y > 0)
            return part + (size_t)(blockIdx.y - 1) * M * N;
    }
    return y;
}

// XOR swizzle of 16-byte chunk c of row r in an LDS tile whose rows hold kCh
// chunks.  An MFMA fragment read has 16 lanes reading one chunk of 16
// consecutive rows.  The XOR terms are the ones measured free of LDS bank
// conflicts on gfx950 for exactly that read (SQ_LDS_BANK_CONFLICT = 0 for a
// ds_read_b128 of 16 rows x 4 chunks), per row width: 64-byte rows
// (r >> 1) & 3, 128-byte rows (r >> 1) & 7, 256- and 512-byte rows r & 15.
template <int kCh>
__device__ __forceinline__ int swz(int r, int c)
{
    if constexpr (kCh >= 16)
        return c ^ (r & 15);
    else if constexpr (kCh == 8)
        return c ^ ((r >> 1) & 7);
    else
        return c ^ ((r >> 1) & 3);
}

// ---------------------------------------------------------------------------
// Grouped rows.  Offsets are read clamped to 0..R and an expert's row count
// is max(0, off[e+1] - off[e]), so malformed offsets can never send a kernel
// outside rows 0..R-1.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int clamp_off(int v, int R) { return v < 0 ? 0 : (v > R ? R : v); }

// When it is launched, the four-wave kernel takes all the rows of every
// expert above the streaming threshold, in blocks of 256 rows; the last block
// holds the rest, as a 128x256 block when at most 128 rows are left.
// big_count: the blocks of an expert with c rows; big_rows: the rows they
// cover (big = 0: the kernel is not launched and the tiled kernel serves
// them).
__device__ __forceinline__ int big_count(int c) { return (c + 255) / 256; }
__device__ __forceinline__ int big_rows(int c, int big) { return big > 0 ? c : 0; }

// Plan of a grouped call, built by every block in its own LDS: s_off[e] =
// offsets[e] clamped to 0..R, and s_first[e] = the m-blocks of the experts
// before e that the kernel serves (row count c with cmin < c <= cmax; the
// rows past big_rows(c, big), in ceil(rows / bm) m-blocks, or one when bm
// is 0); s_first[E] is their total.  Wave 0 scans 64 experts at a time.
__device__ void grouped_plan(const int32_t* __restrict__ off, int E, int R, int bm, int cmin,
                             int cmax, int big, int* s_off, int* s_first)
{
    for (int e = threadIdx.x; e <= E; e += blockDim.x)
        s_off[e] = clamp_off(off[e], R);
    __syncthreads();
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int carry = 0;
        for (int base = 0; base < E; base += 64) {
            const int e = base + lane;
            const int c = e < E ? max(s_off[e + 1] - s_off[e], 0) : 0;
            const int rest = c - big_rows(c, big);
            const int mine = (c > cmin && c <= cmax && rest > 0) ? (bm > 0 ? (rest - 1) / bm + 1 : 1) : 0;
            int v = mine;
            for (int d = 1; d < 64; d <<= 1) {
                const int u = __shfl_up(v, d, 64);
                if (lane >= d)
                    v += u;
            }
            if (e < E)
                s_first[e] = carry + v - mine;
            carry += __shfl(v, 63, 64);
        }
        if (lane == 0)
            s_first[E] = carry;
    }
    __syncthreads();
}

// The expert owning m-block `slot` (0 <= slot < s_first[E]): the last e with
// s_first[e] <= slot, which serves at least one m-block.  Sets its block
// index and row range.
__device__ __forceinline__ int grouped_slot(const int* s_off, const int* s_first, int E, int bm, int big,
                                            int slot, int* m0, int* hi)
{
    int lo = 0, up = E;
    while (up - lo > 1) {
        const int mid = (lo + up) >> 1;
        if (s_first[mid] <= slot)
            lo = mid;
        else
            up = mid;
    }
    const int c = max(s_off[lo + 1] - s_off[lo], 0);
    *m0 = s_off[lo] + big_rows(c, big) + (slot - s_first[lo]) * bm;
    *hi = s_off[lo] + c;
    return lo;
}

// The four-wave kernel's share of a grouped call, found without LDS (its
// stages fill all of it): every wave scans the offsets itself, 64 experts at
// a time.  An expert with c > cmin rows has big_count(c) blocks.
__device__ __forceinline__ int big_blocks(const int32_t* __restrict__ off, int e, int E, int R, int cmin, int* lo)
{
    if (e >= E) {
        *lo = 0;
        return 0;
    }
    const int a = clamp_off(off[e], R);
    const int c = max(clamp_off(off[e + 1], R) - a, 0);
    *lo = a;
    return c > cmin ? big_count(c) : 0;
}

__device__ int big_total(const int32_t* __restrict__ off, int E, int R, int cmin)
{
    const int lane = threadIdx.x & 63;
    int total = 0;
    for (int base = 0; base < E; base += 64) {
        int lo;
        int v = big_blocks(off, base + lane, E, R, cmin, &lo);
        for (int d = 32; d > 0; d >>= 1)
            v += __shfl_xor(v, d, 64);
        total += v;
    }
    return __builtin_amdgcn_readfirstlane(total);
}

// Expert, first row and row end of 256-row block `slot` (0 <= slot <
// big_total): the blocks are numbered expert by expert, in order.
__device__ int big_slot(const int32_t* __restrict__ off, int E, int R, int cmin, int slot, int* m0, int* hi)
{
    const int lane = threadIdx.x & 63;
    int carry = 0;
    for (int base = 0; base < E; base += 64) {
        int lo;
        const int nb = big_blocks(off, base + lane, E, R, cmin, &lo);
        int v = nb;
        for (int d = 1; d < 64; d <<= 1) {
            const int u = __shfl_up(v, d, 64);
            if (lane >= d)
                v += u;
        }
        const int chunk = __builtin_amdgcn_readfirstlane(__shfl(v, 63, 64));
        if (slot < carry + chunk) {
            const uint64_t hit = __ballot(carry + v > slot);
            const int L = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)hit) - 1);
            const int first = carry + __shfl(v - nb, L, 64);
            const int a = __shfl(lo, L, 64);
            const int e = base + L;
            const int c = max(clamp_off(off[e + 1], R) - a, 0);
            *m0 = __builtin_amdgcn_readfirstlane(a + (slot - first) * 256);
            *hi = __builtin_amdgcn_readfirstlane(a + c);
            return __builtin_amdgcn_readfirstlane(e);
        }
        carry += chunk;
    }
    *m0 = 0;
    *hi = 0;
    return 0;
}

// ---------------------------------------------------------------------------
// Tiled kernel (mid and large M)
// ---------------------------------------------------------------------------
// BM rows of x by BN rows of W per block, WM x WN waves, BK values of k per
// LDS stage, NS stages in flight.
template <int BM, int BN, int WM, int WN, int BK, int NS>
struct TiledCfg {
    static constexpr int kWaves = WM * WN;
    static constexpr int kThreads = kWaves * 64;
    static constexpr int TM = BM / WM;  // rows of x per wave
    static constexpr int TN = BN / WN;  // rows of W per wave
    static constexpr int FM = TM / 16;
    static constexpr int FN = TN / 16;
    static constexpr int kCh = BK / 8;  // 16-byte chunks per row per stage
    static constexpr int kStageUnits = (BM + BN) * kCh;  // W rows first, then x rows
    static constexpr int kInstr = kStageUnits / (64 * kWaves);  // loads per wave per stage
    static constexpr int kLdsBytes = NS * kStageUnits * 16;
    static constexpr int kSteps = BK / 32;
    static_assert(BK == kSlab, "a stage is one slab of the packed W: two MFMA k-steps");
    static_assert(NS >= 2, "at least double buffering");
    static_assert(kStageUnits % (64 * kWaves) == 0, "a stage must split evenly over the waves");
    static_assert((BN * kCh) % 64 == 0, "one load instruction must not straddle W and x");
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tiles are whole MFMA tiles");
    static_assert(kInstr * NS < 64, "loads in flight must fit vmcnt");
    static_assert(kLdsBytes <= 160 * 1024, "LDS");
};

// One BM x BN output block: rows m0 .. m0+BM-1 of x/y (rows at or past
// row_hi read as zeros and are never stored), columns n0 .. n0+BN-1 of y
// (rows of Wb past N likewise).  Wb is the packed W (slab-major).
// With kIdx, row i of the logical x is row xidx[i] of the stored x (xn rows;
// an index outside 0..xn-1 is clamped into it): the MoE layer's gather of
// token rows into expert order, done by the loads themselves.
//
// With kNorm, x holds raw rows and the block multiplies the RMSNorm of them:
// before any fragment read of a stage, its x tile is rewritten in LDS as
// bf16((x * r) * g) (bi::rms_scale_chunk, the standalone RMSNorm's rounding),
// r = rstd[row] and g the gain of the stage's k range.  Each thread rewrites
// one row's chunks, the same logical chunks in every wave, so the gain
// arrives through scalar loads.
// kNtW: the W loads are non-temporal (a call whose W strips are each read by
// one block: a single m-block).
template <int BM, int BN, int WM, int WN, int BK, int NS, bool kIdx = false, bool kNorm = false, bool kNtW = false>
__device__ __forceinline__ void tiled_block(uint4* lds, const uint16_t* __restrict__ x,
                                            const uint16_t* __restrict__ Wb,
                                            float* __restrict__ y, int m0, int row_hi, int n0,
                                            int N, int K, Split sp,
                                            const int32_t* __restrict__ xidx = nullptr, int xn = 0,
                                            const float* __restrict__ rstd = nullptr,
                                            const uint4* __restrict__ gain = nullptr)
{
    using C = TiledCfg<BM, BN, WM, WN, BK, NS>;
    constexpr int kCh = C::kCh;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave % WM;
    const int wn = wave / WM;
    static_assert(!kNorm || (C::kThreads % BM == 0 && (8 * BM) % C::kThreads == 0), "normalising split");
    static_assert(!kNorm || NS >= 3, "the norm rewrites a stage two ahead of the one being read");
    constexpr int kNC = kNorm ? 8 * BM / C::kThreads : 0;  // chunks of a row per thread
    const int nrow = threadIdx.x % BM;
    const int nc0 = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / BM) * kNC);
    const uint32_t rowb = (uint32_t)K * 2;

    const int wrows = min(BN, N - n0);
    const int xrows = min(BM, row_hi - m0);
    const __amdgpu_buffer_rsrc_t rW = make_rsrc(Wb + (size_t)n0 * kSlab, wpk_bytes(N, K, wrows));
    const __amdgpu_buffer_rsrc_t rX =
        kIdx ? make_rsrc(x, (uint32_t)xn * rowb) : make_rsrc(x + (size_t)m0 * K, (uint32_t)xrows * rowb);

    // Byte offset of each of this lane's loads within a stage's rows.  Unit
    // u of the stage (lane-linear in LDS) holds logical chunk swz(r, u % kCh)
    // of row r; rows past the valid range get an offset past the end of
    // their buffer (zeros, no memory access).  W rows of a stage are 128
    // bytes apart (one slab), x rows 2K bytes.
    uint32_t voff[C::kInstr];
#pragma unroll
    for (int j = 0; j < C::kInstr; ++j) {
        const int u = (wave * C::kInstr + j) * 64 + lane;
        if (u < BN * kCh) {
            const int r = u / kCh;
            voff[j] = r < wrows ? wpk_row(r, swz<kCh>(r, u % kCh)) : wpk_bytes(N, K, wrows);
        } else {
            const int uu = u - BN * kCh;
            const int r = uu / kCh;
            uint32_t row = (uint32_t)min(r, xrows - 1);
            if constexpr (kIdx) {
                const int t = xidx[m0 + (int)row];
                row = (uint32_t)(t < 0 ? 0 : (t >= xn ? xn - 1 : t));
            }
            voff[j] = r < xrows ? row * rowb + swz<kCh>(r, uu % kCh) * 16 : (uint32_t)(kIdx ? xn : xrows) * rowb;
        }
    }
    auto issue = [&](int s, int buf) {
#pragma unroll
        for (int j = 0; j < C::kInstr; ++j) {
            const int u0 = (wave * C::kInstr + j) * 64;
            const int k = sp.k0 + s * BK;
            if (u0 < BN * kCh)
                dma16<kNtW ? kCachePolicyNT : 0>(rW, voff[j], wpk_slab(k, N), lds + buf * C::kStageUnits + u0);
            else
                dma16(rX, voff[j], (uint32_t)k * 2, lds + buf * C::kStageUnits + u0);
        }
    };

    f32x4 acc[C::FN][C::FM];
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < C::FM; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Fragments of one MFMA k-step, double buffered in registers: the reads
    // for step g+1 are issued between the two halves of step g's MFMAs.
    using FragA = uint4[C::FN];
    using FragB = uint4[C::FM];
    FragA fa0, fa1;
    FragB fb0, fb1;
    auto read_frags = [&](int s, int ks, FragA& fa, FragB& fb) {
        const uint4* sW = lds + (s % NS) * C::kStageUnits;
        const uint4* sX = sW + BN * kCh;
        const int cl = ks * 4 + (lane >> 4);
#pragma unroll
        for (int t = 0; t < C::FN; ++t) {
            const int r = wn * C::TN + t * 16 + (lane & 15);
            fa[t] = sW[r * kCh + swz<kCh>(r, cl)];
        }
#pragma unroll
        for (int t = 0; t < C::FM; ++t) {
            const int r = wm * C::TM + t * 16 + (lane & 15);
            fb[t] = sX[r * kCh + swz<kCh>(r, cl)];
        }
    };
    // MFMAs of W-fragment rows [i0, i1) of one k-step; every accumulator
    // takes its k-steps in ascending order.
    auto mfmas = [&](const FragA& fa, const FragB& fb, int i0, int i1) {
#pragma unroll
        for (int i = 0; i < C::FN; ++i)
#pragma unroll
            for (int j = 0; j < C::FM; ++j)
                if (i >= i0 && i < i1)
                    acc[i][j] = mfma_step(fa[i], fb[j], acc[i][j]);
    };
    constexpr int kHalf = C::FN / 2 > 0 ? C::FN / 2 : 1;

    const int nk = sp.klen / BK;
    float nr = 0.f;
    if constexpr (kNorm)
        nr = rstd[m0 + min(nrow, xrows - 1)];
    // the x tile of stage s in place, as the model's normalised rows
    auto normalize = [&](int s) {
        if constexpr (kNorm) {
            uint4* sX = lds + (s % NS) * C::kStageUnits + BN * kCh;
            const uint4* g = gain + (sp.k0 + s * BK) / 8;
#pragma unroll
            for (int c = 0; c < kNC; ++c) {
                const int cc = nc0 + c;
                uint4* q = sX + nrow * kCh + swz<kCh>(nrow, cc);
                *q = bi::rms_scale_chunk(*q, nr, g[cc]);
            }
        }
    };
    // Stage s lives in buffer s % NS.  All NS buffers are filled up front;
    // stage s + NS is issued once every wave has read stage s.  With kNorm
    // the x tile of stage s + 2 is rewritten while stage s + 1 is read, so
    // its latency stays off the path from the barrier to the MFMAs: the
    // barrier after stage s then also waits for stage s + 2 to land.
#pragma unroll
    for (int q = 0; q < NS; ++q)
        issue(min(q, nk - 1), q);
    if constexpr (kNorm) {
        wait_vmcnt<C::kInstr * (NS - 2)>();  // stages 0 and 1 have landed
        barrier_after_lds_reads();
        normalize(0);
        if (nk > 1)
            normalize(1);
        barrier_after_lds_reads();  // stages 0 and 1 rewritten by every wave
    } else {
        wait_vmcnt<C::kInstr * (NS - 1)>();  // stage 0 has landed
        barrier_after_lds_reads();
    }
    read_frags(0, 0, fa0, fb0);

    // k-step ks of stage s, which has a successor step; branch free so the
    // scheduler can interleave its loads, fragment reads and MFMAs.  After a
    // stage's last step the next step is in stage s+1: wait until it has
    // landed and every wave has read stage s, then refill stage s's buffer
    // with stage s+NS.  Past the last stage the last one is loaded again
    // into a buffer that is never read, which keeps the count of loads in
    // flight the same at every stage: after stage s+1, NS-2 are outstanding.
    auto step = [&](int s, auto ksc, const FragA& fa, const FragB& fb, FragA& na, FragB& nb) {
        constexpr int ks = decltype(ksc)::value;
        mfmas(fa, fb, 0, kHalf);
        if constexpr (ks + 1 == C::kSteps) {
            if constexpr (kNorm)
                wait_vmcnt<C::kInstr * (NS - 3)>();  // this wave's loads of stage s+2 have landed
            else
                wait_vmcnt<C::kInstr * (NS - 2)>();  // this wave's loads of stage s+1 have landed
            barrier_after_lds_reads();           // every wave's have; all have read stage s
            issue(min(s + NS, nk - 1), s % NS);
            read_frags(s + 1, 0, na, nb);
            if constexpr (kNorm) {
                // stage s+2 is read after the next barrier, which orders these writes
                if (s + 2 < nk)
                    normalize(s + 2);
            }
        } else {
            read_frags(s, ks + 1, na, nb);
        }
        mfmas(fa, fb, kHalf, C::FN);
    };
    using K0 = std::integral_constant<int, 0>;
    using K1 = std::integral_constant<int, 1>;
    int s = 0;
    if constexpr (C::kSteps == 2) {
        // one stage per iteration: step 0 from fa0 into fa1, step 1 back
        for (; s + 1 < nk; ++s) {
            step(s, K0{}, fa0, fb0, fa1, fb1);
            step(s, K1{}, fa1, fb1, fa0, fb0);
        }
        step(s, K0{}, fa0, fb0, fa1, fb1);
        mfmas(fa1, fb1, 0, C::FN);
    } else {
        // two stages per iteration, alternating fragment sets
        for (; s + 2 < nk; s += 2) {
            step(s, K0{}, fa0, fb0, fa1, fb1);
            step(s + 1, K0{}, fa1, fb1, fa0, fb0);
        }
        if (s + 1 < nk) {
            step(s, K0{}, fa0, fb0, fa1, fb1);
            mfmas(fa1, fb1, 0, C::FN);
        } else {
            mfmas(fa0, fb0, 0, C::FN);
        }
    }
    wait_vmcnt<0>();  // no load into LDS may outlive the block

#pragma unroll
    for (int j = 0; j < C::FM; ++j) {
        const int m = m0 + wm * C::TM + j * 16 + (lane & 15);
        if (m >= row_hi)
            continue;
#pragma unroll
        for (int i = 0; i < C::FN; ++i) {
            const int n = n0 + wn * C::TN + i * 16 + 4 * (lane >> 4);
            if (n < N)
                emit4(y + (size_t)m * N + n, acc[i][j], sp.fold);
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

// Block -> tile for the four-wave kernels: the tile grid is cut into 8
// rectangles, MR along m by 8 / MR along n, and XCD x (which hardware hands
// block b when b % 8 == x) takes rectangle (x % MR, x / MR), walking groups
// of 4 of its m-blocks column by column.  With MR = 4, each half of the W
// columns is read by one set of four XCDs (x / 4), and the four XCDs of a
// set share those W tiles while each keeps its own x rows; with the order of
// tile_of_block every XCD reads the same W half at once (measured on the
// down-proj: about 3% faster at M = 4096 and 8192).  What an XCD's L2 fetches
// in a round is the x and W panels its rectangle's blocks touch: with 32
// blocks per XCD, 4 x panels and 8 W panels for MR = 4, 8 and 4 for MR = 2.
// With 256-row blocks both come to 12 panels of the same size; with 128-row
// blocks an x panel is half a W panel, and MR = 2 fetches 20% fewer bytes.
// Grids that do not cut evenly use tile_of_block.
template <int MR>
__device__ __forceinline__ void tile_of_block_rect(int b, int nblocks, int tiles_m, int tiles_n, int* tm, int* tn)
{
    constexpr int NR = 8 / MR;
    if (tiles_m % MR != 0 || tiles_n % NR != 0 || nblocks != tiles_m * tiles_n) {
        tile_of_block(b, nblocks, tiles_m, tiles_n, 4, tm, tn);
        return;
    }
    const int xcd = b % 8, i = b / 8;
    const int rm = tiles_m / MR, rn = tiles_n / NR;
    const int gm = rm < 4 ? rm : 4;  // rm is a multiple of gm: 1, 2, 3 or a multiple of 4 ...
    const int rows = rm % gm == 0 ? gm : 1;  // ... else walk one m-block at a time
    const int span = rows * rn, g = i / span, r = i % span;
    *tm = (xcd % MR) * rm + g * rows + r % rows;
    *tn = (xcd / MR) * rn + r / rows;
}

// Rectangles along m for the four-wave kernel with XT x tiles per wave
// (blocks of 32 XT rows): 2 when a block's x panel is smaller than its W
// panel, else 4.  At M = 2048 on the down-proj (128x256 blocks) the panel
// count gives 470 MB of L2 fills per launch with MR = 2 against 587 MB (as
// counted) with MR = 4; the call timed 197.9-199.2 us against 199.2-201.9,
// interleaved on one box: each CU's load path, not the fabric, bounds it.
template <int XT>
constexpr int rect_m() { return XT < 8 ? 2 : 4; }

template <int BM, int BN, int WM, int WN, int BK, int NS, int kMode = kPlain>
__global__ void __launch_bounds__(WM * WN * 64)
    bigemm_tiled(const uint16_t* __restrict__ x, const uint16_t* __restrict__ W,
                 float* __restrict__ y, int M, int N, int K, Split sp, int tiles_m, int tiles_n,
                 int group_m, float* part, const float* __restrict__ rstd, const uint4* __restrict__ gain)
{
    using C = TiledCfg<BM, BN, WM, WN, BK, NS>;
    __shared__ uint4 lds[NS * C::kStageUnits];
    y = cmp_split<kMode>(sp, y, part, M, N);
    int tm, tn;
    tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, &tm, &tn);
    tiled_block<BM, BN, WM, WN, BK, NS, false, kMode == kNormX, kMode == kStreamOnce>(lds, x, W, y, tm * BM, M,
                                                                                     tn * BN, N, K, sp, nullptr, 0,
                                                                                     rstd, gain);
}

// ---------------------------------------------------------------------------
// Four-wave 256x256 block (large M)
// ---------------------------------------------------------------------------
// Same tree as tiled_block, 256x256 output blocks, but four waves of 128x128
// each instead of eight of 128x64: a CU reads each stage from LDS 8 times
// instead of 12 and half as many waves meet at each barrier.  A wave's 64
// accumulator tiles (256 values per lane) live in the accumulation registers
// a0..a255, which the MFMAs read and write directly.  They are written only
// by the inline-asm MFMAs below and read only by the epilogue; the compiler
// never allocates them, because the kernel keeps its own registers below 256
// and never spills (a CPU test checks the built code for exactly this).  The
// compiler still places the fragment reads and loads, which sit between the
// MFMA statements in source order, and inserts the waits for the fragments
// each MFMA reads.
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Declares a0..a255 used, so that the kernel descriptor reserves them.
#define BIG_AGPRS10(p) "a" #p "0", "a" #p "1", "a" #p "2", "a" #p "3", "a" #p "4", "a" #p "5", "a" #p "6", \
    "a" #p "7", "a" #p "8", "a" #p "9"
__device__ __forceinline__ void claim_agprs()
{
    asm volatile("" ::: "a0", "a1", "a2", "a3", "a4", "a5", "a6", "a7", "a8", "a9", BIG_AGPRS10(1),
                 BIG_AGPRS10(2), BIG_AGPRS10(3), BIG_AGPRS10(4), BIG_AGPRS10(5), BIG_AGPRS10(6),
                 BIG_AGPRS10(7), BIG_AGPRS10(8), BIG_AGPRS10(9), BIG_AGPRS10(10), BIG_AGPRS10(11),
                 BIG_AGPRS10(12), BIG_AGPRS10(13), BIG_AGPRS10(14), BIG_AGPRS10(15), BIG_AGPRS10(16),
                 BIG_AGPRS10(17), BIG_AGPRS10(18), BIG_AGPRS10(19), BIG_AGPRS10(20), BIG_AGPRS10(21),
                 BIG_AGPRS10(22), BIG_AGPRS10(23), BIG_AGPRS10(24), "a250", "a251", "a252", "a253",
                 "a254", "a255");
}
#undef BIG_AGPRS10

// Accumulator tile T is a[4T .. 4T+3].  kZero starts the chain from +0 (the
// inline constant), as the first k-step of every split does.
template <int T, bool kZero>
__device__ __forceinline__ void mfma_agpr(const uint4& a, const uint4& b)
{
    if constexpr (kZero)
        asm volatile("v_mfma_f32_16x16x32_bf16 a[%c2:%c3], %0, %1, 0" ::"v"(__builtin_bit_cast(i32x4, a)),
                     "v"(__builtin_bit_cast(i32x4, b)), "n"(4 * T), "n"(4 * T + 3));
    else
        asm volatile("v_mfma_f32_16x16x32_bf16 a[%c2:%c3], %0, %1, a[%c2:%c3]" ::"v"(__builtin_bit_cast(i32x4, a)),
                     "v"(__builtin_bit_cast(i32x4, b)), "n"(4 * T), "n"(4 * T + 3));
}

template <int T>
__device__ __forceinline__ f32x4 read_agpr_tile()
{
    f32x4 v;
    asm volatile("v_accvgpr_read_b32 %0, a%c4\n\t"
                 "v_accvgpr_read_b32 %1, a%c5\n\t"
                 "v_accvgpr_read_b32 %2, a%c6\n\t"
                 "v_accvgpr_read_b32 %3, a%c7"
                 : "=v"(v[0]), "=v"(v[1]), "=v"(v[2]), "=v"(v[3])
                 : "n"(4 * T), "n"(4 * T + 1), "n"(4 * T + 2), "n"(4 * T + 3));
    return v;
}

// f(integral_constant<int, T>) for T = 0 .. n-1, in order, unrolled.
template <typename F, int... T>
__device__ __forceinline__ void for_each_t(F&& f, std::integer_sequence<int, T...>)
{
    (f(std::integral_constant<int, T>{}), ...);
}

// LDS: W triple-buffered (3 x 32 KB) and x double-buffered (2 x 32 KB at
// 256 x rows), 160 KB.  A stage is 64 values of k (two MFMA k-steps, full
// 128-byte row segments).  Stage t's W is loaded during k-step 0 of stage t-2
// and its x during k-step 1 of stage t-2, the loads spread over each k-step's
// MFMAs: loads issued in bursts stall the issuing wave (a CU accepts one
// 1 KB load about every 16 cycles) and, with one wave per SIMD, the MFMA
// pipe with it.
//
// XT: x tiles per wave.  XT = 8 is the 256x256 block; XT = 4 the same block
// over 128 x rows (each wave 64 x rows by 128 W rows, 128 accumulation
// registers), for M too small to give every CU a 256-row block.

// The fragment read q (0 .. 7+XT) of the next k-step issued after MFMA T of
// a k-step's 8 XT: spread evenly, in the order the MFMAs consume them.
template <int XT>
constexpr int tiled4_read_at(int T)
{
    for (int q = 0; q < 8 + XT; ++q)
        if (((q + 1) * 8 * XT) / (8 + XT) - 1 == T)
            return q;
    return -1;
}

// kSwiGLU: W is a gated projection packed with the gate/up row interleave
// (bigemm_pack_w), so W tiles 2t and 2t+1 of a wave hold 16 gate columns and
// their up columns; the epilogue writes bf16 SwiGLU of each pair, a
// [rows, N / 2] bf16 at y, instead of the fp32 product.
template <int XT, bool kIdx = false, bool kSwiGLU = false, bool kNtW = false>
__device__ __forceinline__ void tiled4_block(uint4* lds, const uint16_t* __restrict__ x,
                                              const uint16_t* __restrict__ Wb, float* __restrict__ y, int m0,
                                              int row_hi, int n0, int N, int K, Split sp,
                                              const int32_t* __restrict__ xidx = nullptr, int xn = 0)
{
    static_assert(XT >= 4 && XT <= 8, "x tiles per wave");
    constexpr int BM = 32 * XT, BN = 256, BK = 64, kCh = BK / 8;
    constexpr int kPart = 256 * kCh;      // units (16 B) of one 256-row W part of a stage: 32 KB
    constexpr int kXPart = BM * kCh;      // units of one stage's x rows
    constexpr int kXBase = 3 * kPart;     // x buffers follow the three W buffers
    constexpr int kT = 8 * XT;            // MFMAs per k-step
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave & 1;
    const int wn = wave >> 1;
    const uint32_t rowb = (uint32_t)K * 2;

    const int wrows = min(BN, N - n0);
    const int xrows = min(BM, row_hi - m0);
    const sgpr4 aW = rsrc_words(Wb + (size_t)n0 * kSlab, wpk_bytes(N, K, wrows));
    const sgpr4 aX = kIdx ? rsrc_words(x, (uint32_t)xn * rowb) : rsrc_words(x + (size_t)m0 * K, (uint32_t)xrows * rowb);

    // load j < 8: W unit (8 wave + j) 64 + lane; j >= 8: x unit
    // (XT wave + j - 8) 64 + lane
    uint32_t voff[8 + XT];
#pragma unroll
    for (int j = 0; j < 8 + XT; ++j) {
        const int u = (j < 8 ? wave * 8 + j : wave * XT + j - 8) * 64 + lane;
        const int r = u / kCh;
        const int c = swz<kCh>(r, u % kCh);
        if (j < 8) {
            voff[j] = r < wrows ? wpk_row(r, c) : wpk_bytes(N, K, wrows);
        } else {
            uint32_t row = (uint32_t)min(r, xrows - 1);
            if constexpr (kIdx) {
                const int t = xidx[m0 + (int)row];
                row = (uint32_t)(t < 0 ? 0 : (t >= xn ? xn - 1 : t));
            }
            voff[j] = r < xrows ? row * rowb + c * 16 : (uint32_t)(kIdx ? xn : xrows) * rowb;
        }
    }
    auto issueW = [&](int j, int t, int wbuf) {
        dma16_asm<kNtW>(aW, voff[j], wpk_slab(sp.k0 + t * BK, N), lds + wbuf * kPart + (wave * 8 + j) * 64);
    };
    auto issueX = [&](int j, int t, int xbuf) {
        dma16_asm(aX, voff[8 + j], (uint32_t)(sp.k0 + t * BK) * 2, lds + kXBase + xbuf * kXPart + (wave * XT + j) * 64);
    };
    // fragment q of k-step ks of the stage in W buffer wbuf and x buffer
    // xbuf: q = 0 is W tile 0, 1..XT are x tiles 0..XT-1, the rest W tiles 1..7
    auto read1 = [&](int q, int wbuf, int xbuf, int ks, uint4* fa, uint4* fb) {
        const int cl = ks * 4 + (lane >> 4);
        if (q >= 1 && q <= XT) {
            const int r = wm * 16 * XT + (q - 1) * 16 + (lane & 15);
            fb[q - 1] = lds[kXBase + xbuf * kXPart + r * kCh + swz<kCh>(r, cl)];
        } else {
            const int tt = q == 0 ? 0 : q - XT;
            const int r = wn * 128 + tt * 16 + (lane & 15);
            fa[tt] = lds[wbuf * kPart + r * kCh + swz<kCh>(r, cl)];
        }
    };

    uint4 fa0[8], fb0[XT], fa1[8], fb1[XT];
    const int nk = sp.klen / BK;

    // Step 0 of stage t: MFMAs of k-step 0, the fragments of k-step 1, and
    // W of stage t+2 into W buffer (t+2) % 3 (freed by the barrier of
    // stage t-1).  Step 1: after two MFMAs, wait for stage t+1 (all but the
    // 8 W loads just issued) and the barrier (every wave has read stage t);
    // then the fragments of stage t+1's k-step 0 and x of stage t+2 into x
    // buffer t % 2.  Loads past the last stage repeat the last one into a
    // buffer that is not read again.
    auto step0 = [&](auto zero, int t, int wb, int xb) {
        constexpr bool kZ = decltype(zero)::value;
        const int tl = min(t + 2, nk - 1);
        const int wl = wb == 0 ? 2 : wb - 1;  // (t + 2) % 3
        for_each_t([&](auto tc) {
            constexpr int T = decltype(tc)::value;
            mfma_agpr<T, kZ>(fa0[T / XT], fb0[T % XT]);
            if constexpr (tiled4_read_at<XT>(T) >= 0)
                read1(tiled4_read_at<XT>(T), wb, xb, 1, fa1, fb1);
            if constexpr (T % XT == (5 * XT) / 8)  // one W load per XT MFMAs
                issueW(T / XT, tl, wl);
        }, std::make_integer_sequence<int, kT>{});
    };
    auto step1 = [&](int t, int wb, int xb) {
        const int tl = min(t + 2, nk - 1);
        const int wn1 = wb == 2 ? 0 : wb + 1;  // (t + 1) % 3
        for_each_t([&](auto tc) {
            constexpr int T = decltype(tc)::value;
            mfma_agpr<T, false>(fa1[T / XT], fb1[T % XT]);
            if constexpr (T == 1) {
                wait_vmcnt<8>();
                barrier_after_lds_reads();
            }
            if constexpr (T >= 2 && T < 2 + 2 * (8 + XT) && T % 2 == 0)
                read1((T - 2) / 2, wn1, xb ^ 1, 0, fa0, fb0);
            if constexpr (T % 8 == 3 && T / 8 < XT)  // after MFMAs 3, 11, ...
                issueX(T / 8, tl, xb);
        }, std::make_integer_sequence<int, kT>{});
    };

    claim_agprs();
    const int t1 = min(1, nk - 1);
#pragma unroll
    for (int j = 0; j < 8; ++j)
        issueW(j, 0, 0);
#pragma unroll
    for (int j = 0; j < XT; ++j)
        issueX(j, 0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j)
        issueW(j, t1, 1);
#pragma unroll
    for (int j = 0; j < XT; ++j)
        issueX(j, t1, 1);
    wait_vmcnt<8 + XT>();  // stage 0 has landed
    barrier_after_lds_reads();
#pragma unroll
    for (int q = 0; q < 8 + XT; ++q)
        read1(q, 0, 0, 0, fa0, fb0);
    step0(std::true_type{}, 0, 0, 0);
    step1(0, 0, 0);
    int wb = 1;
    for (int t = 1; t < nk; ++t) {
        step0(std::false_type{}, t, wb, t & 1);
        step1(t, wb, t & 1);
        wb = wb == 2 ? 0 : wb + 1;
    }
    wait_vmcnt<0>();  // no load into LDS may outlive the block
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

    // x tile j outer, W tile i inner: the two 64-byte halves of a 128-byte
    // line of y (tiles i and i+1 of one row) are stored back to back
    if constexpr (kSwiGLU) {
        // tiles i (gate) and i+1 (up) of x tile j: 4 columns of a row per
        // lane, gate column c = (row of tile i) / 2 within the 32-row group
        const int half = N / 2;
        uint16_t* a = reinterpret_cast<uint16_t*>(y);
        for_each_t([&](auto uc) {
            constexpr int U = decltype(uc)::value;
            constexpr int j = U / 4, i = 2 * (U % 4);
            const int m = m0 + wm * 16 * XT + j * 16 + (lane & 15);
            const int c = (n0 + wn * 128 + i * 16) / 2 + 4 * (lane >> 4);
            const f32x4 g = read_agpr_tile<XT * i + j>();
            const f32x4 u = read_agpr_tile<XT * (i + 1) + j>();
            if (m < row_hi && c < half) {
                const float gg[4] = {g[0], g[1], g[2], g[3]};
                const float uu[4] = {u[0], u[1], u[2], u[3]};
                *reinterpret_cast<uint2*>(a + (size_t)m * half + c) = bi::swiglu4(gg, uu);
            }
        }, std::make_integer_sequence<int, kT / 2>{});
    } else {
        for_each_t([&](auto uc) {
            constexpr int U = decltype(uc)::value;
            constexpr int j = U / 8, i = U % 8, T = XT * i + j;
            const int m = m0 + wm * 16 * XT + j * 16 + (lane & 15);
            const int n = n0 + wn * 128 + i * 16 + 4 * (lane >> 4);
            const f32x4 v = read_agpr_tile<T>();
            if (m < row_hi && n < N)
                emit4(y + (size_t)m * N + n, v, sp.fold);
        }, std::make_integer_sequence<int, kT>{});
    }
}

// (32 XT) x 256 output blocks, one per workgroup.
template <int XT, int kMode = kPlain>
__global__ void __launch_bounds__(256)
    bigemm_tiled4(const uint16_t* __restrict__ x, const uint16_t* __restrict__ W, float* __restrict__ y, int M,
                   int N, int K, Split sp, int tiles_m, int tiles_n, int group_m, float* part)
{
    __shared__ uint4 lds[3 * 256 * 8 + 2 * 32 * XT * 8];
    y = cmp_split<kMode>(sp, y, part, M, N);
    int tm, tn;
    tile_of_block_rect<rect_m<XT>()>(blockIdx.x, gridDim.x, tiles_m, tiles_n, &tm, &tn);
    tiled4_block<XT>(lds, x, W, y, tm * 32 * XT, M, tn * 256, N, K, sp);
}

// Grouped, persistent: the row blocks (big_count) of the experts with more
// than cmin rows, by 256 W rows; a block of at most 128 rows runs as a
// 128x256 block.  The tiles are cut into 8 contiguous ranges, one per XCD,
// as in bigemm_tiled_grouped.  kIdx: x rows are read through xidx.
// kSwiGLU: a gated projection's SwiGLU, bf16 [R, N / 2] at y (tiled4_block).
template <bool kIdx, bool kSwiGLU = false, bool kNtW = false>
__global__ void __launch_bounds__(256)
    bigemm_tiled4_grouped(const uint16_t* __restrict__ x, const uint16_t* __restrict__ W, float* __restrict__ y,
                          const int32_t* __restrict__ off, int E, int R, int N, int K, Split sp, int tiles_n,
                          int cmin, const int32_t* __restrict__ xidx, int xn)
{
    __shared__ uint4 lds[5 * 256 * 8];
    const int total = big_total(off, E, R, cmin) * tiles_n;
    const int xcd = blockIdx.x % 8;
    const int per_xcd = gridDim.x / 8;
    const int t_end = (int)((long long)total * (xcd + 1) / 8);
    for (int t = (int)((long long)total * xcd / 8) + (int)(blockIdx.x / 8); t < t_end; t += per_xcd) {
        int m0, hi;
        const int e = big_slot(off, E, R, cmin, t / tiles_n, &m0, &hi);
        barrier_after_lds_reads();  // every wave is done with the previous tile's stages
        if (hi - m0 <= 128)
            tiled4_block<4, kIdx, kSwiGLU, kNtW>(lds, x, W + (size_t)e * N * K, y, m0, hi, (t % tiles_n) * 256, N, K,
                                                 sp, xidx, xn);
        else
            tiled4_block<8, kIdx, kSwiGLU, kNtW>(lds, x, W + (size_t)e * N * K, y, m0, hi, (t % tiles_n) * 256, N, K,
                                                 sp, xidx, xn);
    }
}

// Grouped, persistent: the output tiles (slot, tn) -- slot enumerating the
// m-blocks of the experts with more than cmin rows -- are counted on the
// device and cut into 8 contiguous ranges, one per XCD (hardware hands block b
// to XCD b % 8; the grid is a multiple of 8), so each XCD's L2 holds few
// experts at a time and every XCD gets the same share whatever the routing.
// kIdx: x rows are read through xidx.
template <int BM, int BN, int WM, int WN, int BK, int NS, bool kIdx>
__global__ void __launch_bounds__(WM * WN * 64)
    bigemm_tiled_grouped(const uint16_t* __restrict__ x, const uint16_t* __restrict__ W,
                         float* __restrict__ y, const int32_t* __restrict__ off, int E, int R,
                         int N, int K, Split sp, int tiles_n, int cmin, int big,
                         const int32_t* __restrict__ xidx, int xn)
{
    using C = TiledCfg<BM, BN, WM, WN, BK, NS>;
    __shared__ uint4 lds[NS * C::kStageUnits];
    __shared__ int s_off[kMaxExperts + 1];
    __shared__ int s_first[kMaxExperts + 1];
    grouped_plan(off, E, R, BM, cmin, 0x7fffffff, big, s_off, s_first);
    const int total = s_first[E] * tiles_n;
    const int xcd = blockIdx.x % 8;
    const int per_xcd = gridDim.x / 8;
    const int t_end = (int)((long long)total * (xcd + 1) / 8);
    for (int t = (int)((long long)total * xcd / 8) + (int)(blockIdx.x / 8); t < t_end; t += per_xcd) {
        int m0, hi;
        const int e = grouped_slot(s_off, s_first, E, BM, big, t / tiles_n, &m0, &hi);
        barrier_after_lds_reads();  // every wave is done with the previous tile's stages
        tiled_block<BM, BN, WM, WN, BK, NS, kIdx>(lds, x, W + (size_t)e * N * K, y, m0, hi, (t % tiles_n) * BN,
                                                  N, K, sp, xidx, xn);
    }
}

// ---------------------------------------------------------------------------
// Streaming kernel (small M)
// ---------------------------------------------------------------------------
// MB consumer waves (one 16-row m-tile each) share one strip of 16*NT
// columns of W; each consumer runs NT chains, one per 16-column tile.  A
// stage holds BKS values of k for the 16*NT W rows and the first XR rows of
// the m-block (XR = 16*MB, or fewer when the call has fewer rows: the
// consumer of a single m-tile then re-reads row XR-1 for its padding rows).
// NP producer waves split a stage's loads; NR stages live in an LDS ring.
// NT > 1 (mid M): a CU's bytes are (16 MB + 16 NT) rows over K per item, so
// a 64x64 item moves 128 rows where four 64x16 items move 320.
constexpr int kStreamLdsBudget = 144 * 1024;
constexpr int kStreamWInFlight = 32 * 1024;
// Producer waves per streaming workgroup: the WG has at most 8 waves (two
// per SIMD, so each may use 256 VGPRs); narrower stages have fewer loads and
// use fewer producers.
template <int MB, int BKS>
constexpr int stream_producers()
{
    return BKS >= 256 ? 8 - MB : (BKS == 128 ? (6 - MB > 2 ? 6 - MB : 2) : 2);
}

template <int MB, int XR, int BKS, int NP, int NT = 1>
struct StreamShape {
    static constexpr int kWRows = 16 * NT;   // W rows per stage
    static constexpr int kChunks = BKS / 8;  // 16-byte units per row per stage
    static constexpr int kStageUnits = (kWRows + XR) * kChunks;
    static constexpr int kT = kStageUnits / 64;  // load instructions per stage
    static constexpr int kHi = (kT + NP - 1) / NP;  // share of the first kT % NP producers
    static constexpr int kLo = kT / NP;             // share of the others
    static constexpr int kByLds = kStreamLdsBudget / (kStageUnits * 16);
    static constexpr int kByVmcnt = 63 / kHi + 1;
    // 512-wide stages: at most 32 KB of W in flight per workgroup (8 MB over
    // 256 CUs, about HBM's bandwidth-latency product).  Deeper rings queue
    // more requests at HBM and stream slower (M = 1 on a 117 MB weight:
    // 19.7 us with two stages in flight against 21.2 us with seven).  The
    // narrower stages keep their depth: the grouped kernel's short items
    // (K = 768: three stages an item) lose 3% when capped the same way.
    static constexpr int kByFlight = BKS >= 512 ? kStreamWInFlight / (kWRows * BKS * 2) + 1 : 16;
    static constexpr int kNR0 = kByLds < kByVmcnt ? kByLds : kByVmcnt;
    static constexpr int kNR1 = kNR0 < kByFlight ? kNR0 : kByFlight;
    static constexpr int kNR = kNR1 < 16 ? kNR1 : 16;
};

template <int MB, int XR, int BKS, int NP, int NT = 1>
struct StreamCfg {
    using S = StreamShape<MB, XR, BKS, NP, NT>;
    static constexpr int kWRows = S::kWRows;
    static constexpr int kConsumers = MB;
    static constexpr int kProducers = NP;
    static constexpr int kThreads = (MB + NP) * 64;
    static constexpr int kChunks = S::kChunks;
    static constexpr int kStageUnits = S::kStageUnits;
    static constexpr int kT = S::kT;
    static constexpr int kHi = S::kHi;
    static constexpr int kLo = S::kLo;
    static constexpr int NR = S::kNR;
    static constexpr int kSteps = BKS / 32;
    static constexpr int kLdsBytes = NR * kStageUnits * 16;
    static_assert(XR == 16 * MB || (MB == 1 && XR < 16), "x rows per stage");
    static_assert(kStageUnits % 64 == 0, "a stage is whole load instructions");
    static_assert((kWRows * kChunks) % 64 == 0, "one load must not straddle W and x");
    static_assert(NT == 1 || XR == 16 * MB, "wide strips take whole m-blocks");
    static_assert(kLo >= 1, "every producer loads something");
    static_assert(NR >= 3, "ring too shallow");
    static_assert(kHi * (NR - 1) < 64, "loads in flight must fit vmcnt");
    static_assert(kLdsBytes <= kStreamLdsBudget, "LDS");
};

// Where work item `item` lives: rows m0 .. row_hi-1 of x/y, W rows
// n0 .. n0+16NT-1 of the expert weight Wb.
struct StreamItem {
    int m0, row_hi, n0;
    const uint16_t* Wb;
};

// kNtW: W loads are non-temporal (for calls that read every W line once).
// kSwiGLU (NT = 2, one split): W is a gated projection packed with the
// gate/up row interleave (bigemm_pack_w), so a 32-row strip holds 16 gate
// columns and their 16 up columns; the epilogue writes bf16 SwiGLU of each
// pair, a [rows, N / 2] bf16 at y, instead of the fp32 product.
template <int MB, int XR, int BKS, int NP, bool kIdx = false, int NT = 1, bool kNtW = false, bool kSwiGLU = false>
__device__ __forceinline__ void stream_body(uint4* ring, const uint16_t* __restrict__ x,
                                            const uint16_t* __restrict__ W, float* __restrict__ y,
                                            int N, int K, Split sp, int tiles_n, int nitems,
                                            // dense: M rows; grouped: clamped offsets and
                                            // the expert list, both in LDS
                                            int M, const int* sh_off, const int* elist,
                                            // grouped, kIdx: row indices into x (xn rows)
                                            const int32_t* __restrict__ xidx = nullptr, int xn = 0)
{
    using C = StreamCfg<MB, XR, BKS, NP, NT>;
    constexpr int kCh = C::kChunks;
    constexpr int NR = C::NR;
    constexpr int kWR = C::kWRows;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = gridDim.x;
    const int mine = nitems > (int)blockIdx.x ? (nitems - 1 - (int)blockIdx.x) / G + 1 : 0;
    const int nst = sp.klen / BKS;
    const int total = mine * nst;

    auto item_at = [&](int it) {
        const int item = blockIdx.x + it * G;
        const int mb = item / tiles_n;
        StreamItem s;
        s.n0 = (item % tiles_n) * kWR;
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
        // ---- producers: keep NR-1 stages of W and x in flight ----
        const int pw = wave - MB;
        auto produce = [&](auto count_tag, int first) {
            constexpr int kI = decltype(count_tag)::value;
            const uint32_t rowb = (uint32_t)K * 2;
            __amdgpu_buffer_rsrc_t rW = make_rsrc(W, 16), rX = make_rsrc(x, 16);
            uint32_t voff[kI];
            int cur_it = -1, k_stage = nst;
            // indexed x rows: each item's row indices are loaded while the
            // item before it streams (pend), not when the item starts
            int pend[kI];
            auto load_idx = [&](int it) {
                if (!kIdx || it >= mine)
                    return;
                const StreamItem s = item_at(it);
                const int xrows = min(XR, s.row_hi - s.m0);
#pragma unroll
                for (int j = 0; j < kI; ++j) {
                    const int r = ((first + j) * 64 + lane) / kCh;
                    pend[j] = r >= kWR ? xidx[s.m0 + min(r - kWR, xrows - 1)] : 0;
                }
            };
            if constexpr (kIdx)
                load_idx(0);
            // stages are issued in order q = 0, 1, 2, ...: nst stages per item
            auto issue = [&](int q) {
                if (k_stage == nst) {  // entering the next item: its rows, once
                    ++cur_it;
                    k_stage = 0;
                    const StreamItem s = item_at(cur_it);
                    const int xrows = min(XR, s.row_hi - s.m0);
                    // W rows past N (a strip wider than what is left) load
                    // nothing: their offsets aim past the end of the buffer
                    const int wrows = min(kWR, N - s.n0);
                    rW = make_rsrc(s.Wb + (size_t)s.n0 * kSlab, wpk_bytes(N, K, wrows));
                    rX = kIdx ? make_rsrc(x, (uint32_t)xn * rowb)
                              : make_rsrc(x + (size_t)s.m0 * K, (uint32_t)xrows * rowb);
#pragma unroll
                    for (int j = 0; j < kI; ++j) {
                        const int u = (first + j) * 64 + lane;
                        const int r = u / kCh;
                        const int c = swz<kCh>(r, u % kCh);
                        uint32_t row = r < kWR ? (uint32_t)r : (uint32_t)min(r - kWR, xrows - 1);
                        if constexpr (kIdx) {
                            if (r >= kWR) {
                                const int t = pend[j];
                                row = (uint32_t)(t < 0 ? 0 : (t >= xn ? xn - 1 : t));
                            }
                        }
                        // W: chunk c of the stage is chunk c % 8 of its slab c / 8
                        voff[j] = r < kWR ? (r < wrows ? wpk_slab(kSlab * (c / 8), N) + wpk_row(r, c % 8)
                                                       : wpk_bytes(N, K, wrows))
                                          : (r - kWR < xrows ? row * rowb + c * 16
                                                             : (uint32_t)(kIdx ? xn : xrows) * rowb);
                    }
                    if constexpr (kIdx)
                        load_idx(cur_it + 1);
                }
                uint4* dst = ring + (q % NR) * C::kStageUnits;
#pragma unroll
                for (int j = 0; j < kI; ++j) {
                    const int u0 = (first + j) * 64;
                    const int k = sp.k0 + k_stage * BKS;
                    if (u0 < kWR * kCh)
                        dma16<kNtW ? kCachePolicyNT : 0>(rW, voff[j], wpk_slab(k, N), dst + u0);
                    else
                        dma16(rX, voff[j], (uint32_t)k * 2, dst + u0);
                }
                ++k_stage;
            };
            const int pro = total < NR - 1 ? total : NR - 1;
            for (int q = 0; q < pro; ++q)
                issue(q);
            for (int q = 0; q < total; ++q) {
                if (q + NR - 2 < total)
                    wait_vmcnt<kI * (NR - 2)>();
                else
                    wait_vmcnt<0>();
                barrier_after_lds_reads();  // stage q is in LDS; slot (q-1) % NR is free
                if (q + NR - 1 < total)
                    issue(q + NR - 1);
            }
        };
        constexpr int kExtra = C::kT % NP;  // producers that take kHi loads
        if (pw < kExtra)
            produce(std::integral_constant<int, C::kHi>{}, pw * C::kHi);
        else
            produce(std::integral_constant<int, C::kLo>{}, kExtra * C::kHi + (pw - kExtra) * C::kLo);
    } else {
        // ---- consumer: the MFMA chain of m-tile `wave`.  Fragments are
        // double-buffered by half stage: the reads of the next half overlap
        // the chain of the current one, and the next stage's first half is
        // read once the barrier says it has landed.
        const int ci = wave;
        const int rw = lane & 15;
        const int rx = kWR + (MB == 1 ? min(rw, XR - 1) : 16 * ci + rw);
        constexpr int kH = C::kSteps / 2;  // k-steps per half stage
        uint4 a0[kH * NT], b0[kH], a1[kH * NT], b1[kH];
        auto read = [&](int q, int h, uint4* a, uint4* b) {
            const uint4* st = ring + (q % NR) * C::kStageUnits;
#pragma unroll
            for (int t = 0; t < kH; ++t) {
                const int cl = 4 * (h * kH + t) + (lane >> 4);
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const int r = 16 * j + rw;
                    a[t * NT + j] = st[r * kCh + swz<kCh>(r, cl)];
                }
                b[t] = st[rx * kCh + swz<kCh>(rx, cl)];
            }
        };
        // the NT chains of a k-step side by side; each chain in ascending k
        auto chain = [&](f32x4* acc, const uint4* a, const uint4* b) {
#pragma unroll
            for (int t = 0; t < kH; ++t)
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    acc[j] = mfma_step(a[t * NT + j], b[t], acc[j]);
        };
        f32x4 acc[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j)
            acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (total > 0) {
            barrier_after_lds_reads();
            read(0, 0, a0, b0);
        }
        for (int q = 0; q < total; ++q) {
            read(q, 1, a1, b1);
            chain(acc, a0, b0);
            if (q + 1 < total) {
                barrier_after_lds_reads();  // stage q+1 has landed; stage q is read
                read(q + 1, 0, a0, b0);
            }
            chain(acc, a1, b1);
            if ((q + 1) % nst == 0) {
                const StreamItem s = item_at(q / nst);
                const int m = s.m0 + 16 * ci + rw;
                if constexpr (kSwiGLU) {
                    static_assert(NT == 2, "a gate tile and its up tile");
                    // gate columns n0/2 .. n0/2+15 of the strip; 4 per lane
                    if (m < s.row_hi && s.n0 < N) {
                        const float gg[4] = {acc[0][0], acc[0][1], acc[0][2], acc[0][3]};
                        const float uu[4] = {acc[1][0], acc[1][1], acc[1][2], acc[1][3]};
                        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + (size_t)m * (N / 2) + s.n0 / 2 +
                                                  4 * (lane >> 4)) = bi::swiglu4(gg, uu);
                    }
                    acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
                    acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
                } else {
#pragma unroll
                    for (int j = 0; j < NT; ++j) {
                        if (m < s.row_hi && s.n0 + 16 * j < N)
                            emit4(y + (size_t)m * N + s.n0 + 16 * j + 4 * (lane >> 4), acc[j], sp.fold);
                        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
                    }
                }
            }
        }
    }
}

template <int MB, int XR, int BKS, int NP, int kMode = kPlain, int NT = 1>
__global__ void __launch_bounds__((MB + NP) * 64)
    bigemm_stream(const uint16_t* __restrict__ x, const uint16_t* __restrict__ W,
                  float* __restrict__ y, int M, int N, int K, Split sp, float* part)
{
    using C = StreamCfg<MB, XR, BKS, NP, NT>;
    __shared__ uint4 ring[C::NR * C::kStageUnits];
    y = cmp_split<kMode>(sp, y, part, M, N);
    const int tiles_n = (N + 16 * NT - 1) / (16 * NT);
    const int mblocks = (M + 16 * MB - 1) / (16 * MB);
    stream_body<MB, XR, BKS, NP, false, NT, kMode == kStreamOnce>(ring, x, W, y, N, K, sp, tiles_n,
                                                                  mblocks * tiles_n, M, nullptr, nullptr);
}

// Grouped: one m-block per expert whose row count c satisfies 0 < c <= cmax
// (cmax <= XR).  kIdx: x rows are read through xidx.  NT = 2 with kSwiGLU:
// the gated projection's SwiGLU, bf16 [R, N / 2] at y (stream_body).
template <int MB, int XR, int BKS, int NP, bool kIdx, int NT = 1, bool kSwiGLU = false>
__global__ void __launch_bounds__((MB + NP) * 64)
    bigemm_stream_grouped(const uint16_t* __restrict__ x, const uint16_t* __restrict__ W,
                          float* __restrict__ y, const int32_t* __restrict__ off, int E, int R,
                          int N, int K, Split sp, int cmax, const int32_t* __restrict__ xidx, int xn)
{
    using C = StreamCfg<MB, XR, BKS, NP, NT>;
    __shared__ uint4 ring[C::NR * C::kStageUnits];
    __shared__ int sh_off[kMaxExperts + 1];
    __shared__ int first[kMaxExperts + 1];
    __shared__ int elist[kMaxExperts];
    // compact, ascending list of the experts this kernel serves
    grouped_plan(off, E, R, 0, 0, cmax, 0, sh_off, first);
    const int count = first[E];
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const int c = sh_off[e + 1] - sh_off[e];
        if (c > 0 && c <= cmax)
            elist[first[e]] = e;
    }
    __syncthreads();
    const int tiles_n = (N + 16 * NT - 1) / (16 * NT);
    // one m-block per expert: every W line the call loads is read once
    stream_body<MB, XR, BKS, NP, kIdx, NT, true, kSwiGLU>(ring, x, W, y, N, K, sp, tiles_n, count * tiles_n, 0,
                                                          sh_off, elist, xidx, xn);
}

// ---------------------------------------------------------------------------
// Launch helpers
// ---------------------------------------------------------------------------
// ysplits > 1 (comparison path only): the kCmp instance over a grid of
// ysplits concurrent K splits, partials of splits 1.. into `part`.
// Extra inputs of a launch beyond the product GEMM's: ysplits > 1 and part
// (comparison path only) run the kCmp instance over a grid of ysplits
// concurrent K splits, partials of splits 1.. into part; rstd and gain
// (RMSNorm'd rows) run the kNormX instance.
struct LaunchExtra {
    int ysplits = 1;
    float* part = nullptr;
    const float* rstd = nullptr;
    const void* gain = nullptr;
};

template <int BM, int BN, int WM, int WN, int BK, int NS>
hipError_t run_tiled(const void* W, const void* x, int M, float* y, int N, int K, Split sp,
                     hipStream_t stream, const LaunchExtra& ex = LaunchExtra())
{
    using C = TiledCfg<BM, BN, WM, WN, BK, NS>;
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    const int nblocks = tiles_m * tiles_n;
    const uint16_t* xx = static_cast<const uint16_t*>(x);
    const uint16_t* ww = static_cast<const uint16_t*>(W);
    const uint4* g = static_cast<const uint4*>(ex.gain);
    if (ex.ysplits > 1)
        hipLaunchKernelGGL((bigemm_tiled<BM, BN, WM, WN, BK, NS, kCmp>), dim3(nblocks, ex.ysplits),
                           dim3(C::kThreads), 0, stream, xx, ww, y, M, N, K, sp, tiles_m, tiles_n, 4, ex.part,
                           nullptr, nullptr);
    else if (ex.rstd) {
        if constexpr (NS >= 3)
            hipLaunchKernelGGL((bigemm_tiled<BM, BN, WM, WN, BK, NS, kNormX>), dim3(nblocks), dim3(C::kThreads), 0,
                               stream, xx, ww, y, M, N, K, sp, tiles_m, tiles_n, 4, nullptr, ex.rstd, g);
        else
            return hipErrorInvalidValue;  // too shallow to normalise its tiles
    } else if (tiles_m == 1)
        // one m-block: each W strip is read by one block, once (non-temporal
        // loads; see the weight streamer's single-m-block calls)
        hipLaunchKernelGGL((bigemm_tiled<BM, BN, WM, WN, BK, NS, kStreamOnce>), dim3(nblocks), dim3(C::kThreads), 0,
                           stream, xx, ww, y, M, N, K, sp, tiles_m, tiles_n, 4, nullptr, nullptr, nullptr);
    else
        hipLaunchKernelGGL((bigemm_tiled<BM, BN, WM, WN, BK, NS>), dim3(nblocks), dim3(C::kThreads), 0, stream, xx,
                           ww, y, M, N, K, sp, tiles_m, tiles_n, 4, nullptr, nullptr, nullptr);
    return hipGetLastError();
}

template <int XT>
hipError_t run_tiled4(const void* W, const void* x, int M, float* y, int N, int K, Split sp, hipStream_t stream,
                      const LaunchExtra& ex = LaunchExtra())
{
    const int tiles_m = (M + 32 * XT - 1) / (32 * XT);
    const int tiles_n = (N + 255) / 256;
    if (ex.rstd)
        return hipErrorInvalidValue;  // no normalising instance of this kernel
    if (ex.ysplits > 1)
        hipLaunchKernelGGL((bigemm_tiled4<XT, kCmp>), dim3(tiles_m * tiles_n, ex.ysplits), dim3(256), 0, stream,
                           static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W), y, M, N, K, sp,
                           tiles_m, tiles_n, 4, ex.part);
    else
        hipLaunchKernelGGL(bigemm_tiled4<XT>, dim3(tiles_m * tiles_n), dim3(256), 0, stream,
                           static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W), y, M, N, K, sp,
                           tiles_m, tiles_n, 4, nullptr);
    return hipGetLastError();
}

template <int MB, int XR, int BKS, int NP, int NT = 1>
hipError_t run_stream(const void* W, const void* x, int M, float* y, int N, int K, Split sp,
                      int num_cus, hipStream_t stream, const LaunchExtra& ex = LaunchExtra())
{
    using C = StreamCfg<MB, XR, BKS, NP, NT>;
    const int items = ((M + 16 * MB - 1) / (16 * MB)) * ((N + 16 * NT - 1) / (16 * NT));
    const int grid = items < num_cus ? items : num_cus;
    if (ex.rstd)
        return hipErrorInvalidValue;  // no normalising instance of this kernel
    if (ex.ysplits > 1)
        hipLaunchKernelGGL((bigemm_stream<MB, XR, BKS, NP, kCmp, NT>), dim3(grid, ex.ysplits), dim3(C::kThreads),
                           0, stream, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W), y, M, N, K,
                           sp, ex.part);
    else {
        // one 16-row m-block: each W line is read once, by one item, so the
        // W loads are non-temporal (measured on the down-proj right after its
        // M = 8192 call: M = 1 24.3 -> 20.6 us; on the 70B shard after
        // M = 16384: M = 1 20.5 -> 11.9 us).  Wider m-blocks and strips keep
        // the default policy (at M = 32 non-temporal W loads were 1% slower).
        if constexpr (MB == 1 && NT == 1) {
            if (M <= 16) {
                hipLaunchKernelGGL((bigemm_stream<MB, XR, BKS, NP, kStreamOnce, NT>), dim3(grid), dim3(C::kThreads),
                                   0, stream, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W), y, M,
                                   N, K, sp, nullptr);
                return hipGetLastError();
            }
        }
        hipLaunchKernelGGL((bigemm_stream<MB, XR, BKS, NP, kPlain, NT>), dim3(grid), dim3(C::kThreads), 0, stream,
                           static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W), y, M, N, K, sp,
                           nullptr);
    }
    return hipGetLastError();
}

// The stage depth: 512 values of k for a single m-tile (1 KB of every row per
// stage), else 256, when K allows it.  x rows per stage: at least what a
// 64-row load group of that stage width needs.
template <int MB, int XR>
hipError_t run_stream_k(const void* W, const void* x, int M, float* y, int N, int K, Split sp,
                        int num_cus, hipStream_t stream, const LaunchExtra& ex = LaunchExtra())
{
    if constexpr (MB == 1) {
        if (sp.klen % 512 == 0)
            return run_stream<MB, XR, 512, stream_producers<MB, 512>()>(W, x, M, y, N, K, sp, num_cus, stream, ex);
    }
    if (sp.klen % 256 == 0)
        return run_stream<MB, XR, 256, stream_producers<MB, 256>()>(W, x, M, y, N, K, sp, num_cus, stream, ex);
    if (sp.klen % 128 == 0)
        return run_stream<MB, (XR < 4 ? 4 : XR), 128, stream_producers<MB, 128>()>(W, x, M, y, N, K, sp, num_cus,
                                                                                   stream, ex);
    return run_stream<MB, (XR < 8 ? 8 : XR), 64, stream_producers<MB, 64>()>(W, x, M, y, N, K, sp, num_cus, stream,
                                                                             ex);
}

// Wide strips (NT > 1): the widest stage, up to 256 values of k, of which
// three fit the LDS budget and that divides the split; every wave that is not
// a consumer produces.
template <int MB, int NT>
constexpr int wide_stage()
{
    return 3 * (16 * (MB + NT)) * 256 * 2 <= kStreamLdsBudget ? 256 : 128;
}
template <int MB, int NT>
hipError_t run_stream_wide(const void* W, const void* x, int M, float* y, int N, int K, Split sp,
                           int num_cus, hipStream_t stream, const LaunchExtra& ex = LaunchExtra())
{
    constexpr int XR = 16 * MB, NP = 8 - MB, B = wide_stage<MB, NT>();
    if (sp.klen % B == 0)
        return run_stream<MB, XR, B, NP, NT>(W, x, M, y, N, K, sp, num_cus, stream, ex);
    if (B > 128 && sp.klen % 128 == 0)
        return run_stream<MB, XR, 128, NP, NT>(W, x, M, y, N, K, sp, num_cus, stream, ex);
    return run_stream<MB, XR, 64, NP, NT>(W, x, M, y, N, K, sp, num_cus, stream, ex);
}

// y += part[0] + part[1] + ... (in that order), 4 values per thread and step:
// the comparison path's combine of its concurrent splits.
__global__ void __launch_bounds__(256)
    splitk_reduce(float4* __restrict__ y, const float4* __restrict__ part, long long n4, int parts)
{
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long long)gridDim.x * 256) {
        float4 v = y[i];
        for (int s = 0; s < parts; ++s) {
            const float4 q = part[(long long)s * n4 + i];
            v.x += q.x;
            v.y += q.y;
            v.z += q.z;
            v.w += q.w;
        }
        y[i] = v;
    }
}

template <int MB, int XR, int BKS, int NP>
hipError_t run_stream_grouped(const void* W, const void* x, const int32_t* off, int E, int R,
                              float* y, int N, int K, Split sp, int cmax, int num_cus, const int32_t* xidx,
                              int xn, hipStream_t stream)
{
    using C = StreamCfg<MB, XR, BKS, NP>;
    if (xidx)
        hipLaunchKernelGGL((bigemm_stream_grouped<MB, XR, BKS, NP, true>), dim3(num_cus), dim3(C::kThreads), 0,
                           stream, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W), y,
                           off, E, R, N, K, sp, cmax, xidx, xn);
    else
        hipLaunchKernelGGL((bigemm_stream_grouped<MB, XR, BKS, NP, false>), dim3(num_cus), dim3(C::kThreads), 0,
                           stream, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W), y,
                           off, E, R, N, K, sp, cmax, xidx, xn);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int BK, int NS>
hipError_t run_tiled_grouped(const void* W, const void* x, const int32_t* off, int E, int R,
                             float* y, int N, int K, Split sp, int cmin, int big, int num_cus,
                             const int32_t* xidx, int xn, hipStream_t stream)
{
    using C = TiledCfg<BM, BN, WM, WN, BK, NS>;
    if (R <= cmin)
        return hipSuccess;  // no expert can have more than cmin rows
    const int tiles_n = (N + BN - 1) / BN;
    // resident blocks: as many per CU as LDS allows (at most two), rounded
    // to whole sets of 8 (one per XCD)
    const int per_cu = 2 * (C::kLdsBytes + 4 * (2 * kMaxExperts + 2)) <= 160 * 1024 ? 2 : 1;
    const int grid = (num_cus * per_cu + 7) / 8 * 8;
    if (xidx)
        hipLaunchKernelGGL((bigemm_tiled_grouped<BM, BN, WM, WN, BK, NS, true>), dim3(grid), dim3(C::kThreads),
                           0, stream, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W), y,
                           off, E, R, N, K, sp, tiles_n, cmin, big, xidx, xn);
    else
        hipLaunchKernelGGL((bigemm_tiled_grouped<BM, BN, WM, WN, BK, NS, false>), dim3(grid), dim3(C::kThreads),
                           0, stream, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W), y,
                           off, E, R, N, K, sp, tiles_n, cmin, big, xidx, xn);
    return hipGetLastError();
}

// The 256-row blocks of the experts with more than cmin rows: one block
// per CU (its LDS holds one), a multiple of 8.
template <bool kIdx, bool kSwiGLU>
hipError_t run_tiled4_grouped_nt(const void* W, const void* x, const int32_t* off, int E, int R, float* y, int N,
                                 int K, Split sp, int cmin, int grid, int tiles_n, const int32_t* xidx, int xn,
                                 bool nt, hipStream_t stream)
{
    if (nt)
        hipLaunchKernelGGL((bigemm_tiled4_grouped<kIdx, kSwiGLU, true>), dim3(grid), dim3(256), 0, stream,
                           static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W), y, off, E, R, N, K,
                           sp, tiles_n, cmin, xidx, xn);
    else
        hipLaunchKernelGGL((bigemm_tiled4_grouped<kIdx, kSwiGLU, false>), dim3(grid), dim3(256), 0, stream,
                           static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W), y, off, E, R, N, K,
                           sp, tiles_n, cmin, xidx, xn);
    return hipGetLastError();
}

// Non-temporal W loads when the experts average under 128 rows, so that each
// of an expert's W tiles is read by a single block (and once), and a tile
// streams at least 1 MB of W (K >= 2048).  Measured on the MoE shapes at
// 2048 rows (16 per expert): the up projection (K = 2048) 157.7 -> 146.5 us,
// the down projection (K = 768) 81.9 -> 84.5 us; at 32768 rows, where about
// half the experts take two blocks, 296 -> 340 us and 187 -> 198 us.
bool grouped_nt_w(int E, int R, int K) { return R < 128 * E && K >= 2048; }

hipError_t run_tiled4_grouped(const void* W, const void* x, const int32_t* off, int E, int R, float* y, int N,
                              int K, Split sp, int cmin, int num_cus, const int32_t* xidx, int xn,
                              hipStream_t stream, bool swiglu = false)
{
    const int tiles_n = (N + 255) / 256;
    const int grid = (num_cus + 7) / 8 * 8;
    const bool nt = grouped_nt_w(E, R, K);
    if (swiglu) {  // the MoE layer's gated up projection: rows always indexed
        if (!xidx)
            return hipErrorInvalidValue;
        return run_tiled4_grouped_nt<true, true>(W, x, off, E, R, y, N, K, sp, cmin, grid, tiles_n, xidx, xn, nt,
                                                 stream);
    }
    if (xidx)
        return run_tiled4_grouped_nt<true, false>(W, x, off, E, R, y, N, K, sp, cmin, grid, tiles_n, xidx, xn, nt,
                                                  stream);
    return run_tiled4_grouped_nt<false, false>(W, x, off, E, R, y, N, K, sp, cmin, grid, tiles_n, xidx, xn, nt,
                                               stream);
}

// The tiled block shapes, largest first.  A shape comes in two depths: a
// shallow pipeline that leaves LDS for two blocks per CU, and a deep one
// (more stages in flight, more waves) for grids with at most one block per
// CU, where nothing else on the CU hides the load latency.
struct TileShape {
    DenseKernel kind, deep;
    int bm, bn;
};
constexpr TileShape kTileShapes[] = {
    {DenseKernel::kTiled256, DenseKernel::kTiled256, 256, 256},
    {DenseKernel::kTiled128x256, DenseKernel::kTiled128x256, 128, 256},
    {DenseKernel::kTiled128, DenseKernel::kTiled128Deep, 128, 128},
    {DenseKernel::kTiled128x64, DenseKernel::kTiled128x64Deep, 128, 64},
    {DenseKernel::kTiled64, DenseKernel::kTiled64, 64, 64},
    {DenseKernel::kTiled64x32, DenseKernel::kTiled64x32, 64, 32},
};

// W [E][N][K] row-major -> the packed slab-major layout, 16 bytes per
// thread and step; a bitwise copy.  Thread v reads unit v of W (row n, the 8
// values from k = 8c) and writes it where the packed layout puts (n, 8c).
// gated_i > 0 (N = 2 gated_i: gate rows, then up rows): packed row n holds,
// for n % 32 < 16, gate row 16 (n / 32) + n % 32, else the up row 16 after
// it, so that a 32-row group holds 16 gate columns and their up columns.
__global__ void __launch_bounds__(256)
    bigemm_pack_w(const uint4* __restrict__ W, uint4* __restrict__ P, int N, int K, long long units, int gated_i)
{
    const long long per = (long long)N * K / 8;  // units per expert
    const int rowu = K / 8;                      // units per W row
    for (long long v = (long long)blockIdx.x * blockDim.x + threadIdx.x; v < units;
         v += (long long)gridDim.x * blockDim.x) {
        const long long e = v / per;
        const long long w = v - e * per;
        int n = (int)(w / rowu);
        const int c = (int)(w % rowu);
        if (gated_i > 0) {
            const int up = n >= gated_i, s = up ? n - gated_i : n;
            n = 32 * (s / 16) + 16 * up + s % 16;
        }
        P[e * per + (long long)(c / 8) * N * 8 + n * 8 + c % 8] = W[v];
    }
}

}  // namespace

hipError_t pack_weights(const void* W, void* packed, int E, int N, int K, hipStream_t stream, int gated_i)
{
    const long long units = (long long)(E > 0 ? E : 1) * N * K / 8;
    const long long blocks = (units + 255) / 256;
    hipLaunchKernelGGL(bigemm_pack_w, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0, stream,
                       static_cast<const uint4*>(W), static_cast<uint4*>(packed), N, K, units, gated_i);
    return hipGetLastError();
}

DenseKernel choose_dense(const Plan& p, int M)
{
    // the pin's tiling list, when it has one: the entry whose row range holds M
    for (int i = 0; i < p.tilings; ++i)
        if (M <= p.tile_m_max[i])
            return static_cast<DenseKernel>(p.tile_kernel[i] & ~BI_KERNEL_CONCURRENT_SPLITS);
    if (M <= p.stream_max_m) {
        if (M <= 16)
            return DenseKernel::kStream16;
        if (M <= 32)
            return DenseKernel::kStream32;
        return DenseKernel::kStream64;
    }
    // The largest output block that still gives every CU a block; failing
    // that, the smallest (the one with the most blocks).
    for (const TileShape& t : kTileShapes) {
        const long long blocks = (long long)((M + t.bm - 1) / t.bm) * ((p.n + t.bn - 1) / t.bn);
        if (blocks >= p.num_cus)
            return blocks <= p.num_cus ? t.deep : t.kind;
    }
    return DenseKernel::kTiled64x32;
}

bool concurrent_splits(const Plan& p, int M)
{
    if (p.splits < 2 || !p.split_ws || M > p.split_ws_rows)
        return false;
    for (int i = 0; i < p.tilings; ++i)
        if (M <= p.tile_m_max[i])
            return (p.tile_kernel[i] & BI_KERNEL_CONCURRENT_SPLITS) != 0;
    return false;
}

const char* dense_kernel_name_cs(DenseKernel k)
{
    switch (k) {
    case DenseKernel::kStream16: return "bigemm_stream<mb=1>,concurrent splits";
    case DenseKernel::kStream32: return "bigemm_stream<mb=2>,concurrent splits";
    case DenseKernel::kStream64: return "bigemm_stream<mb=4>,concurrent splits";
    case DenseKernel::kTiled64x32: return "bigemm_tiled<64x32>,concurrent splits";
    case DenseKernel::kTiled64: return "bigemm_tiled<64x64>,concurrent splits";
    case DenseKernel::kTiled128x64: return "bigemm_tiled<128x64>,concurrent splits";
    case DenseKernel::kTiled128x64Deep: return "bigemm_tiled<128x64,deep>,concurrent splits";
    case DenseKernel::kTiled128: return "bigemm_tiled<128x128>,concurrent splits";
    case DenseKernel::kTiled128Deep: return "bigemm_tiled<128x128,deep>,concurrent splits";
    case DenseKernel::kTiled128x256: return "bigemm_tiled<128x256>,concurrent splits";
    case DenseKernel::kTiled256: return "bigemm_tiled<256x256>,concurrent splits";
    case DenseKernel::kTiled160x256: return "bigemm_tiled<160x256>,concurrent splits";
    case DenseKernel::kTiled192x256: return "bigemm_tiled<192x256>,concurrent splits";
    case DenseKernel::kStream32x32: return "bigemm_stream<mb=2,nt=2>,concurrent splits";
    case DenseKernel::kStream64x32: return "bigemm_stream<mb=4,nt=2>,concurrent splits";
    case DenseKernel::kStream32x64: return "bigemm_stream<mb=2,nt=4>,concurrent splits";
    case DenseKernel::kStream64x64: return "bigemm_stream<mb=4,nt=4>,concurrent splits";
    }
    return "?";
}

const char* kernel_kind_name(int kind)
{
    switch (kind) {
    case BI_KERNEL_STREAM_MB1: return "stream_mb1";
    case BI_KERNEL_STREAM_MB2: return "stream_mb2";
    case BI_KERNEL_STREAM_MB4: return "stream_mb4";
    case BI_KERNEL_TILED_64X32: return "tiled_64x32";
    case BI_KERNEL_TILED_64X64: return "tiled_64x64";
    case BI_KERNEL_TILED_128X64: return "tiled_128x64";
    case BI_KERNEL_TILED_128X64_DEEP: return "tiled_128x64_deep";
    case BI_KERNEL_TILED_128X128: return "tiled_128x128";
    case BI_KERNEL_TILED_128X128_DEEP: return "tiled_128x128_deep";
    case BI_KERNEL_TILED4_128X256: return "tiled4_128x256";
    case BI_KERNEL_TILED4_256X256: return "tiled4_256x256";
    case BI_KERNEL_TILED4_160X256: return "tiled4_160x256";
    case BI_KERNEL_TILED4_192X256: return "tiled4_192x256";
    case BI_KERNEL_STREAM_MB2_N2: return "stream_mb2_n2";
    case BI_KERNEL_STREAM_MB4_N2: return "stream_mb4_n2";
    case BI_KERNEL_STREAM_MB2_N4: return "stream_mb2_n4";
    case BI_KERNEL_STREAM_MB4_N4: return "stream_mb4_n4";
    }
    return "";
}

const char* dense_kernel_name(DenseKernel k)
{
    switch (k) {
    case DenseKernel::kStream16: return "bigemm_stream<mb=1>";
    case DenseKernel::kStream32: return "bigemm_stream<mb=2>";
    case DenseKernel::kStream64: return "bigemm_stream<mb=4>";
    case DenseKernel::kTiled64x32: return "bigemm_tiled<64x32>";
    case DenseKernel::kTiled64: return "bigemm_tiled<64x64>";
    case DenseKernel::kTiled128x64: return "bigemm_tiled<128x64>";
    case DenseKernel::kTiled128x64Deep: return "bigemm_tiled<128x64,deep>";
    case DenseKernel::kTiled128: return "bigemm_tiled<128x128>";
    case DenseKernel::kTiled128Deep: return "bigemm_tiled<128x128,deep>";
    case DenseKernel::kTiled128x256: return "bigemm_tiled<128x256>";
    case DenseKernel::kTiled256: return "bigemm_tiled<256x256>";
    case DenseKernel::kTiled160x256: return "bigemm_tiled<160x256>";
    case DenseKernel::kTiled192x256: return "bigemm_tiled<192x256>";
    case DenseKernel::kStream32x32: return "bigemm_stream<mb=2,nt=2>";
    case DenseKernel::kStream64x32: return "bigemm_stream<mb=4,nt=2>";
    case DenseKernel::kStream32x64: return "bigemm_stream<mb=2,nt=4>";
    case DenseKernel::kStream64x64: return "bigemm_stream<mb=4,nt=4>";
    }
    return "?";
}

namespace {

hipError_t launch_dense_split(const Plan& p, DenseKernel kind, const void* W, const void* x, int M,
                              float* y, Split sp, hipStream_t stream, const LaunchExtra& ex = LaunchExtra())
{
    switch (kind) {
    case DenseKernel::kStream16:
        if (M <= 2)
            return run_stream_k<1, 2>(W, x, M, y, p.n, p.k, sp, p.num_cus, stream, ex);
        if (M <= 4)
            return run_stream_k<1, 4>(W, x, M, y, p.n, p.k, sp, p.num_cus, stream, ex);
        if (M <= 8)
            return run_stream_k<1, 8>(W, x, M, y, p.n, p.k, sp, p.num_cus, stream, ex);
        return run_stream_k<1, 16>(W, x, M, y, p.n, p.k, sp, p.num_cus, stream, ex);
    case DenseKernel::kStream32:
        return run_stream_k<2, 32>(W, x, M, y, p.n, p.k, sp, p.num_cus, stream, ex);
    case DenseKernel::kStream64:
        return run_stream_k<4, 64>(W, x, M, y, p.n, p.k, sp, p.num_cus, stream, ex);
    case DenseKernel::kStream32x32:
        return run_stream_wide<2, 2>(W, x, M, y, p.n, p.k, sp, p.num_cus, stream, ex);
    case DenseKernel::kStream64x32:
        return run_stream_wide<4, 2>(W, x, M, y, p.n, p.k, sp, p.num_cus, stream, ex);
    case DenseKernel::kStream32x64:
        return run_stream_wide<2, 4>(W, x, M, y, p.n, p.k, sp, p.num_cus, stream, ex);
    case DenseKernel::kStream64x64:
        return run_stream_wide<4, 4>(W, x, M, y, p.n, p.k, sp, p.num_cus, stream, ex);
    case DenseKernel::kTiled256:
        return run_tiled4<8>(W, x, M, y, p.n, p.k, sp, stream, ex);
    case DenseKernel::kTiled128x256:
        return run_tiled4<4>(W, x, M, y, p.n, p.k, sp, stream, ex);
    case DenseKernel::kTiled160x256:
        return run_tiled4<5>(W, x, M, y, p.n, p.k, sp, stream, ex);
    case DenseKernel::kTiled192x256:
        return run_tiled4<6>(W, x, M, y, p.n, p.k, sp, stream, ex);
    case DenseKernel::kTiled128:
        return run_tiled<128, 128, 2, 2, 64, 2>(W, x, M, y, p.n, p.k, sp, stream, ex);
    case DenseKernel::kTiled128x64:
        return run_tiled<128, 64, 2, 2, 64, 3>(W, x, M, y, p.n, p.k, sp, stream, ex);
    case DenseKernel::kTiled128x64Deep:
        return run_tiled<128, 64, 2, 2, 64, 6>(W, x, M, y, p.n, p.k, sp, stream, ex);
    case DenseKernel::kTiled128Deep:
        return run_tiled<128, 128, 2, 4, 64, 4>(W, x, M, y, p.n, p.k, sp, stream, ex);
    case DenseKernel::kTiled64x32:
        return run_tiled<64, 32, 2, 2, 64, 8>(W, x, M, y, p.n, p.k, sp, stream, ex);
    case DenseKernel::kTiled64:
        break;
    }
    return run_tiled<64, 64, 2, 2, 64, 4>(W, x, M, y, p.n, p.k, sp, stream, ex);
}

}  // namespace

hipError_t launch_dense(const Plan& p, const void* W, const void* x, int M, float* y,
                        hipStream_t stream)
{
    const DenseKernel kind = choose_dense(p, M);
    // the same tree with its splits side by side: partials of splits 1..S-1
    // into the handle's workspace, then folded into y in split order
    if (concurrent_splits(p, M))
        return launch_splitk(p, static_cast<int>(kind), p.splits, W, x, M, y, p.split_ws, stream);
    const int klen = p.k / p.splits;
    for (int s = 0; s < p.splits; ++s) {
        const hipError_t e = launch_dense_split(p, kind, W, x, M, y, Split{s * klen, klen, s > 0}, stream);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

namespace {

// How a grouped call with R rows splits its experts between the kernels,
// decided on the host from R and E alone.  When the experts average 16 rows
// or more (big), the four-wave kernel takes every expert, the short ones as
// 128-row blocks: one launch that streams each expert's weights once, faster
// than streaming the experts with 16 or fewer rows beside it (on 128 experts
// averaging 16 rows, 8-15% less time than the two launches).  Below
// that, experts with 1..smax rows go to the streaming kernel and the others
// to the tiled kernel.  All realise the same tree, so the split points only
// move work, never bits.
struct GroupedSplit {
    int smax;  // rows at or below which an expert streams (0: no streaming launch)
    bool big;  // the four-wave kernel takes every expert
    bool tiled_launch;  // the tiled kernel is launched (it returns at once when R <= smax)
};

GroupedSplit grouped_split(const Plan& p, int R)
{
    GroupedSplit g;
    g.big = R >= 128 && R >= 16 * p.experts;
    g.smax = g.big ? 0 : (p.stream_max_m < 16 ? p.stream_max_m : 16);
    g.tiled_launch = !g.big && R > g.smax;
    return g;
}

}  // namespace

bool grouped_swiglu_fits(const Plan& p, int R, int max_rows)
{
    if (p.gated_i == 0 || p.splits != 1)
        return false;
    if (max_rows <= kTile)
        return true;  // every expert streams (stream_swiglu)
    const GroupedSplit g = grouped_split(p, R);
    return g.smax == 0 && g.big;
}

namespace {

// The gated projection's SwiGLU when every expert has at most 16 rows: the
// streaming kernel over 32-row strips (a gate tile and its up tile per
// consumer), indexed x rows, the widest stage up to 256 that divides K.
template <int BKS>
hipError_t run_stream_swiglu(const void* W, const void* x, const int32_t* off, int E, int R, void* a, int N, int K,
                             int num_cus, const int32_t* xidx, int xn, hipStream_t stream)
{
    constexpr int NP = stream_producers<1, BKS>();
    using C = StreamCfg<1, 16, BKS, NP, 2>;
    hipLaunchKernelGGL((bigemm_stream_grouped<1, 16, BKS, NP, true, 2, true>), dim3(num_cus), dim3(C::kThreads), 0,
                       stream, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W),
                       static_cast<float*>(a), off, E, R, N, K, Split{0, K, 0}, kTile, xidx, xn);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_swiglu(const Plan& p, const void* W, const void* x, const int32_t* offsets, int R,
                                 void* a, const int32_t* xidx, int xn, int max_rows, hipStream_t stream)
{
    if (!grouped_swiglu_fits(p, R, max_rows) || !xidx)
        return hipErrorInvalidValue;
    if (max_rows <= kTile) {
        if (p.k % 256 == 0)
            return run_stream_swiglu<256>(W, x, offsets, p.experts, R, a, p.n, p.k, p.num_cus, xidx, xn, stream);
        if (p.k % 128 == 0)
            return run_stream_swiglu<128>(W, x, offsets, p.experts, R, a, p.n, p.k, p.num_cus, xidx, xn, stream);
        return run_stream_swiglu<64>(W, x, offsets, p.experts, R, a, p.n, p.k, p.num_cus, xidx, xn, stream);
    }
    // one split, no streaming experts: every expert, whole, in the four-wave kernel
    return run_tiled4_grouped(W, x, offsets, p.experts, R, static_cast<float*>(a), p.n, p.k, Split{0, p.k, 0}, 0,
                              p.num_cus, xidx, xn, stream, true);
}

const char* grouped_kernel_name(const Plan& p, int R)
{
    const GroupedSplit g = grouped_split(p, R);
    if (g.big)
        return "bigemm_tiled4_grouped";
    if (g.smax > 0)
        return g.tiled_launch ? "bigemm_stream_grouped+bigemm_tiled_grouped<128x128>" : "bigemm_stream_grouped";
    return "bigemm_tiled_grouped<128x128>";
}

// The kernels that can normalise their x tiles: the tiled ones with at
// least three stages.  A streaming kind of the pin runs as the 64x32 tiled
// kernel, and the two-stage 128x128 and the four-wave kinds as the deep
// 128x128 one; every kind realises the same tree, so only the speed differs.
DenseKernel norm_kind(DenseKernel k)
{
    switch (k) {
    case DenseKernel::kStream16:
    case DenseKernel::kStream32:
    case DenseKernel::kStream64:
    case DenseKernel::kStream32x32:
    case DenseKernel::kStream64x32:
    case DenseKernel::kStream32x64:
    case DenseKernel::kStream64x64:
        return DenseKernel::kTiled64x32;
    case DenseKernel::kTiled128:  // two stages: too shallow to rewrite one ahead
    case DenseKernel::kTiled128x256:
    case DenseKernel::kTiled256:
    case DenseKernel::kTiled160x256:
    case DenseKernel::kTiled192x256:
        return DenseKernel::kTiled128Deep;
    default:
        return k;
    }
}

hipError_t launch_dense_norm(const Plan& p, const void* W, const void* x, const float* rstd, const void* gain,
                             int M, float* y, hipStream_t stream)
{
    const DenseKernel kind = norm_kind(choose_dense(p, M));
    const int klen = p.k / p.splits;
    LaunchExtra ex;
    ex.rstd = rstd;
    ex.gain = gain;
    for (int s = 0; s < p.splits; ++s) {
        const hipError_t e = launch_dense_split(p, kind, W, x, M, y, Split{s * klen, klen, s > 0}, stream, ex);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

const char* dense_norm_kernel_name(const Plan& p, int M) { return dense_kernel_name(norm_kind(choose_dense(p, M))); }

hipError_t launch_splitk(const Plan& p, int kind, int splits, const void* W, const void* x, int M, float* y,
                         float* part, hipStream_t stream)
{
    const Split sp{0, p.k / splits, 0};
    LaunchExtra ex;
    ex.ysplits = splits;
    ex.part = part;
    hipError_t e = launch_dense_split(p, static_cast<DenseKernel>(kind), W, x, M, y, sp, stream, ex);
    if (e != hipSuccess || splits == 1)
        return e;
    const long long n4 = (long long)M * p.n / 4;
    const long long blocks = (n4 + 255) / 256;
    hipLaunchKernelGGL(splitk_reduce, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, stream,
                       reinterpret_cast<float4*>(y), reinterpret_cast<const float4*>(part), n4, splits - 1);
    return hipGetLastError();
}

hipError_t launch_grouped(const Plan& p, const void* W, const void* x, const int32_t* offsets,
                          int R, float* y, const int32_t* xidx, int xn, hipStream_t stream)
{
    const GroupedSplit g = grouped_split(p, R);
    const int smax = g.smax;
    const int klen = p.k / p.splits;
    for (int s = 0; s < p.splits; ++s) {
        const Split sp{s * klen, klen, s > 0};
        hipError_t err = hipSuccess;
        if (smax > 0) {
            // the widest stage that divides the split: an expert's item is
            // only K / BKS stages, and the narrower the stages the more of
            // them each item pays for (K = 768: 384-wide stages take the
            // 16-token down projection from 67 to 56 us, 128-wide to 101)
            if (klen % 512 == 0)
                err = run_stream_grouped<1, 16, 512, stream_producers<1, 512>()>(W, x, offsets, p.experts, R, y, p.n, p.k, sp, smax, p.num_cus, xidx, xn, stream);
            else if (klen % 384 == 0)
                err = run_stream_grouped<1, 16, 384, stream_producers<1, 384>()>(W, x, offsets, p.experts, R, y, p.n, p.k, sp, smax, p.num_cus, xidx, xn, stream);
            else if (klen % 256 == 0)
                err = run_stream_grouped<1, 16, 256, stream_producers<1, 256>()>(W, x, offsets, p.experts, R, y, p.n, p.k, sp, smax, p.num_cus, xidx, xn, stream);
            else if (klen % 128 == 0)
                err = run_stream_grouped<1, 16, 128, stream_producers<1, 128>()>(W, x, offsets, p.experts, R, y, p.n, p.k, sp, smax, p.num_cus, xidx, xn, stream);
            else
                err = run_stream_grouped<1, 16, 64, stream_producers<1, 64>()>(W, x, offsets, p.experts, R, y, p.n, p.k, sp, smax, p.num_cus, xidx, xn, stream);
            if (err != hipSuccess)
                return err;
        }
        // the four-wave kernel (256- and 128-row blocks) when the experts
        // average 16 rows or more; below that, most experts stream and the
        // few others fill a 128-row block poorly, so the tiled kernel's
        // 128x128 tiles serve them
        const int big = g.big ? 256 : 0;
        if (big)  // every expert, whole (smax is 0 here)
            err = run_tiled4_grouped(W, x, offsets, p.experts, R, y, p.n, p.k, sp, smax, p.num_cus, xidx, xn, stream);
        else
            err = run_tiled_grouped<128, 128, 2, 4, 64, 2>(W, x, offsets, p.experts, R, y, p.n, p.k, sp, smax, big,
                                                           p.num_cus, xidx, xn, stream);
        if (err != hipSuccess)
            return err;
    }
    return hipSuccess;
}

}  // namespace bigemm
