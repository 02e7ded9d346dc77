// Internal declarations shared by the host API and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bi_gemm.h"

namespace bigemm {

// Rows x contributes to one MFMA tile, and the MFMA k depth.  The tree is
// built from v_mfma_f32_16x16x32_bf16 only.
constexpr int kTile = 16;
constexpr int kStepK = 32;

// K granularity the kernels accept (one 64-wide LDS stage of the tiled path).
constexpr int kKGranule = 64;

// Most experts a grouped handle may have (the streaming kernel keeps a list
// of them in LDS).
constexpr int kMaxExperts = 1024;

// Most K splits a tree may have.
constexpr int kMaxSplits = 16;

// What `run` needs from a handle.  The tree (splits) is frozen at create;
// the tiling fields only choose among kernels that realise that tree.
struct Plan {
    int n, k;              // layer shape
    int experts;           // 0 dense, E grouped
    int splits;            // S: contiguous equal K splits, folded in order
    int stream_max_m;      // rows per expert/call at or below which the
                           // weight-streaming kernel runs
    int num_cus;           // compute units of the bound device
    int tilings;           // dense tiling list from the pin (0: built-in rule)
    int tile_m_max[BI_MAX_TILINGS];
    int tile_kernel[BI_MAX_TILINGS];  // kind, | BI_KERNEL_CONCURRENT_SPLITS
    float* split_ws;       // (splits-1) * split_ws_rows * n fp32, or null
    int split_ws_rows;
    int gated_i;           // grouped, gated (the MoE layer's up projection):
                           // n = 2 gated_i and W's rows packed 16 gate rows,
                           // then their 16 up rows (pack_weights); 0 otherwise
};

// The dense kernels `run` may launch; M picks one, the tree is the same.
// The values are the public bi_kernel_kind_t.
enum class DenseKernel {
    kStream16 = BI_KERNEL_STREAM_MB1,
    kStream32 = BI_KERNEL_STREAM_MB2,
    kStream64 = BI_KERNEL_STREAM_MB4,
    kTiled64x32 = BI_KERNEL_TILED_64X32,
    kTiled64 = BI_KERNEL_TILED_64X64,
    kTiled128x64 = BI_KERNEL_TILED_128X64,
    kTiled128x64Deep = BI_KERNEL_TILED_128X64_DEEP,
    kTiled128 = BI_KERNEL_TILED_128X128,
    kTiled128Deep = BI_KERNEL_TILED_128X128_DEEP,
    kTiled128x256 = BI_KERNEL_TILED4_128X256,
    kTiled256 = BI_KERNEL_TILED4_256X256,
    kTiled160x256 = BI_KERNEL_TILED4_160X256,
    kTiled192x256 = BI_KERNEL_TILED4_192X256,
    kStream32x32 = BI_KERNEL_STREAM_MB2_N2,
    kStream64x32 = BI_KERNEL_STREAM_MB4_N2,
    kStream32x64 = BI_KERNEL_STREAM_MB2_N4,
    kStream64x64 = BI_KERNEL_STREAM_MB4_N4,
};
DenseKernel choose_dense(const Plan& p, int M);
// Whether a call with M rows runs its splits concurrently (the tiling
// entry's flag, S > 1, and M within the split workspace).
bool concurrent_splits(const Plan& p, int M);
const char* dense_kernel_name(DenseKernel k);
// The name with ",concurrent splits" appended.
const char* dense_kernel_name_cs(DenseKernel k);
// Table name of a kind ("" when unknown).
const char* kernel_kind_name(int kind);
// The launches a grouped call with R rows makes, e.g.
// "bigemm_stream_grouped+bigemm_tiled4_grouped".
const char* grouped_kernel_name(const Plan& p, int R);

// Host helpers the MoE layer's API shares with the GEMM API
// (bigemm_api.cpp): record the calling thread's bi_last_error() and return
// st; and the current device, failing unless it is a gfx950.
bi_status_t api_fail(bi_status_t st, const char* msg);
bi_status_t api_device(int* dev, int* num_cus);

// Launchers (bigemm_kernels.hip).  They assume validated arguments.  The
// weights they take are packed by pack_weights: slab-major, element (n, k)
// of an [N, K] matrix at index (k / 64) * 64N + 64n + k % 64.
// gated_i > 0: the gate/up row interleave of a gated up projection (Plan).
hipError_t pack_weights(const void* W, void* packed, int E, int N, int K, hipStream_t stream, int gated_i = 0);
hipError_t launch_dense(const Plan& p, const void* W, const void* x, int M, float* y,
                        hipStream_t stream);
// Non-invariant comparison: kernel `kind` over `splits` concurrent K splits,
// partials of splits 1.. in part ([splits-1][M][N] fp32), then added to y.
hipError_t launch_splitk(const Plan& p, int kind, int splits, const void* W, const void* x, int M, float* y,
                         float* part, hipStream_t stream);
// y = RMSNorm(x) W^T with the norm applied to the x tiles in LDS: rstd
// [M] fp32 from the RMSNorm row pass, gain bf16 [K]; the kernel a call with
// M rows runs (a tiled kind; see norm_kind).
hipError_t launch_dense_norm(const Plan& p, const void* W, const void* x, const float* rstd, const void* gain,
                             int M, float* y, hipStream_t stream);
const char* dense_norm_kernel_name(const Plan& p, int M);
// xidx (optional): row i of the grouped x is row xidx[i] of x (xn rows).
hipError_t launch_grouped(const Plan& p, const void* W, const void* x,
                          const int32_t* offsets, int R, float* y, const int32_t* xidx, int xn,
                          hipStream_t stream);
// A gated handle's product with SwiGLU in a kernel's epilogue: a [R,
// gated_i] bf16, a[r][c] = swiglu_bf16(gate, up) of the row's product columns
// c and gated_i + c.  Only when grouped_swiglu_fits (one split, and either
// every expert has at most max_rows <= 16 rows -- the streaming kernel over
// 32-row strips; an expert with more rows would be left unwritten, so the
// caller must know the bound -- or R large enough that every expert runs in
// the four-wave kernel).  x rows always through xidx.
bool grouped_swiglu_fits(const Plan& p, int R, int max_rows);
hipError_t launch_grouped_swiglu(const Plan& p, const void* W, const void* x, const int32_t* offsets, int R,
                                 void* a, const int32_t* xidx, int xn, int max_rows, hipStream_t stream);

// The MoE layer's gated up projection (bigemm_api.cpp): a grouped handle over
// W [E, 2I, K] (gate rows 0..I-1, up rows I..2I-1) whose weights are packed
// with the gate/up row interleave, so that its product columns come out
// interleaved the same way (16 gate columns, then their 16 up columns;
// bi_grouped_gemm_run and _run_indexed work on it as on any grouped handle),
// and its product with SwiGLU applied (a [R, I] bf16) when the call fits.
bi_status_t create_gated(int E, int I, int K, const void* W, bi_gemm_t* out);
bool swiglu_fits(bi_gemm_t h, int R, int max_rows);
bi_status_t run_swiglu_indexed(bi_gemm_t h, const void* x, int x_rows, const int32_t* row_index,
                               const int32_t* expert_offsets, int R, int max_rows, void* a, void* stream);

}  // namespace bigemm
