/*
 * bi_gemm.h -- batch-invariant bf16 linear-layer GEMM for AMD MI355X (gfx950).
 *
 *   y[M,N] (fp32) = x[M,K] (bf16) . W[N,K]^T (bf16), fp32 accumulation.
 *
 * Batch invariance.  Row i of y is a function of row i of x, W and the
 * layer's pin only: the same bits whatever M is, wherever the row sits in x and
 * whatever the other rows hold.  This is the kernel property the pages define
 * (CoRun, §III-B Definition 1: x_i = x'_j implies F_n(X)_i = F_m(X')_j for
 * all n, m, i, j; Detent, §3 eq. 2 and its "kernel batch invariance").
 *
 * How.  Floating-point sums depend on their order (LLM-42 reading notes,
 * §2.2 Fig. 3; CoRun, §III-A Fig. 3), and GEMMs change that order when they
 * choose split-K or tiles from the batch.  This library fixes one reduction
 * tree per layer shape (N, K) -- the "pin" of Detent, §3: a value of the
 * selection replaced by a constant before deployment -- and never derives it
 * from M.  The tree is:
 *   - one MFMA instruction, v_mfma_f32_16x16x32_bf16, for every M;
 *   - a fixed map from k to the instruction's (lane group, element) slots:
 *     within MFMA step t of a split, lane group g (= lane / 16) holds
 *     k = 32 t + 8 g .. 32 t + 8 g + 7;
 *   - S contiguous equal K splits, each a chain of MFMA steps in ascending
 *     k, starting from +0;
 *   - the split partials combined in fp32 round-to-nearest-even in fixed
 *     order, ((p0 + p1) + p2) + ... (CoRun, §III-A Fig. 3b; Detent, Fig. 2b).
 * M only chooses among kernels and tilings that realise this same tree
 * (Detent, §2 Observation 2: agreement of such kernels is established by
 * measurement, here the library's invariance tests).
 *
 * Errors.  Every call validates its arguments on the host before any HIP
 * call; on failure it returns an error code, launches nothing and never falls
 * back to another tree (Detent, §5: a failed check stops the engine with an
 * error and runs no other kernel).
 *
 * Threading.  A handle may be used from several host threads for `run` calls
 * on the same or different streams: `run` keeps no per-call state in the
 * handle -- except a handle whose pin runs splits concurrently
 * (BI_KERNEL_CONCURRENT_SPLITS, bi_pin_info.split_ws_rows > 0): its calls
 * share the handle's split workspace and must not overlap.  `destroy` must
 * not race with any other call on that handle.
 */
#ifndef BI_GEMM_H
#define BI_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BI_OK = 0,
    BI_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, bad handle kind      */
    BI_ERR_MISALIGNED = 2,       /* a device pointer is not 16-byte aligned      */
    BI_ERR_NO_PIN = 3,           /* strict mode and no pin for (arch, N, K)      */
    BI_ERR_UNSUPPORTED_DEVICE = 4, /* the current device is not gfx950           */
    BI_ERR_OUT_OF_MEMORY = 5,    /* a host allocation failed                     */
    BI_ERR_HIP = 6,              /* a HIP runtime call failed                    */
    BI_ERR_BAD_PIN_TABLE = 7     /* the pin table file could not be parsed       */
} bi_status_t;

typedef struct bi_gemm *bi_gemm_t;

/*
 * Dense kernels a tiling entry may name.  All of them realise the same tree;
 * the entry only moves work between them (Detent, §3: a knob of the
 * selection is fixed per deployment, never read from the batch).
 */
typedef enum {
    BI_KERNEL_STREAM_MB1 = 0,     /* weight streamer, 16 x rows per m-block      */
    BI_KERNEL_STREAM_MB2 = 1,     /* weight streamer, 32 x rows per m-block      */
    BI_KERNEL_STREAM_MB4 = 2,     /* weight streamer, 64 x rows per m-block      */
    BI_KERNEL_TILED_64X32 = 3,    /* LDS-pipelined tiles: x rows x W rows        */
    BI_KERNEL_TILED_64X64 = 4,
    BI_KERNEL_TILED_128X64 = 5,
    BI_KERNEL_TILED_128X64_DEEP = 6,
    BI_KERNEL_TILED_128X128 = 7,
    BI_KERNEL_TILED_128X128_DEEP = 8,
    BI_KERNEL_TILED4_128X256 = 9, /* four waves, accumulators in AGPRs           */
    BI_KERNEL_TILED4_256X256 = 10,
    BI_KERNEL_TILED4_160X256 = 11, /* the four-wave kernel at other block heights, */
    BI_KERNEL_TILED4_192X256 = 12, /* for M that 128 and 256 rows divide badly     */
    BI_KERNEL_STREAM_MB2_N2 = 13, /* weight streamer over wide W strips: x rows  */
    BI_KERNEL_STREAM_MB4_N2 = 14, /* per m-block x W rows per strip: 32x32,      */
    BI_KERNEL_STREAM_MB2_N4 = 15, /* 64x32, 32x64, 64x64 (mid M: fewer bytes     */
    BI_KERNEL_STREAM_MB4_N4 = 16, /* per CU than 16-column strips)               */
    BI_KERNEL_COUNT = 17
} bi_kernel_kind_t;

/* Most entries of a pin's tiling list. */
#define BI_MAX_TILINGS 12

/*
 * Flag of a tiling entry (tile_kernel[i] | BI_KERNEL_CONCURRENT_SPLITS; in a
 * pin table the kind's name followed by "+cs"): when the tree has S > 1
 * splits, the entry's calls run the S splits concurrently -- S times the
 * workgroups over the same tiles, each summing its own K range from +0 --
 * with splits 1..S-1 writing partials into the handle's split workspace and
 * a final kernel adding them to y in split order, ((p0 + p1) + p2) + ...
 * That is the tree's in-order fold, so the bits are those of the splits run
 * one after another.  Only entries with a finite row bound may carry it:
 * create allocates (S - 1) * bound * N fp32 of workspace for the largest
 * such bound (a call with more rows runs the splits one after another).
 */
#define BI_KERNEL_CONCURRENT_SPLITS 0x100

/* Tree and tiling a handle runs with (introspection for tests and benches). */
typedef struct bi_pin_info {
    int32_t n, k;                 /* layer shape                                 */
    int32_t experts;              /* 0 for a dense handle, E for a grouped one   */
    int32_t mfma_m, mfma_n, mfma_k; /* 16, 16, 32                                */
    int32_t k_map;                /* 0: lane group g holds k = 32t+8g .. +7      */
    int32_t splits;               /* S: contiguous equal K splits                */
    int32_t split_len;            /* K / S                                       */
    int32_t fold;                 /* 0: in-order left fold in fp32 RNE           */
    int32_t stream_max_m;         /* tiling: a grouped call streams the experts
                                     with at most min(this, 16) rows, unless its
                                     experts average 16 rows or more (then the
                                     four-wave kernel takes them all); a dense
                                     call without a tiling list streams calls
                                     with at most this many rows                */
    int32_t from_table;           /* 1: pin read from the pin table; 0: default  */
    int32_t table_version;        /* version line of the pin table (0: none)     */
    int32_t tilings;              /* entries used below; 0: the built-in rule
                                     (streaming up to stream_max_m rows, then
                                     the largest tile that gives every CU one) */
    int32_t tile_m_max[BI_MAX_TILINGS];  /* ascending row bounds: entry i serves
                                     tile_m_max[i-1] < M <= tile_m_max[i]; the
                                     last entry is INT32_MAX (every larger M)   */
    int32_t tile_kernel[BI_MAX_TILINGS]; /* bi_kernel_kind_t of each entry, with
                                     BI_KERNEL_CONCURRENT_SPLITS where the entry
                                     runs its splits concurrently               */
    int32_t split_ws_rows;        /* rows the handle's split workspace holds (0:
                                     none; concurrent splits need it)            */
} bi_pin_info;

/*
 * Identifier of the tree this library realises (a static string without
 * spaces): the MFMA instruction, the k-to-slot map, the split structure and
 * the fold order.  A pin table names the tree it was tuned for on its `tree`
 * line, and a table naming another tree is rejected: the pins are a cached
 * solve that is only valid for the inputs it was computed from (Detent,
 * §4.1: the solve is keyed by a hash of everything that can change it).
 */
const char *bi_gemm_tree_id(void);

/* Table name of a dense kernel kind ("stream_mb1", "tiled4_256x256", ...;
 * "" for an unknown kind). */
const char *bi_gemm_kernel_kind_name(int kind);

/*
 * Load the pin table (text file; see the package's pins/ directory) used by
 * later create calls.  Passing NULL clears the table.  The environment
 * variable BI_GEMM_PINS names a table that is loaded on first use when this
 * is never called; if that table cannot be read or parsed, every later
 * create fails with the table's status (BI_ERR_INVALID_ARGUMENT or
 * BI_ERR_BAD_PIN_TABLE) and the parse error, until a table is loaded here:
 * a named table is never silently replaced by the default tree.  Not
 * thread-safe with concurrent create calls.
 * Format: a `version V` line (V > 0), a `tree ID` line equal to
 * bi_gemm_tree_id(), then one line per layer shape,
 *   arch N K splits stream_max_m [M:kind,M:kind,...,*:kind]
 * where the optional last field is the tiling list (kinds by their
 * bi_gemm_kernel_kind_name, optionally followed by "+cs" for concurrent
 * splits on an entry with a finite bound; bounds ascending, the last `*`).
 * Returns BI_OK, BI_ERR_INVALID_ARGUMENT (unreadable file) or
 * BI_ERR_BAD_PIN_TABLE (with the offending line in bi_last_error()).
 */
bi_status_t bi_gemm_load_pins(const char *path);

/*
 * Strict mode: when nonzero, create fails with BI_ERR_NO_PIN for a shape the
 * pin table does not list, instead of using the built-in default tree
 * (S = 1).  The environment variable BI_GEMM_STRICT=1 sets it on first use.
 */
void bi_gemm_set_strict(int strict);

/*
 * Create a dense handle for a layer with weight W.
 *   N, K: layer shape; N % 16 == 0, K % 64 == 0, both > 0, N*K < 2^31.
 *   W:    device pointer, bf16 [N,K] row-major (nn.Linear layout, K
 *         contiguous), 16-byte aligned.  COPIED: create packs W into the
 *         handle's own device memory (N*K*2 bytes, freed by bi_gemm_destroy)
 *         in the layout the kernels stream, each 64-wide k range of all N
 *         rows contiguous: element (n, k) at (k/64)*64N + 64n + k%64.  The
 *         copy is bitwise.  W may be freed or changed once create returns.
 *   out:  receives the handle.
 * The tree is looked up by (device arch, N, K) and frozen here.  Create
 * synchronizes the device (every earlier write to W has completed when the
 * copy starts), runs the packing kernel and waits for it; it fails with
 * BI_ERR_OUT_OF_MEMORY when the copy cannot be allocated.  The current HIP
 * device must be a gfx950; the handle is bound to it.
 */
bi_status_t bi_gemm_create(int N, int K, const void *W, bi_gemm_t *out);

/*
 * Create a dense handle with an explicit pin instead of the table's.  For the
 * offline tuner, which measures each legal candidate by swapping the pin's
 * constants (Detent, §6 "Search": a repin regenerates the selector without
 * solving again), and for tests that force a kernel path.  Only
 * pin->splits, pin->stream_max_m and the tiling list (pin->tilings,
 * tile_m_max, tile_kernel) are read; the pin must be legal for (N, K)
 * (1 <= splits <= 16, K % (64 * splits) == 0, 0 <= stream_max_m <= 4096;
 * 0 <= tilings <= BI_MAX_TILINGS, bounds ascending and positive, the last
 * INT32_MAX, every kernel a bi_kernel_kind_t), else
 * BI_ERR_INVALID_ARGUMENT.  Otherwise as bi_gemm_create.
 */
bi_status_t bi_gemm_create_pinned(int N, int K, const void *W, const bi_pin_info *pin,
                                  bi_gemm_t *out);

/*
 * y = x W^T for M rows.
 *   x: device bf16 [M,K] row-major, 16-byte aligned; rows are K apart.
 *   y: device fp32 [M,N] row-major, 16-byte aligned.
 *   M: 0 <= M <= 2^31/max(N,K); M == 0 returns BI_OK and launches nothing.
 *   stream: HIP stream (hipStream_t) the kernels are enqueued on; NULL is the
 *           default stream.
 * Asynchronous: no allocation, no synchronisation, no compilation, so the
 * call may be captured into a HIP graph.  x and y are borrowed for the
 * duration of the enqueued work; y must not overlap x or W.  A tree with
 * S > 1 splits enqueues S kernels on `stream`: the first writes each split-0
 * partial into y, each later one adds its split's partial to y in order.
 */
bi_status_t bi_gemm_run(bi_gemm_t h, const void *x, int M, float *y, void *stream);

/*
 * Create a grouped (MoE expert) handle: E experts, each with weight
 * W[e] = W + e*N*K (bf16 [E,N,K], row-major, 16-byte aligned, COPIED as
 * above: E*N*K*2 bytes, each expert packed on its own).  Every expert uses
 * the tree of the dense layer (N, K), so a row
 * computed here has the bits it would have in a dense handle over W[e].
 */
bi_status_t bi_grouped_gemm_create(int E, int N, int K, const void *W, bi_gemm_t *out);

/*
 * Grouped run.  Rows of x are grouped by expert: expert e owns rows
 * expert_offsets[e] .. expert_offsets[e+1]-1, and y[r] = x[r] W[e]^T for them.
 *   x: device bf16 [R,K]; y: device fp32 [R,N]; both 16-byte aligned.
 *   expert_offsets: DEVICE int32 [E+1], read by the kernels (never by the
 *       host): offsets[0] == 0, offsets[E] == R, nondecreasing.  Violating
 *       this is undefined: rows outside any expert are left unwritten, and
 *       the kernels never read x or write y outside rows 0..R-1.
 *   R: total rows, 0 <= R; R == 0 returns BI_OK and launches nothing.
 * Per-expert row counts stay on the device; the kernels choose per expert
 * between kernels that share one tree.  Asynchronous and allocation-free
 * like bi_gemm_run.
 */
bi_status_t bi_grouped_gemm_run(bi_gemm_t h, const void *x, const int32_t *expert_offsets,
                                int R, float *y, void *stream);

/*
 * Grouped run over indexed rows: grouped row i is row row_index[i] of x, so
 * y[i] = x[row_index[i]] W[e]^T for the rows i of expert e.  This is the
 * MoE layer's gather of token rows into expert order (each token appears
 * once per expert it is routed to) done by the kernels' own loads; the
 * result is bit for bit that of bi_grouped_gemm_run on the gathered rows.
 *   x: device bf16 [x_rows, K], 16-byte aligned; 1 <= x_rows, x_rows*K < 2^31.
 *   row_index: DEVICE int32 [R], 4-byte aligned; an index outside
 *       0..x_rows-1 is clamped into it.
 * Other arguments and guarantees as bi_grouped_gemm_run.
 */
bi_status_t bi_grouped_gemm_run_indexed(bi_gemm_t h, const void *x, int x_rows, const int32_t *row_index,
                                        const int32_t *expert_offsets, int R, float *y, void *stream);

/* Release a handle (dense or grouped) and its packed weights; waits for the
 * device work that may still read them.  NULL is ignored. */
void bi_gemm_destroy(bi_gemm_t h);

/* The tree and tiling of a handle. */
bi_status_t bi_gemm_get_pin(bi_gemm_t h, bi_pin_info *out);

/*
 * Name of the kernel a run with M rows launches on this handle, e.g.
 * "bigemm_tiled<256x256>" (a static string; "" for an invalid handle or
 * M <= 0).  For a grouped handle M is the total row count R, and the name
 * lists the launches a run with R rows makes, e.g.
 * "bigemm_stream_grouped+bigemm_tiled4_grouped".  For benches and tests: it
 * launches nothing.  Every name realises the same tree; the choice only
 * moves work.
 */
const char *bi_gemm_kernel_name(bi_gemm_t h, int M);

/* A static English string for a status code. */
const char *bi_status_string(bi_status_t s);

/* Detail of the most recent failure on the calling thread ("" if none). */
const char *bi_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BI_GEMM_H */
