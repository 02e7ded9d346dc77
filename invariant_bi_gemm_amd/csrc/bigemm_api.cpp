// Host side of the batch-invariant GEMM library: handles, validation, the pin
// table and dispatch.  Every argument check runs on the host before any HIP
// call, and a failed check returns an error without launching anything
// (Detent, §5: a failed precondition stops the engine with an error and runs
// no other kernel).  The tree a handle runs with is frozen at create from
// (device arch, N, K) only; `run` reads M solely to pick among kernels that
// realise that tree (Detent, §3: pins depend on the deployment, never on the
// batch).

#include <hip/hip_runtime.h>

#include <cerrno>
#include <cmath>
#include <climits>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <unordered_set>
#include <vector>

#include "../../include/bi_gemm_ref.h"
#include "../../include/bi_norm.h"
#include "norm_internal.h"
#include "bigemm_internal.h"

namespace {

constexpr uint32_t kMagic = 0xB16E3A11u;
constexpr int kMaxDevices = 64;

thread_local std::string g_last_error;

bi_status_t fail(bi_status_t st, const std::string& msg)
{
    g_last_error = msg;
    return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---- pin table -------------------------------------------------------------

// The tree this library realises, as a pin table names it.  Change the
// last component whenever a kernel change could change any output bit
// (instruction, k-to-slot map, split structure, fold order): tables tuned
// for the old tree are then rejected instead of read.
constexpr const char* kTreeId = "mfma_f32_16x16x32_bf16.kmap_g8.contiguous_splits.left_fold.t1";

struct Tiling {
    int count = 0;
    int m_max[BI_MAX_TILINGS];
    int kernel[BI_MAX_TILINGS];
};

struct PinRow {
    std::string arch;
    int n, k, splits, stream_max_m;
    Tiling tiling;
};

struct PinTable {
    int version = 0;
    std::vector<PinRow> rows;
};

std::mutex g_pin_mu;
PinTable g_pins;
bool g_pins_env_checked = false;
// a BI_GEMM_PINS table that failed to load: its status and message, returned
// by every create until bi_gemm_load_pins replaces it
bi_status_t g_pins_env_status = BI_OK;
std::string g_pins_env_error;
int g_strict = -1;  // -1: read BI_GEMM_STRICT on first use

// The default tiling when the table has no entry: the streaming kernel for
// up to 16 rows.  The default tree is S = 1.
constexpr int kDefaultStreamMaxM = 16;

// A pin is legal for (N, K) when its splits divide K into equal parts that
// are whole 64-wide stages, and the streaming threshold is sane.
bool pin_legal(int N, int K, int splits, int stream_max_m, std::string* why)
{
    (void)N;
    if (splits < 1 || splits > bigemm::kMaxSplits) {
        *why = "splits must be within 1..16";
        return false;
    }
    if (K % (splits * bigemm::kKGranule) != 0) {
        *why = "K must split into equal parts that are multiples of 64";
        return false;
    }
    if (stream_max_m < 0 || stream_max_m > 4096) {
        *why = "stream_max_m must be within 0..4096";
        return false;
    }
    return true;
}

// Largest row bound of a tiling entry that runs concurrent splits (it sizes
// the handle's split workspace).
constexpr int kMaxSplitWsRows = 16384;

// A tiling list is legal when its bounds ascend, are positive, end with
// INT32_MAX and every kernel is a known kind; concurrent splits only on
// entries with a bound of at most kMaxSplitWsRows.
bool tiling_legal(int count, const int* m_max, const int* kernel, std::string* why)
{
    if (count < 0 || count > BI_MAX_TILINGS) {
        *why = "a tiling list has 0.." + std::to_string(BI_MAX_TILINGS) + " entries";
        return false;
    }
    for (int i = 0; i < count; ++i) {
        const int kind = kernel[i] & ~BI_KERNEL_CONCURRENT_SPLITS;
        if (kind < 0 || kind >= BI_KERNEL_COUNT) {
            *why = "unknown kernel kind " + std::to_string(kernel[i]);
            return false;
        }
        if ((kernel[i] & BI_KERNEL_CONCURRENT_SPLITS) && i == count - 1) {
            *why = "the entry that covers every larger M cannot run concurrent splits (its workspace would be unbounded)";
            return false;
        }
        if ((kernel[i] & BI_KERNEL_CONCURRENT_SPLITS) && m_max[i] > kMaxSplitWsRows) {
            *why = "concurrent splits are allowed up to " + std::to_string(kMaxSplitWsRows) + " rows";
            return false;
        }
        if (m_max[i] < 1 || (i > 0 && m_max[i] <= m_max[i - 1])) {
            *why = "tiling bounds must be positive and ascending";
            return false;
        }
    }
    if (count > 0 && m_max[count - 1] != INT32_MAX) {
        *why = "the last tiling entry must cover every larger M";
        return false;
    }
    return true;
}

// "M:kind,M:kind,...,*:kind" -> a tiling list
bool parse_tiling(const char* text, Tiling* t, std::string* why)
{
    t->count = 0;
    std::string item;
    const std::string all(text);
    size_t pos = 0;
    while (pos <= all.size()) {
        const size_t comma = all.find(',', pos);
        item = all.substr(pos, comma == std::string::npos ? std::string::npos : comma - pos);
        pos = comma == std::string::npos ? all.size() + 1 : comma + 1;
        const size_t colon = item.find(':');
        if (colon == std::string::npos || colon == 0) {
            *why = "tiling entries are M:kind";
            return false;
        }
        if (t->count == BI_MAX_TILINGS) {
            *why = "too many tiling entries";
            return false;
        }
        const std::string m = item.substr(0, colon), kind = item.substr(colon + 1);
        int bound;
        if (m == "*") {
            bound = INT32_MAX;
        } else {
            char* end = nullptr;
            const long v = std::strtol(m.c_str(), &end, 10);
            if (!end || *end || v < 1 || v >= INT32_MAX) {
                *why = "bad tiling bound '" + m + "'";
                return false;
            }
            bound = (int)v;
        }
        std::string base = kind;
        int flag = 0;
        if (base.size() > 3 && base.compare(base.size() - 3, 3, "+cs") == 0) {
            base = base.substr(0, base.size() - 3);
            flag = BI_KERNEL_CONCURRENT_SPLITS;
        }
        int k = -1;
        for (int c = 0; c < BI_KERNEL_COUNT; ++c)
            if (base == bigemm::kernel_kind_name(c))
                k = c | flag;
        if (k < 0) {
            *why = "unknown kernel kind '" + kind + "'";
            return false;
        }
        t->m_max[t->count] = bound;
        t->kernel[t->count] = k;
        ++t->count;
    }
    return tiling_legal(t->count, t->m_max, t->kernel, why);
}

bi_status_t parse_pins(const char* path, PinTable* out)
{
    FILE* f = std::fopen(path, "r");
    if (!f)
        return fail(BI_ERR_INVALID_ARGUMENT, std::string("cannot open pin table ") + path + ": " +
                                                 std::strerror(errno));
    PinTable t;
    char line[640];
    int lineno = 0;
    bool tree_seen = false;
    bi_status_t st = BI_OK;
    while (std::fgets(line, sizeof line, f)) {
        ++lineno;
        char* hash = std::strchr(line, '#');
        if (hash)
            *hash = 0;
        char a[64];
        int n, k, s, sm, v;
        char extra[8];
        char tiles[400];
        if (std::sscanf(line, " %63s", a) != 1)
            continue;  // blank
        if (std::strcmp(a, "version") == 0) {
            if (std::sscanf(line, " version %d %7s", &v, extra) != 1 || v <= 0) {
                st = fail(BI_ERR_BAD_PIN_TABLE, "pin table line " + std::to_string(lineno) + ": bad version line");
                break;
            }
            t.version = v;
            continue;
        }
        if (std::strcmp(a, "tree") == 0) {
            char id[200];
            if (std::sscanf(line, " tree %199s %7s", id, extra) != 1) {
                st = fail(BI_ERR_BAD_PIN_TABLE, "pin table line " + std::to_string(lineno) + ": bad tree line");
                break;
            }
            if (std::strcmp(id, kTreeId) != 0) {
                st = fail(BI_ERR_BAD_PIN_TABLE, "pin table line " + std::to_string(lineno) + ": the table was tuned for tree " +
                                                    id + ", this library realises " + kTreeId);
                break;
            }
            tree_seen = true;
            continue;
        }
        const int got = std::sscanf(line, " %63s %d %d %d %d %399s %7s", a, &n, &k, &s, &sm, tiles, extra);
        if (got != 5 && got != 6) {
            st = fail(BI_ERR_BAD_PIN_TABLE, "pin table line " + std::to_string(lineno) +
                                                ": expected 'arch N K splits stream_max_m [tilings]'");
            break;
        }
        std::string why;
        if (n <= 0 || k <= 0 || n % bigemm::kTile || k % bigemm::kKGranule ||
            !pin_legal(n, k, s, sm, &why)) {
            st = fail(BI_ERR_BAD_PIN_TABLE, "pin table line " + std::to_string(lineno) +
                                                ": illegal pin " + (why.empty() ? "shape" : why));
            break;
        }
        Tiling tiling;
        if (got == 6 && !parse_tiling(tiles, &tiling, &why)) {
            st = fail(BI_ERR_BAD_PIN_TABLE, "pin table line " + std::to_string(lineno) + ": " + why);
            break;
        }
        for (const PinRow& r : t.rows)
            if (r.arch == a && r.n == n && r.k == k) {
                st = fail(BI_ERR_BAD_PIN_TABLE, "pin table line " + std::to_string(lineno) + ": duplicate shape");
                break;
            }
        if (st != BI_OK)
            break;
        t.rows.push_back(PinRow{a, n, k, s, sm, tiling});
    }
    std::fclose(f);
    if (st == BI_OK && t.version == 0)
        st = fail(BI_ERR_BAD_PIN_TABLE, "pin table has no version line");
    if (st == BI_OK && !tree_seen)
        st = fail(BI_ERR_BAD_PIN_TABLE, std::string("pin table has no tree line (this library realises ") +
                                            kTreeId + ")");
    if (st == BI_OK)
        *out = std::move(t);
    return st;
}

void check_env_locked()
{
    if (!g_pins_env_checked) {
        g_pins_env_checked = true;
        const char* p = std::getenv("BI_GEMM_PINS");
        if (p && *p) {
            PinTable t;
            const bi_status_t st = parse_pins(p, &t);
            if (st == BI_OK) {
                g_pins = std::move(t);
            } else {
                g_pins_env_status = st;
                g_pins_env_error = std::string("BI_GEMM_PINS=") + p + ": " + g_last_error;
            }
        }
    }
    if (g_strict < 0) {
        const char* s = std::getenv("BI_GEMM_STRICT");
        g_strict = (s && std::strcmp(s, "1") == 0) ? 1 : 0;
    }
}

// ---- devices ---------------------------------------------------------------

struct DeviceInfo {
    bool known = false;
    bool gfx950 = false;
    int num_cus = 0;
    std::string arch;
};
std::mutex g_dev_mu;
DeviceInfo g_dev[kMaxDevices];

bi_status_t current_device(int* dev, DeviceInfo* info)
{
    hipError_t e = hipGetDevice(dev);
    if (e != hipSuccess)
        return fail(BI_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    if (*dev < 0 || *dev >= kMaxDevices)
        return fail(BI_ERR_UNSUPPORTED_DEVICE, "device index out of range");
    std::lock_guard<std::mutex> g(g_dev_mu);
    DeviceInfo& d = g_dev[*dev];
    if (!d.known) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, *dev);
        if (e != hipSuccess)
            return fail(BI_ERR_HIP, std::string("hipGetDeviceProperties: ") + hipGetErrorString(e));
        d.arch = prop.gcnArchName;
        d.gfx950 = d.arch.compare(0, 6, "gfx950") == 0;
        d.num_cus = prop.multiProcessorCount;
        d.known = true;
    }
    *info = d;
    return BI_OK;
}

}  // namespace

struct bi_gemm {
    uint32_t magic;
    int device;
    void* W;  // the handle's packed copy of the weights (slab-major), owned
    void* split_ws;  // partials of concurrent splits, owned (or null)
    bigemm::Plan plan;
    bi_pin_info pin;
};

namespace {

// Live handles, so that a stale or foreign pointer is rejected instead of
// being read.
std::mutex g_live_mu;
std::unordered_set<const bi_gemm*> g_live;

bi_gemm* handle_of(bi_gemm_t h)
{
    if (!h)
        return nullptr;
    {
        std::lock_guard<std::mutex> g(g_live_mu);
        if (g_live.find(h) == g_live.end())
            return nullptr;
    }
    return h->magic == kMagic ? h : nullptr;
}

bi_status_t create_common(int E, int N, int K, const void* W, const bi_pin_info* forced,
                          bi_gemm_t* out, int gated_i = 0)
{
    if (!out)
        return fail(BI_ERR_INVALID_ARGUMENT, "out is NULL");
    *out = nullptr;
    if (!W)
        return fail(BI_ERR_INVALID_ARGUMENT, "W is NULL");
    if (N <= 0 || K <= 0)
        return fail(BI_ERR_INVALID_ARGUMENT, "N and K must be positive");
    if (N % bigemm::kTile != 0)
        return fail(BI_ERR_INVALID_ARGUMENT, "N must be a multiple of 16");
    if (K % bigemm::kKGranule != 0)
        return fail(BI_ERR_INVALID_ARGUMENT, "K must be a multiple of 64");
    if ((long long)N * K >= (1LL << 31))
        return fail(BI_ERR_INVALID_ARGUMENT, "N*K must be below 2^31");
    if (E < 0 || E > bigemm::kMaxExperts)
        return fail(BI_ERR_INVALID_ARGUMENT, "E must be within 1..1024");
    if (!aligned16(W))
        return fail(BI_ERR_MISALIGNED, "W must be 16-byte aligned");

    // the pin: forced (tuner), table, or default
    int splits = 1, stream_max_m = kDefaultStreamMaxM, from_table = 0, version = 0;
    Tiling tiling;
    if (forced) {
        std::string why;
        if (!pin_legal(N, K, forced->splits, forced->stream_max_m, &why) ||
            !tiling_legal(forced->tilings, forced->tile_m_max, forced->tile_kernel, &why))
            return fail(BI_ERR_INVALID_ARGUMENT, "illegal pin: " + why);
        splits = forced->splits;
        stream_max_m = forced->stream_max_m;
        tiling.count = forced->tilings;
        for (int i = 0; i < tiling.count; ++i) {
            tiling.m_max[i] = forced->tile_m_max[i];
            tiling.kernel[i] = forced->tile_kernel[i];
        }
    }

    if (!forced) {
        // a table named by BI_GEMM_PINS that failed to load stops every
        // create that would read it, before any HIP call
        std::lock_guard<std::mutex> g(g_pin_mu);
        check_env_locked();
        if (g_pins_env_status != BI_OK)
            return fail(g_pins_env_status, g_pins_env_error);
    }

    int dev;
    DeviceInfo info;
    bi_status_t st = current_device(&dev, &info);
    if (st != BI_OK)
        return st;
    if (!info.gfx950)
        return fail(BI_ERR_UNSUPPORTED_DEVICE, "device " + std::to_string(dev) + " is " + info.arch +
                                                   ", this library is built for gfx950 only");

    if (!forced) {
        std::lock_guard<std::mutex> g(g_pin_mu);
        if (g_pins_env_status != BI_OK)
            return fail(g_pins_env_status, g_pins_env_error);
        const PinRow* row = nullptr;
        for (const PinRow& r : g_pins.rows)
            if (r.n == N && r.k == K && info.arch.compare(0, r.arch.size(), r.arch) == 0)
                row = &r;
        if (row) {
            splits = row->splits;
            stream_max_m = row->stream_max_m;
            tiling = row->tiling;
            from_table = 1;
            version = g_pins.version;
        } else if (g_strict) {
            return fail(BI_ERR_NO_PIN, "strict mode: no pin for N=" + std::to_string(N) +
                                           " K=" + std::to_string(K) + " on " + info.arch);
        }
    }

    // The packed copy of W: every earlier write to W on the device has
    // completed when the copy starts, and the copy has when create returns,
    // so the caller may then free or change W.
    const size_t wbytes = (size_t)(E > 0 ? E : 1) * N * K * 2;
    void* packed = nullptr;
    hipError_t he = hipDeviceSynchronize();
    if (he != hipSuccess)
        return fail(BI_ERR_HIP, std::string("hipDeviceSynchronize: ") + hipGetErrorString(he));
    if (hipMalloc(&packed, wbytes) != hipSuccess) {
        (void)hipGetLastError();
        return fail(BI_ERR_OUT_OF_MEMORY, "out of device memory for the packed weights (" +
                                              std::to_string(wbytes) + " bytes)");
    }
    he = bigemm::pack_weights(W, packed, E, N, K, nullptr, gated_i);
    if (he == hipSuccess)
        he = hipStreamSynchronize(nullptr);
    if (he != hipSuccess) {
        (void)hipFree(packed);
        return fail(BI_ERR_HIP, std::string("packing W: ") + hipGetErrorString(he));
    }

    // the split workspace: (S - 1) partials of the largest row bound whose
    // tiling entry runs its splits concurrently
    int ws_rows = 0;
    if (E == 0 && splits > 1)
        for (int i = 0; i < tiling.count; ++i)
            if ((tiling.kernel[i] & BI_KERNEL_CONCURRENT_SPLITS) && tiling.m_max[i] > ws_rows)
                ws_rows = tiling.m_max[i];
    void* split_ws = nullptr;
    if (ws_rows > 0) {
        const size_t bytes = (size_t)(splits - 1) * ws_rows * N * sizeof(float);
        if (hipMalloc(&split_ws, bytes) != hipSuccess) {
            (void)hipGetLastError();
            (void)hipFree(packed);
            return fail(BI_ERR_OUT_OF_MEMORY, "out of device memory for the split workspace (" +
                                                  std::to_string(bytes) + " bytes)");
        }
    }

    bi_gemm* h = new (std::nothrow) bi_gemm;
    if (!h) {
        (void)hipFree(packed);
        (void)hipFree(split_ws);
        return fail(BI_ERR_OUT_OF_MEMORY, "out of host memory");
    }
    h->magic = kMagic;
    h->device = dev;
    h->W = packed;
    h->split_ws = split_ws;
    h->plan.n = N;
    h->plan.k = K;
    h->plan.experts = E;
    h->plan.splits = splits;
    h->plan.stream_max_m = stream_max_m;
    h->plan.num_cus = info.num_cus;
    // a grouped handle always uses the built-in split between its kernels
    h->plan.tilings = E > 0 ? 0 : tiling.count;
    for (int i = 0; i < h->plan.tilings; ++i) {
        h->plan.tile_m_max[i] = tiling.m_max[i];
        h->plan.tile_kernel[i] = tiling.kernel[i];
    }
    h->plan.split_ws = static_cast<float*>(split_ws);
    h->plan.split_ws_rows = ws_rows;
    h->plan.gated_i = gated_i;
    bi_pin_info& p = h->pin;
    std::memset(&p, 0, sizeof p);
    p.n = N;
    p.k = K;
    p.experts = E;
    p.mfma_m = bigemm::kTile;
    p.mfma_n = bigemm::kTile;
    p.mfma_k = bigemm::kStepK;
    p.k_map = 0;
    p.splits = splits;
    p.split_len = K / splits;
    p.fold = 0;
    p.stream_max_m = stream_max_m;
    p.from_table = from_table;
    p.table_version = version;
    p.tilings = h->plan.tilings;
    for (int i = 0; i < p.tilings; ++i) {
        p.tile_m_max[i] = h->plan.tile_m_max[i];
        p.tile_kernel[i] = h->plan.tile_kernel[i];
    }
    p.split_ws_rows = ws_rows;
    try {
        std::lock_guard<std::mutex> g(g_live_mu);
        g_live.insert(h);
    } catch (...) {
        (void)hipFree(h->W);
        (void)hipFree(h->split_ws);
        delete h;
        return fail(BI_ERR_OUT_OF_MEMORY, "out of host memory");
    }
    *out = h;
    g_last_error.clear();
    return BI_OK;
}

bi_status_t check_run_device(const bi_gemm* h)
{
    int dev;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(BI_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    if (dev != h->device)
        return fail(BI_ERR_INVALID_ARGUMENT, "the current device is not the handle's device");
    return BI_OK;
}

}  // namespace

namespace bigemm {

bi_status_t api_fail(bi_status_t st, const char* msg) { return fail(st, msg); }

bi_status_t api_device(int* dev, int* num_cus)
{
    DeviceInfo info;
    const bi_status_t st = current_device(dev, &info);
    if (st != BI_OK)
        return st;
    if (!info.gfx950)
        return fail(BI_ERR_UNSUPPORTED_DEVICE, "device " + std::to_string(*dev) + " is " + info.arch +
                                                   ", the kernels are built for gfx950");
    *num_cus = info.num_cus;
    return BI_OK;
}

}  // namespace bigemm

extern "C" {

const char* bi_gemm_tree_id(void) { return kTreeId; }

const char* bi_gemm_kernel_kind_name(int kind) { return bigemm::kernel_kind_name(kind); }

bi_status_t bi_gemm_load_pins(const char* path)
{
    std::lock_guard<std::mutex> g(g_pin_mu);
    g_pins_env_checked = true;
    if (!path) {
        g_pins = PinTable();
        g_pins_env_status = BI_OK;
        return BI_OK;
    }
    PinTable t;
    bi_status_t st = parse_pins(path, &t);
    if (st == BI_OK) {
        g_pins = std::move(t);
        g_pins_env_status = BI_OK;
    }
    return st;
}

void bi_gemm_set_strict(int strict)
{
    std::lock_guard<std::mutex> g(g_pin_mu);
    g_strict = strict ? 1 : 0;
}

bi_status_t bi_gemm_create(int N, int K, const void* W, bi_gemm_t* out)
{
    return create_common(0, N, K, W, nullptr, out);
}

bi_status_t bi_gemm_create_pinned(int N, int K, const void* W, const bi_pin_info* pin, bi_gemm_t* out)
{
    if (!pin) {
        if (out)
            *out = nullptr;
        return fail(BI_ERR_INVALID_ARGUMENT, "pin is NULL");
    }
    return create_common(0, N, K, W, pin, out);
}

bi_status_t bi_grouped_gemm_create(int E, int N, int K, const void* W, bi_gemm_t* out)
{
    if (E <= 0) {
        if (out)
            *out = nullptr;
        return fail(BI_ERR_INVALID_ARGUMENT, "E must be within 1..1024");
    }
    if ((long long)E * N * K >= (1LL << 40)) {
        if (out)
            *out = nullptr;
        return fail(BI_ERR_INVALID_ARGUMENT, "E*N*K too large");
    }
    return create_common(E, N, K, W, nullptr, out);
}

bi_status_t bi_gemm_run(bi_gemm_t hh, const void* x, int M, float* y, void* stream)
{
    bi_gemm* h = handle_of(hh);
    if (!h)
        return fail(BI_ERR_INVALID_ARGUMENT, "invalid handle");
    if (h->plan.experts != 0)
        return fail(BI_ERR_INVALID_ARGUMENT, "grouped handle passed to bi_gemm_run");
    if (M < 0)
        return fail(BI_ERR_INVALID_ARGUMENT, "M must be >= 0");
    if (M == 0)
        return BI_OK;
    if (!x || !y)
        return fail(BI_ERR_INVALID_ARGUMENT, "x or y is NULL");
    if (!aligned16(x) || !aligned16(y))
        return fail(BI_ERR_MISALIGNED, "x and y must be 16-byte aligned");
    const long long wide = h->plan.n > h->plan.k ? h->plan.n : h->plan.k;
    if ((long long)M * wide >= (1LL << 31))
        return fail(BI_ERR_INVALID_ARGUMENT, "M*max(N,K) must be below 2^31");
    bi_status_t st = check_run_device(h);
    if (st != BI_OK)
        return st;
    hipError_t e = bigemm::launch_dense(h->plan, h->W, x, M, y, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(BI_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
    return BI_OK;
}

bi_status_t bi_gemm_run_splitk(bi_gemm_t hh, const void* x, int M, float* y, int kind, int splits, float* workspace,
                               void* stream)
{
    bi_gemm* h = handle_of(hh);
    if (!h)
        return fail(BI_ERR_INVALID_ARGUMENT, "invalid handle");
    if (h->plan.experts != 0)
        return fail(BI_ERR_INVALID_ARGUMENT, "grouped handle passed to bi_gemm_run_splitk");
    if (kind < 0 || kind >= BI_KERNEL_COUNT)
        return fail(BI_ERR_INVALID_ARGUMENT, "unknown kernel kind");
    if (splits < 1 || splits > bigemm::kMaxSplits || h->plan.k % (splits * bigemm::kKGranule) != 0)
        return fail(BI_ERR_INVALID_ARGUMENT, "splits must be within 1..16 and cut K into equal multiples of 64");
    if (M < 0)
        return fail(BI_ERR_INVALID_ARGUMENT, "M must be >= 0");
    if (M == 0)
        return BI_OK;
    if (!x || !y || (splits > 1 && !workspace))
        return fail(BI_ERR_INVALID_ARGUMENT, "x, y or workspace is NULL");
    if (!aligned16(x) || !aligned16(y) || (splits > 1 && !aligned16(workspace)))
        return fail(BI_ERR_MISALIGNED, "x, y and workspace must be 16-byte aligned");
    const long long wide = h->plan.n > h->plan.k ? h->plan.n : h->plan.k;
    if ((long long)M * wide >= (1LL << 31))
        return fail(BI_ERR_INVALID_ARGUMENT, "M*max(N,K) must be below 2^31");
    if (splits > 1) {
        const char* wb = reinterpret_cast<const char*>(workspace);
        const char* yb = reinterpret_cast<const char*>(y);
        const size_t ybytes = (size_t)M * h->plan.n * 4, wbytes = ybytes * (size_t)(splits - 1);
        if (wb < yb + ybytes && yb < wb + wbytes)
            return fail(BI_ERR_INVALID_ARGUMENT, "workspace must not overlap y");
    }
    bi_status_t st = check_run_device(h);
    if (st != BI_OK)
        return st;
    hipError_t e = bigemm::launch_splitk(h->plan, kind, splits, h->W, x, M, y, workspace,
                                         static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(BI_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
    return BI_OK;
}

bi_status_t bi_rmsnorm_gemm_run(bi_gemm_t hh, const void* x, const void* gain, float eps, int M, float* rstd,
                                float* y, void* stream)
{
    bi_gemm* h = handle_of(hh);
    if (!h)
        return fail(BI_ERR_INVALID_ARGUMENT, "invalid handle");
    if (h->plan.experts != 0)
        return fail(BI_ERR_INVALID_ARGUMENT, "grouped handle passed to bi_rmsnorm_gemm_run");
    if (h->plan.k > 65536)
        return fail(BI_ERR_INVALID_ARGUMENT, "the normalised width K must be at most 65536");
    if (!std::isfinite(eps) || eps < 0.f)
        return fail(BI_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
    if (M < 0)
        return fail(BI_ERR_INVALID_ARGUMENT, "M must be >= 0");
    if (M == 0)
        return BI_OK;
    if (!x || !gain || !rstd || !y)
        return fail(BI_ERR_INVALID_ARGUMENT, "x, gain, rstd or y is NULL");
    if (!aligned16(x) || !aligned16(gain) || !aligned16(y) || (reinterpret_cast<uintptr_t>(rstd) & 3u) != 0)
        return fail(BI_ERR_MISALIGNED, "x, gain and y must be 16-byte aligned, rstd 4-byte aligned");
    const long long wide = h->plan.n > h->plan.k ? h->plan.n : h->plan.k;
    if ((long long)M * wide >= (1LL << 31))
        return fail(BI_ERR_INVALID_ARGUMENT, "M*max(N,K) must be below 2^31");
    const char* yb = reinterpret_cast<const char*>(y);
    const char* xb = static_cast<const char*>(x);
    const char* rb = reinterpret_cast<const char*>(rstd);
    const size_t ybytes = (size_t)M * h->plan.n * 4, xbytes = (size_t)M * h->plan.k * 2, rbytes = (size_t)M * 4;
    if ((xb < yb + ybytes && yb < xb + xbytes) || (rb < yb + ybytes && yb < rb + rbytes) ||
        (rb < xb + xbytes && xb < rb + rbytes))
        return fail(BI_ERR_INVALID_ARGUMENT, "y, x and rstd must not overlap");
    bi_status_t st = check_run_device(h);
    if (st != BI_OK)
        return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = binorm::launch_rstd(x, M, h->plan.k, eps, rstd, s);
    if (e == hipSuccess)
        e = bigemm::launch_dense_norm(h->plan, h->W, x, rstd, gain, M, y, s);
    if (e != hipSuccess)
        return fail(BI_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
    return BI_OK;
}

const char* bi_rmsnorm_gemm_kernel_name(bi_gemm_t hh, int M)
{
    bi_gemm* h = handle_of(hh);
    if (!h || M <= 0 || h->plan.experts != 0)
        return "";
    return bigemm::dense_norm_kernel_name(h->plan, M);
}

namespace {

// y: the product (fp32 [R, N]); or, for a gated handle, a: the product with
// SwiGLU applied (bf16 [R, N / 2]), y then NULL, with max_rows the caller's
// bound on any expert's rows (grouped_swiglu_fits).
bi_status_t grouped_run(bi_gemm_t hh, const void* x, int xn, const int32_t* xidx, const int32_t* expert_offsets,
                        int R, float* y, void* stream, void* a = nullptr, int max_rows = 1 << 30)
{
    bi_gemm* h = handle_of(hh);
    if (!h)
        return fail(BI_ERR_INVALID_ARGUMENT, "invalid handle");
    if (h->plan.experts == 0)
        return fail(BI_ERR_INVALID_ARGUMENT, "dense handle passed to bi_grouped_gemm_run");
    if (a && (h->plan.gated_i == 0 || !bigemm::grouped_swiglu_fits(h->plan, R, max_rows)))
        return fail(BI_ERR_INVALID_ARGUMENT, "the fused SwiGLU needs a gated handle and a call it fits");
    if (R < 0)
        return fail(BI_ERR_INVALID_ARGUMENT, "R must be >= 0");
    if (R == 0)
        return BI_OK;
    void* out = a ? a : static_cast<void*>(y);
    if (!x || !out || !expert_offsets)
        return fail(BI_ERR_INVALID_ARGUMENT, "x, y or expert_offsets is NULL");
    if (!aligned16(x) || !aligned16(out))
        return fail(BI_ERR_MISALIGNED, "x and y must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(expert_offsets) & 3u) != 0)
        return fail(BI_ERR_MISALIGNED, "expert_offsets must be 4-byte aligned");
    const long long wide = h->plan.n > h->plan.k ? h->plan.n : h->plan.k;
    if ((long long)R * wide >= (1LL << 31))
        return fail(BI_ERR_INVALID_ARGUMENT, "R*max(N,K) must be below 2^31");
    if (xidx) {
        if (xn < 1 || (long long)xn * h->plan.k >= (1LL << 31))
            return fail(BI_ERR_INVALID_ARGUMENT, "need 1 <= x_rows and x_rows*K below 2^31");
        if ((reinterpret_cast<uintptr_t>(xidx) & 3u) != 0)
            return fail(BI_ERR_MISALIGNED, "row_index must be 4-byte aligned");
    }
    bi_status_t st = check_run_device(h);
    if (st != BI_OK)
        return st;
    hipError_t e = a ? bigemm::launch_grouped_swiglu(h->plan, h->W, x, expert_offsets, R, a, xidx, xn, max_rows,
                                                     static_cast<hipStream_t>(stream))
                     : bigemm::launch_grouped(h->plan, h->W, x, expert_offsets, R, y, xidx, xn,
                                              static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(BI_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
    return BI_OK;
}

}  // namespace

bi_status_t bi_grouped_gemm_run(bi_gemm_t hh, const void* x, const int32_t* expert_offsets, int R,
                                float* y, void* stream)
{
    return grouped_run(hh, x, 0, nullptr, expert_offsets, R, y, stream);
}

bi_status_t bi_grouped_gemm_run_indexed(bi_gemm_t hh, const void* x, int x_rows, const int32_t* row_index,
                                        const int32_t* expert_offsets, int R, float* y, void* stream)
{
    if (R > 0 && !row_index)
        return fail(BI_ERR_INVALID_ARGUMENT, "row_index is NULL");
    return grouped_run(hh, x, x_rows, R > 0 ? row_index : nullptr, expert_offsets, R, y, stream);
}


void bi_gemm_destroy(bi_gemm_t hh)
{
    if (!hh)
        return;
    {
        std::lock_guard<std::mutex> g(g_live_mu);
        if (g_live.erase(hh) == 0)
            return;
    }
    hh->magic = 0;
    // hipFree waits for the device work that may still read the weights; it
    // runs with the handle's device current
    int cur = -1;
    const bool switched = hipGetDevice(&cur) == hipSuccess && cur != hh->device &&
                          hipSetDevice(hh->device) == hipSuccess;
    (void)hipFree(hh->W);
    (void)hipFree(hh->split_ws);
    if (switched)
        (void)hipSetDevice(cur);
    delete hh;
}

bi_status_t bi_gemm_get_pin(bi_gemm_t hh, bi_pin_info* out)
{
    bi_gemm* h = handle_of(hh);
    if (!h)
        return fail(BI_ERR_INVALID_ARGUMENT, "invalid handle");
    if (!out)
        return fail(BI_ERR_INVALID_ARGUMENT, "out is NULL");
    *out = h->pin;
    return BI_OK;
}

const char* bi_gemm_kernel_name(bi_gemm_t hh, int M)
{
    bi_gemm* h = handle_of(hh);
    if (!h || M <= 0)
        return "";
    if (h->plan.experts != 0)
        return bigemm::grouped_kernel_name(h->plan, M);
    const bigemm::DenseKernel k = bigemm::choose_dense(h->plan, M);
    return bigemm::concurrent_splits(h->plan, M) ? bigemm::dense_kernel_name_cs(k) : bigemm::dense_kernel_name(k);
}

const char* bi_status_string(bi_status_t s)
{
    switch (s) {
    case BI_OK: return "success";
    case BI_ERR_INVALID_ARGUMENT: return "invalid argument";
    case BI_ERR_MISALIGNED: return "misaligned pointer";
    case BI_ERR_NO_PIN: return "no pin for this shape (strict mode)";
    case BI_ERR_UNSUPPORTED_DEVICE: return "unsupported device (gfx950 only)";
    case BI_ERR_OUT_OF_MEMORY: return "out of memory";
    case BI_ERR_HIP: return "HIP runtime error";
    case BI_ERR_BAD_PIN_TABLE: return "malformed pin table";
    }
    return "unknown status";
}

const char* bi_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

namespace bigemm {

bi_status_t create_gated(int E, int I, int K, const void* W, bi_gemm_t* out)
{
    if (E <= 0 || I <= 0 || I % 16 != 0 || (long long)E * 2 * I * K >= (1LL << 40)) {
        if (out)
            *out = nullptr;
        return fail(BI_ERR_INVALID_ARGUMENT, "gated up projection: need E >= 1, I a multiple of 16");
    }
    return create_common(E, 2 * I, K, W, nullptr, out, I);
}

bool swiglu_fits(bi_gemm_t hh, int R, int max_rows)
{
    bi_gemm* h = handle_of(hh);
    return h && h->plan.gated_i > 0 && grouped_swiglu_fits(h->plan, R, max_rows);
}

bi_status_t run_swiglu_indexed(bi_gemm_t hh, const void* x, int x_rows, const int32_t* row_index,
                               const int32_t* expert_offsets, int R, int max_rows, void* a, void* stream)
{
    if (R > 0 && !row_index)
        return fail(BI_ERR_INVALID_ARGUMENT, "row_index is NULL");
    if (R > 0 && !a)
        return fail(BI_ERR_INVALID_ARGUMENT, "a is NULL");
    if (max_rows < 1)
        return fail(BI_ERR_INVALID_ARGUMENT, "max_rows must be >= 1");
    return grouped_run(hh, x, x_rows, R > 0 ? row_index : nullptr, expert_offsets, R, nullptr, stream, a, max_rows);
}

}  // namespace bigemm

