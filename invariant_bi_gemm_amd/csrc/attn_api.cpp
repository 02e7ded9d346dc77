// Host side of batch-invariant decode attention: the handle and its split
// workspace, argument checks, launches.  Every check runs before any HIP
// call and a failure launches nothing (Detent, §5).

#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>
#include <new>
#include <string>
#include <unordered_set>

#include "../../include/bi_attn.h"
#include "attn_internal.h"
#include "bigemm_internal.h"

using bigemm::api_fail;

struct bi_attn {
    uint32_t magic;
    int device;
    int Hq, Hkv, D, S, max_batch, max_len;
    biattn::Workspace ws;
    void* mem;
};

namespace {

constexpr uint32_t kAttnMagic = 0xB1A77E11u;
std::mutex g_mu;
std::unordered_set<const bi_attn*> g_live;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bi_attn* attn_of(bi_attn_t h)
{
    if (!h)
        return nullptr;
    std::lock_guard<std::mutex> g(g_mu);
    if (g_live.find(h) == g_live.end())
        return nullptr;
    return h->magic == kAttnMagic ? h : nullptr;
}

}  // namespace

extern "C" {

bi_status_t bi_attn_create(int Hq, int Hkv, int D, int split, int max_batch, int max_seq_len, bi_attn_t* out)
{
    if (!out)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "out is NULL");
    *out = nullptr;
    if (D != biattn::kHeadDim)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "the head dimension must be 128");
    if (Hkv < 1 || Hq < Hkv || Hq % Hkv != 0)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "need Hkv >= 1 and Hq a multiple of Hkv");
    const int G = Hq / Hkv;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "Hq / Hkv must be 1, 2, 4 or 8");
    if (split < 64 || split > 16384 || split % 64 != 0)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "the split size must be a multiple of 64 within 64..16384");
    // the kernel addresses one split's keys of a kv head with 32-bit offsets
    if ((long long)split * Hkv * D * 2 >= (1LL << 32))
        return api_fail(BI_ERR_INVALID_ARGUMENT, "split * Hkv * D * 2 bytes must stay below 4 GiB");
    if (max_batch < 1 || max_batch > 65535 || max_seq_len < 1 || max_seq_len > (1 << 24))
        return api_fail(BI_ERR_INVALID_ARGUMENT, "need 1 <= max_batch <= 65535 and 1 <= max_seq_len <= 2^24");
    const long long splits = (max_seq_len + (long long)split - 1) / split;
    const long long entries = (long long)max_batch * Hq * splits;
    if (entries * (D + 2) >= (1LL << 40) / 4)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "workspace too large");
    int dev, cus;
    bi_status_t st = bigemm::api_device(&dev, &cus);
    if (st != BI_OK)
        return st;
    bi_attn* h = new (std::nothrow) bi_attn();
    if (!h)
        return api_fail(BI_ERR_OUT_OF_MEMORY, "out of host memory");
    h->magic = kAttnMagic;
    h->device = dev;
    h->Hq = Hq;
    h->Hkv = Hkv;
    h->D = D;
    h->S = split;
    h->max_batch = max_batch;
    h->max_len = max_seq_len;
    const size_t bytes_o = (size_t)entries * D * sizeof(float);
    const size_t bytes_ml = (size_t)entries * 2 * sizeof(float);
    const size_t bytes = bytes_o + bytes_ml + (size_t)(max_batch + 2) * sizeof(int);
    const hipError_t e = hipMalloc(&h->mem, bytes);
    if (e != hipSuccess) {
        delete h;
        return api_fail(BI_ERR_OUT_OF_MEMORY, (std::string("hipMalloc of the split workspace: ") +
                                               hipGetErrorString(e)).c_str());
    }
    h->ws.o = static_cast<float*>(h->mem);
    h->ws.ml = reinterpret_cast<float*>(static_cast<char*>(h->mem) + bytes_o);
    h->ws.plan = reinterpret_cast<int*>(static_cast<char*>(h->mem) + bytes_o + bytes_ml);
    h->ws.splits = (int)splits;
    h->ws.num_cus = cus;
    try {
        std::lock_guard<std::mutex> g(g_mu);
        g_live.insert(h);
    } catch (...) {
        (void)hipFree(h->mem);
        delete h;
        return api_fail(BI_ERR_OUT_OF_MEMORY, "out of host memory");
    }
    *out = h;
    return BI_OK;
}

bi_status_t bi_attn_decode(bi_attn_t hh, const void* q, const void* k, const void* v, const int32_t* seq_start,
                           int B, int Ntok, float scale, float* out, void* stream)
{
    bi_attn* h = attn_of(hh);
    if (!h)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "invalid attention handle");
    if (B < 0 || B > h->max_batch)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "need 0 <= B <= max_batch");
    if (Ntok < 0)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "need Ntok >= 0");
    if (!std::isfinite(scale))
        return api_fail(BI_ERR_INVALID_ARGUMENT, "scale must be finite");
    if (B == 0)
        return BI_OK;
    if (!q || !seq_start || !out || (Ntok > 0 && (!k || !v)))
        return api_fail(BI_ERR_INVALID_ARGUMENT, "a pointer is NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        (reinterpret_cast<uintptr_t>(seq_start) & 3) != 0)
        return api_fail(BI_ERR_MISALIGNED, "q, k, v and out must be 16-byte aligned, seq_start 4-byte");
    int dev;
    if (hipGetDevice(&dev) != hipSuccess || dev != h->device)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "the current device is not the handle's device");
    const hipError_t e = biattn::launch_decode(q, k, v, seq_start, B, h->Hq, h->Hkv, h->S, h->max_len, Ntok,
                                               scale, h->ws, out, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return api_fail(BI_ERR_HIP, (std::string("kernel launch: ") + hipGetErrorString(e)).c_str());
    return BI_OK;
}

}  // extern "C"

// ---- allocation-free variant ------------------------------------------------
// The split partials and the work list of bi_attn_decode_noalloc live in one
// file-scope device array per GPU (each device holds its own copy for as long
// as the process runs).  Host code never passes the array's name to a kernel
// or a copy: in host code it stands for the host-side shadow, not a device
// address.  The device address comes from hipGetSymbolAddress, once per
// device with that device current, and is kept here.
namespace {

static __device__ __align__(256) unsigned char scratch[BI_ATTN_NOALLOC_SCRATCH_BYTES];

struct ScratchSlot {
    std::once_flag once;
    void* ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[64];

// The calling thread's current device's copy of `scratch` (its device
// address), or an error.
bi_status_t scratch_of_device(int dev, void** out)
{
    if (dev < 0 || dev >= 64)
        return api_fail(BI_ERR_UNSUPPORTED_DEVICE, "device index out of range");
    ScratchSlot& s = g_scratch[dev];
    std::call_once(s.once, [&] { s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch)); });
    if (s.err != hipSuccess || !s.ptr)
        return api_fail(BI_ERR_HIP, (std::string("hipGetSymbolAddress of the attention scratch: ") +
                                     hipGetErrorString(s.err)).c_str());
    *out = s.ptr;
    return BI_OK;
}

}  // namespace

extern "C" {

bi_status_t bi_attn_decode_noalloc(int Hq, int Hkv, int D, int split, int max_seq_len, const void* q, const void* k,
                                   const void* v, const int32_t* seq_start, int B, int Ntok, float scale, float* out,
                                   void* stream)
{
    if (D != biattn::kHeadDim)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "the head dimension must be 128");
    if (Hkv < 1 || Hq < Hkv || Hq % Hkv != 0)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "need Hkv >= 1 and Hq a multiple of Hkv");
    const int G = Hq / Hkv;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "Hq / Hkv must be 1, 2, 4 or 8");
    if (split < 64 || split > 16384 || split % 64 != 0)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "the split size must be a multiple of 64 within 64..16384");
    if ((long long)split * Hkv * D * 2 >= (1LL << 32))
        return api_fail(BI_ERR_INVALID_ARGUMENT, "split * Hkv * D * 2 bytes must stay below 4 GiB");
    if (max_seq_len < 1 || max_seq_len > (1 << 24))
        return api_fail(BI_ERR_INVALID_ARGUMENT, "need 1 <= max_seq_len <= 2^24");
    if (B < 0 || B > 65535 || Ntok < 0)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "need 0 <= B <= 65535 and Ntok >= 0");
    if (!std::isfinite(scale))
        return api_fail(BI_ERR_INVALID_ARGUMENT, "scale must be finite");
    const long long splits = (max_seq_len + (long long)split - 1) / split;
    const long long entries = (long long)B * Hq * splits;
    const long long need = entries * (D + 2) * (long long)sizeof(float) + (long long)(B + 2) * (long long)sizeof(int);
    if (need > (long long)BI_ATTN_NOALLOC_SCRATCH_BYTES)
        return api_fail(BI_ERR_INVALID_ARGUMENT,
                        ("the split partials need " + std::to_string(need) + " bytes, beyond the " +
                         std::to_string((long long)BI_ATTN_NOALLOC_SCRATCH_BYTES) +
                         "-byte scratch of the allocation-free entry point (B * Hq * ceil(max_seq_len / split) "
                         "* (D + 2) * 4 + (B + 2) * 4)").c_str());
    if (B == 0)
        return BI_OK;
    if (!q || !seq_start || !out || (Ntok > 0 && (!k || !v)))
        return api_fail(BI_ERR_INVALID_ARGUMENT, "a pointer is NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        (reinterpret_cast<uintptr_t>(seq_start) & 3) != 0)
        return api_fail(BI_ERR_MISALIGNED, "q, k, v and out must be 16-byte aligned, seq_start 4-byte");
    int dev, cus;
    bi_status_t st = bigemm::api_device(&dev, &cus);
    if (st != BI_OK)
        return st;
    void* base = nullptr;
    st = scratch_of_device(dev, &base);
    if (st != BI_OK)
        return st;
    biattn::Workspace ws;
    const size_t bytes_o = (size_t)entries * D * sizeof(float);
    const size_t bytes_ml = (size_t)entries * 2 * sizeof(float);
    ws.o = static_cast<float*>(base);
    ws.ml = reinterpret_cast<float*>(static_cast<char*>(base) + bytes_o);
    ws.plan = reinterpret_cast<int*>(static_cast<char*>(base) + bytes_o + bytes_ml);
    ws.splits = (int)splits;
    ws.num_cus = cus;
    const hipError_t e = biattn::launch_decode(q, k, v, seq_start, B, Hq, Hkv, split, max_seq_len, Ntok, scale, ws,
                                               out, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return api_fail(BI_ERR_HIP, (std::string("kernel launch: ") + hipGetErrorString(e)).c_str());
    return BI_OK;
}

void bi_attn_destroy(bi_attn_t hh)
{
    bi_attn* h = attn_of(hh);
    if (!h)
        return;
    {
        std::lock_guard<std::mutex> g(g_mu);
        g_live.erase(h);
    }
    h->magic = 0;
    (void)hipFree(h->mem);
    delete h;
}

}  // extern "C"
