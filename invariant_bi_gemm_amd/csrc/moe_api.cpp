// Host side of the MoE expert layer: argument checks, the layer handle and
// its workspace, and the order of the steps.  As for the GEMM, every check
// runs before any HIP call and a failure launches nothing (Detent, §5).

#include <hip/hip_runtime.h>

#include <mutex>
#include <new>
#include <string>
#include <unordered_set>

#include "../../include/bi_moe.h"
#include "bigemm_internal.h"
#include "moe_internal.h"

namespace {

using bigemm::api_fail;

constexpr uint32_t kMoeMagic = 0xB1A0E5C7u;
constexpr long long kLim = 1LL << 31;

bool aligned(const void* p, unsigned a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bi_status_t launched(hipError_t e)
{
    if (e != hipSuccess)
        return api_fail(BI_ERR_HIP, (std::string("kernel launch: ") + hipGetErrorString(e)).c_str());
    return BI_OK;
}

bi_status_t device_ok()
{
    int dev, cus;
    return bigemm::api_device(&dev, &cus);
}

bi_status_t check_topk(const float* logits, int T, int E, int k, const int32_t* ids, const float* w)
{
    if (T < 0 || E < 1 || E > bimoe::kMaxExperts)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "need T >= 0 and 1 <= E <= 1024");
    if (k < 1 || k > E || k > bimoe::kMaxTopK)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "need 1 <= k <= min(E, 64)");
    if ((long long)T * E >= kLim)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "T*E must be below 2^31");
    if (T > 0 && (!logits || !ids || !w))
        return api_fail(BI_ERR_INVALID_ARGUMENT, "a pointer is NULL");
    if (!aligned(logits, 4) || !aligned(ids, 4) || !aligned(w, 4))
        return api_fail(BI_ERR_MISALIGNED, "logits, ids and weights must be 4-byte aligned");
    return BI_OK;
}

bi_status_t check_permute(const int32_t* ids, int T, int E, int k, const int32_t* off,
                          const int32_t* tok, const int32_t* row_of)
{
    if (T < 0 || E < 1 || E > bimoe::kMaxExperts || k < 1 || k > bimoe::kMaxTopK)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "need T >= 0, 1 <= E <= 1024 and 1 <= k <= 64");
    if ((long long)T * k >= kLim)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "T*k must be below 2^31");
    if (!off || (T > 0 && (!ids || !tok || !row_of)))
        return api_fail(BI_ERR_INVALID_ARGUMENT, "a pointer is NULL");
    if (!aligned(ids, 4) || !aligned(off, 4) || !aligned(tok, 4) || !aligned(row_of, 4))
        return api_fail(BI_ERR_MISALIGNED, "ids, offsets, token_of_row and row_of must be 4-byte aligned");
    return BI_OK;
}

bi_status_t check_gather(const void* src, int nsrc, const int32_t* idx, int R, int K, const void* dst)
{
    if (nsrc < 0 || R < 0 || K <= 0 || K % 8 != 0)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "need nsrc >= 0, R >= 0 and K > 0 a multiple of 8");
    if ((long long)R * K >= kLim || (long long)nsrc * K >= kLim)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "R*K and nsrc*K must be below 2^31");
    if (R > 0 && (!idx || !dst || (nsrc > 0 && !src)))
        return api_fail(BI_ERR_INVALID_ARGUMENT, "a pointer is NULL");
    if (!aligned(src, 16) || !aligned(dst, 16) || !aligned(idx, 4))
        return api_fail(BI_ERR_MISALIGNED, "src and dst must be 16-byte aligned, idx 4-byte");
    return BI_OK;
}

bi_status_t check_swiglu(const float* h, int R, int I, const void* a)
{
    if (R < 0 || I <= 0 || I % 4 != 0)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "need R >= 0 and I > 0 a multiple of 4");
    if ((long long)R * 2 * I >= kLim)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "R*2I must be below 2^31");
    if (R > 0 && (!h || !a))
        return api_fail(BI_ERR_INVALID_ARGUMENT, "a pointer is NULL");
    if (!aligned(h, 16) || !aligned(a, 8))
        return api_fail(BI_ERR_MISALIGNED, "h must be 16-byte and a 8-byte aligned");
    return BI_OK;
}

bi_status_t check_combine(const float* o, int R, const int32_t* ids, const float* w,
                          const int32_t* row_of, int T, int k, int H, const float* y)
{
    if (R < 0 || T < 0 || k < 1 || k > bimoe::kMaxTopK || H <= 0 || H % 4 != 0)
        return api_fail(BI_ERR_INVALID_ARGUMENT,
                        "need R >= 0, T >= 0, 1 <= k <= 64 and H > 0 a multiple of 4");
    if ((long long)R * H >= kLim || (long long)T * H >= kLim || (long long)T * k >= kLim)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "R*H, T*H and T*k must be below 2^31");
    if (T > 0 && (!ids || !w || !row_of || !y || (R > 0 && !o)))
        return api_fail(BI_ERR_INVALID_ARGUMENT, "a pointer is NULL");
    if (!aligned(o, 16) || !aligned(y, 16) || !aligned(ids, 4) || !aligned(w, 4) || !aligned(row_of, 4))
        return api_fail(BI_ERR_MISALIGNED, "o and y must be 16-byte aligned, the rest 4-byte");
    return BI_OK;
}

}  // namespace

struct bi_moe {
    uint32_t magic;
    int device;
    int E, k, H, I, max_tokens;
    bi_gemm_t router, up, down;
    void* ws;  // one allocation, carved below
    float* logits;
    int32_t* ids;
    float* w;
    int32_t* offsets;
    int32_t* tok;
    int32_t* row_of;
    float* h;  // fp32 [maxT*k, 2I]
    void* a;   // bf16 [maxT*k, I]
    float* o;  // fp32 [maxT*k, H]
};

namespace {

std::mutex g_moe_mu;
std::unordered_set<const bi_moe*> g_moe_live;

bi_moe* moe_of(bi_moe_t h)
{
    if (!h)
        return nullptr;
    std::lock_guard<std::mutex> g(g_moe_mu);
    if (g_moe_live.find(h) == g_moe_live.end())
        return nullptr;
    return h->magic == kMoeMagic ? h : nullptr;
}

void release(bi_moe* m)
{
    bi_gemm_destroy(m->router);
    bi_gemm_destroy(m->up);
    bi_gemm_destroy(m->down);
    if (m->ws)
        (void)hipFree(m->ws);
    delete m;
}

}  // namespace

extern "C" {

bi_status_t bi_moe_topk(const float* logits, int T, int E, int k, int32_t* ids, float* weights,
                        void* stream)
{
    bi_status_t st = check_topk(logits, T, E, k, ids, weights);
    if (st != BI_OK || T == 0)
        return st;
    if ((st = device_ok()) != BI_OK)
        return st;
    return launched(bimoe::launch_topk(logits, T, E, k, ids, weights, static_cast<hipStream_t>(stream)));
}

bi_status_t bi_moe_permute(const int32_t* ids, int T, int E, int k, int32_t* offsets,
                           int32_t* token_of_row, int32_t* row_of, void* stream)
{
    bi_status_t st = check_permute(ids, T, E, k, offsets, token_of_row, row_of);
    if (st != BI_OK)
        return st;
    if ((st = device_ok()) != BI_OK)
        return st;
    return launched(bimoe::launch_permute(ids, T, E, k, offsets, token_of_row, row_of,
                                          static_cast<hipStream_t>(stream)));
}

bi_status_t bi_gather_rows(const void* src, int nsrc, const int32_t* idx, int R, int K, void* dst,
                           void* stream)
{
    bi_status_t st = check_gather(src, nsrc, idx, R, K, dst);
    if (st != BI_OK || R == 0)
        return st;
    if ((st = device_ok()) != BI_OK)
        return st;
    return launched(bimoe::launch_gather(src, nsrc, idx, R, K, dst, static_cast<hipStream_t>(stream)));
}

bi_status_t bi_swiglu(const float* h, int R, int I, void* a, void* stream)
{
    bi_status_t st = check_swiglu(h, R, I, a);
    if (st != BI_OK || R == 0)
        return st;
    if ((st = device_ok()) != BI_OK)
        return st;
    return launched(bimoe::launch_swiglu(h, R, I, a, static_cast<hipStream_t>(stream)));
}

bi_status_t bi_moe_combine(const float* o, int R, const int32_t* ids, const float* weights,
                           const int32_t* row_of, int T, int k, int H, float* y, void* stream)
{
    bi_status_t st = check_combine(o, R, ids, weights, row_of, T, k, H, y);
    if (st != BI_OK || T == 0)
        return st;
    if ((st = device_ok()) != BI_OK)
        return st;
    return launched(bimoe::launch_combine(o, R, ids, weights, row_of, T, k, H, y,
                                          static_cast<hipStream_t>(stream)));
}

bi_status_t bi_moe_create(int E, int k, int H, int I, const void* W_router, const void* W_up,
                          const void* W_down, int max_tokens, bi_moe_t* out)
{
    if (!out)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "out is NULL");
    *out = nullptr;
    if (E < 16 || E > bimoe::kMaxExperts || E % 16 != 0)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "E must be a multiple of 16 within 16..1024");
    if (k < 1 || k > E || k > bimoe::kMaxTopK)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "need 1 <= k <= min(E, 64)");
    if (H <= 0 || H % 64 != 0 || I <= 0 || I % 64 != 0)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "H and I must be positive multiples of 64");
    const long long rows = (long long)max_tokens * k;
    if (max_tokens < 1 || rows * (H > 2 * I ? H : 2 * I) >= kLim || (long long)max_tokens * E >= kLim)
        return api_fail(BI_ERR_INVALID_ARGUMENT,
                        "need max_tokens >= 1 and max_tokens*k*max(H, 2I) below 2^31");
    if (!W_router || !W_up || !W_down)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "a weight pointer is NULL");
    int dev, cus;
    bi_status_t st = bigemm::api_device(&dev, &cus);
    if (st != BI_OK)
        return st;
    bi_moe* m = new (std::nothrow) bi_moe();
    if (!m)
        return api_fail(BI_ERR_OUT_OF_MEMORY, "out of host memory");
    m->magic = kMoeMagic;
    m->device = dev;
    m->E = E;
    m->k = k;
    m->H = H;
    m->I = I;
    m->max_tokens = max_tokens;
    if ((st = bi_gemm_create(E, H, W_router, &m->router)) != BI_OK ||
        (st = bigemm::create_gated(E, I, H, W_up, &m->up)) != BI_OK ||
        (st = bi_grouped_gemm_create(E, H, I, W_down, &m->down)) != BI_OK) {
        release(m);
        return st;
    }
    // workspace: each region rounded up to 256 bytes
    auto up256 = [](long long b) { return (b + 255) / 256 * 256; };
    const long long b_logits = up256((long long)max_tokens * E * 4);
    const long long b_pair = up256(rows * 4);
    const long long b_off = up256((long long)(E + 1) * 4);
    const long long b_h = up256(rows * 2 * I * 4);
    const long long b_a = up256(rows * I * 2);
    const long long b_o = up256(rows * H * 4);
    const long long total = b_logits + 4 * b_pair + b_off + b_h + b_a + b_o;
    hipError_t e = hipMalloc(&m->ws, (size_t)total);
    if (e != hipSuccess) {
        m->ws = nullptr;
        release(m);
        return api_fail(BI_ERR_OUT_OF_MEMORY, (std::string("hipMalloc of the layer workspace: ") +
                                               hipGetErrorString(e)).c_str());
    }
    char* p = static_cast<char*>(m->ws);
    m->logits = reinterpret_cast<float*>(p);
    p += b_logits;
    m->ids = reinterpret_cast<int32_t*>(p);
    p += b_pair;
    m->w = reinterpret_cast<float*>(p);
    p += b_pair;
    m->tok = reinterpret_cast<int32_t*>(p);
    p += b_pair;
    m->row_of = reinterpret_cast<int32_t*>(p);
    p += b_pair;
    m->offsets = reinterpret_cast<int32_t*>(p);
    p += b_off;
    m->h = reinterpret_cast<float*>(p);
    p += b_h;
    m->a = p;
    p += b_a;
    m->o = reinterpret_cast<float*>(p);
    try {
        std::lock_guard<std::mutex> g(g_moe_mu);
        g_moe_live.insert(m);
    } catch (...) {
        release(m);
        return api_fail(BI_ERR_OUT_OF_MEMORY, "out of host memory");
    }
    *out = m;
    return BI_OK;
}

bi_status_t bi_moe_run(bi_moe_t hh, const void* x, int T, float* y, void* stream)
{
    bi_moe* m = moe_of(hh);
    if (!m)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "invalid layer handle");
    if (T < 0 || T > m->max_tokens)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "need 0 <= T <= max_tokens");
    if (T == 0)
        return BI_OK;
    if (!x || !y)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "x or y is NULL");
    if (!aligned(x, 16) || !aligned(y, 16))
        return api_fail(BI_ERR_MISALIGNED, "x and y must be 16-byte aligned");
    int dev;
    if (hipGetDevice(&dev) != hipSuccess || dev != m->device)
        return api_fail(BI_ERR_INVALID_ARGUMENT, "the current device is not the layer's device");
    const int R = T * m->k;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    bi_status_t st;
    if ((st = bi_gemm_run(m->router, x, T, m->logits, stream)) != BI_OK)
        return st;
    // routing and grouping: one launch for a few tokens (T = 1: 44 -> 41 us
    // per layer call; at T = 16 the two launches were 1 us faster), else two
    if (T <= bimoe::kRouteMaxTokens) {
        if ((st = launched(bimoe::launch_route(m->logits, T, m->E, m->k, m->ids, m->w, m->offsets, m->tok,
                                               m->row_of, s))) != BI_OK)
            return st;
    } else {
        if ((st = launched(bimoe::launch_topk(m->logits, T, m->E, m->k, m->ids, m->w, s))) != BI_OK)
            return st;
        if ((st = launched(bimoe::launch_permute(m->ids, T, m->E, m->k, m->offsets, m->tok, m->row_of, s))) !=
            BI_OK)
            return st;
    }
    // the up projection reads each row's token straight from x (no gathered
    // copy); its weights are packed gate/up interleaved, so that when every
    // expert runs in one kernel that holds a gate tile beside its up tile --
    // the streaming kernel over 32-row strips when no expert has more than 16
    // rows, the four-wave kernel when every expert takes its blocks -- the
    // epilogue applies SwiGLU and writes a directly (same bits as the product
    // then the SwiGLU kernel).  Top-k picks k distinct experts per token, so
    // no expert gets more than T rows.
    if (bigemm::swiglu_fits(m->up, R, T)) {
        if ((st = bigemm::run_swiglu_indexed(m->up, x, T, m->tok, m->offsets, R, T, m->a, stream)) != BI_OK)
            return st;
    } else {
        if ((st = bi_grouped_gemm_run_indexed(m->up, x, T, m->tok, m->offsets, R, m->h, stream)) != BI_OK)
            return st;
        if ((st = launched(bimoe::launch_swiglu(m->h, R, m->I, m->a, s, true))) != BI_OK)
            return st;
    }
    if ((st = bi_grouped_gemm_run(m->down, m->a, m->offsets, R, m->o, stream)) != BI_OK)
        return st;
    return launched(bimoe::launch_combine(m->o, R, m->ids, m->w, m->row_of, T, m->k, m->H, y, s));
}

void bi_moe_destroy(bi_moe_t hh)
{
    bi_moe* m = moe_of(hh);
    if (!m)
        return;
    {
        std::lock_guard<std::mutex> g(g_moe_mu);
        g_moe_live.erase(m);
    }
    m->magic = 0;
    release(m);
}

}  // extern "C"
