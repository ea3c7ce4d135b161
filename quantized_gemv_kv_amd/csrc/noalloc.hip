// noalloc.hip — the split-KV flash-decode attention for callers that cannot allocate device
// memory (code under HIP graph capture, serving loops that forbid allocation): the same kernels as
// tsd_attention, with the per-chunk partials in a fixed array that lives in the library's device
// image instead of a caller-provided scratch buffer.
//
// The array is a file-scope __device__ variable, so every GPU the library runs on holds its own
// copy (TSD_NOALLOC_SCRATCH_BYTES) until the process ends.  In host code its name is only a
// stand-in: its device address on each GPU is looked up once, with that GPU current, through
// hipGetSymbolAddress, and only that address is ever handed to a kernel.  Every call on one GPU
// shares the array, so calls that overlap on one GPU (different streams, or threads) race; the
// partials are fully rewritten by each call before they are read, so nothing needs clearing.
#include <mutex>

#include "model.h"

namespace tsd {
namespace {

__device__ __align__(256) unsigned char scratch[TSD_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_ptr[MAX_DEVICES] = {};

// the array's device address on the current GPU (looked up on the first call on that GPU)
hipError_t scratch_ptr(void** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace
}  // namespace tsd

using namespace tsd;

extern "C" tsd_status tsd_attention_noalloc(const float* d_q, const uint16_t* d_k, const uint16_t* d_v, int B, int H,
                                            int Hkv, int hd, int n_keys, int n_ctx, float* d_out, void* stream)
{
    size_t need = 0;
    tsd_status s = tsd_attention_scratch_bytes(B, H, n_ctx, hd, &need);
    if (s != TSD_OK) return s;
    if (need > TSD_NOALLOC_SCRATCH_BYTES)
        return fail(nullptr, TSD_ERR_INVALID_ARGUMENT,
                    "the partials of this shape need " + std::to_string(need) + " bytes, more than the " +
                        std::to_string((size_t)TSD_NOALLOC_SCRATCH_BYTES) + " the library holds per GPU");
    if (Hkv <= 0 || H % Hkv || n_keys < 1 || n_keys > n_ctx) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "bad shape");
    if (!d_q || !d_k || !d_v || !d_out) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "null buffer");
    void* part = nullptr;
    hipError_t e = scratch_ptr(&part);
    if (e != hipSuccess) return hip_fail(nullptr, e, "scratch address");
    hipStream_t st = (hipStream_t)stream;
    AttnArgs a{};
    a.q = d_q;
    a.ldq = H * hd;
    a.k = (const __half*)d_k;
    a.v = (const __half*)d_v;
    a.out = d_out;
    a.ldo = H * hd;
    a.part = (float*)part;
    a.B = B;
    a.H = H;
    a.Hkv = Hkv;
    a.hd = hd;
    a.n_ctx = n_ctx;
    a.pos = nullptr;
    a.n_keys = n_keys;
    e = launch_attention(a, st);
    if (e == hipSuccess) e = launch_attention_merge(a, n_keys, st);
    return e == hipSuccess ? TSD_OK : hip_fail(nullptr, e, "attention");
}
