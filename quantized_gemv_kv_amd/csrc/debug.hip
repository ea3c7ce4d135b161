// debug.hip — a plain mat-vec on the canonical weight blocks, for checking a weight blob or a
// packed kernel against the format's definition.  One thread per output (row, batch row) walks
// the row's blocks in order, decodes each weight from its bytes exactly as the format defines it
// ("Chatterbox -> ggml Port: Development Journal", appendix A3 and §3.23: the legacy 32-weight
// blocks; "Every Frame Is a Memory Read", §3 and §5.8: affine groups of 64 or 32) and accumulates
// w * x in fp32 in K order.  It is deliberately simple and slow: no repacking, no LDS, no
// cross-lane work; the step's kernels never call it.
#include "model.h"

namespace tsd {
namespace {

__device__ __forceinline__ float half_at(const uint8_t* p)
{
    return __half2float(__ushort_as_half((unsigned short)(p[0] | (p[1] << 8))));
}

// weight k of row n, decoded from the canonical blob
__device__ float weight_at(int fmt, const uint8_t* w, int N, int K, int n, int k)
{
    const int blk = k / 32, j = k % 32;
    switch (fmt) {
    case TSD_W_Q4_0: {   // fp16 d, 16 bytes: element j < 16 low nibble of byte j, j + 16 its high nibble
        const uint8_t* b = w + ((size_t)n * (K / 32) + blk) * 18;
        const int q = j < 16 ? (b[2 + j] & 0xF) : (b[2 + j - 16] >> 4);
        return (float)(q - 8) * half_at(b);
    }
    case TSD_W_Q8_0: {   // fp16 d, 32 int8
        const uint8_t* b = w + ((size_t)n * (K / 32) + blk) * 34;
        return (float)(int8_t)b[2 + j] * half_at(b);
    }
    case TSD_W_Q5_0: {   // fp16 d, 32-bit word of fifth bits, 16 nibble bytes as Q4_0
        const uint8_t* b = w + ((size_t)n * (K / 32) + blk) * 22;
        const uint32_t hb = (uint32_t)b[2] | ((uint32_t)b[3] << 8) | ((uint32_t)b[4] << 16) | ((uint32_t)b[5] << 24);
        const int lo = j < 16 ? (b[6 + j] & 0xF) : (b[6 + j - 16] >> 4);
        const int q = lo | (int)((hb >> j) & 1u) << 4;
        return (float)(q - 16) * half_at(b);
    }
    case TSD_W_AFFINE8_G64: {   // planar q[N][K] bytes, s[N][K/64], b[N][K/64] fp16
        const size_t G = K / 64;
        const uint8_t* s = w + (size_t)N * K;
        const uint8_t* bb = s + (size_t)N * G * 2;
        const size_t g = (size_t)n * G + k / 64;
        return fmaf(half_at(s + 2 * g), (float)w[(size_t)n * K + k], half_at(bb + 2 * g));
    }
    default: {   // 4-bit affine: q[N][K/2] (element 2i low nibble of byte i), s, b per group of G
        const int gs = fmt == TSD_W_AFFINE4_G64 ? 64 : 32;
        const size_t G = K / gs;
        const uint8_t* s = w + (size_t)N * K / 2;
        const uint8_t* bb = s + (size_t)N * G * 2;
        const size_t g = (size_t)n * G + k / gs;
        const uint8_t byte = w[(size_t)n * (K / 2) + k / 2];
        const int q = (k & 1) ? byte >> 4 : byte & 0xF;
        return fmaf(half_at(s + 2 * g), (float)q, half_at(bb + 2 * g));
    }
    }
}

__global__ void k_debug_gemv(int fmt, const uint8_t* __restrict__ w, const float* __restrict__ x, float* __restrict__ y,
                             int N, int K, int B)
{
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (long long)N * B) return;
    const int b = (int)(i / N), n = (int)(i - (long long)b * N);
    float acc = 0.f;
    for (int k = 0; k < K; ++k) acc = fmaf(weight_at(fmt, w, N, K, n, k), x[(size_t)b * K + k], acc);
    y[(size_t)b * N + n] = acc;
}

}  // namespace
}  // namespace tsd

using namespace tsd;

extern "C" tsd_status tsd_debug_gemv(int wfmt, const void* d_w, size_t w_bytes, const float* d_x, float* d_y, int N, int K,
                                     int B, void* stream)
{
    if (!d_w || !d_x || !d_y) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "null buffer");
    if (wfmt < 0 || wfmt >= FMT_COUNT) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "unknown weight format");
    if (N <= 0 || K <= 0 || B <= 0) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "N, K and B must be positive");
    if (K % group_of(wfmt)) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "K must be a multiple of the format's group");
    if (w_bytes != canonical_matrix_bytes(wfmt, N, K))
        return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "w_bytes does not match the canonical size of an N x K matrix");
    const long long n = (long long)N * B;
    hipLaunchKernelGGL(k_debug_gemv, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream, wfmt,
                       (const uint8_t*)d_w, d_x, d_y, N, K, B);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(nullptr, e, "debug gemv launch");
    return TSD_OK;
}
