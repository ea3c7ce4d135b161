// sampler.hip — the top-k draw as its own one-workgroup kernel: the sampler of the per-operator
// step (after the head GEMV) and the standalone tsd_sample_topk.  The draw itself is sampler.h.
#include "kernels.h"
#include "sampler.h"

namespace tsd {
namespace {

constexpr int NT = 256;

// logits[0..n) -> id.  The position of the counter is *posp (the step's device position) or
// pos_value; with hist, the id is also appended at hist[pos * hist_stride] and *posp advanced.
__global__ __launch_bounds__(NT) void k_topk(const float* __restrict__ logits, int n, int k, float temperature,
                                             unsigned long long seed, int row, int pass, int* posp, int pos_value,
                                             int* out, int* hist, int hist_stride)
{
    extern __shared__ uint32_t keys[];
    __shared__ samp::Scratch S;
    for (int i = threadIdx.x; i < n; i += NT) keys[i] = float_order_key(logits[i]);
    __syncthreads();
    const int pos = posp ? *posp : pos_value;
    const float u = samp::uniform24(seed, (uint32_t)row, (uint32_t)pos, (uint32_t)pass);
    const int id = samp::topk_draw<NT>(keys, n, k, temperature, u, S);
    if (threadIdx.x == 0) {
        out[0] = id;
        if (hist) {
            hist[(size_t)pos * hist_stride] = id;
            *posp = pos + 1;
        }
    }
}

}  // namespace

size_t topk_lds_bytes(int n) { return (size_t)n * sizeof(uint32_t); }

bool topk_supported(int n, int k) { return n > 0 && k >= 1 && k <= n && k <= samp::KMAX && topk_lds_bytes(n) + sizeof(samp::Scratch) <= 64 * 1024; }

hipError_t launch_topk(const float* logits, int n, int k, float temperature, unsigned long long seed, int row, int pass,
                       int* posp, int pos_value, int* out, int* hist, int hist_stride, hipStream_t st)
{
    if (!topk_supported(n, k)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_topk, dim3(1), dim3(NT), topk_lds_bytes(n), st, logits, n, k, temperature, seed, row, pass, posp,
                       pos_value, out, hist, hist_stride);
    return hipGetLastError();
}

}  // namespace tsd
