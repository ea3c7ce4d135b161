// sampler.hip — the sampler chain as its own one-workgroup kernel: the sampler of the
// per-operator step (after the head GEMV) and the standalone tsd_sample / tsd_sample_topk.  The
// draw itself is sampler.h.
#include "kernels.h"
#include "sampler.h"

namespace tsd {
namespace {

constexpr int NT = 256;

// the classifier-free-guided logit of id i: cond + w (cond - uncond)
__device__ __forceinline__ float guided(const float* c, const float* u, float w, int i) { return fmaf(w, c[i] - u[i], c[i]); }

__global__ __launch_bounds__(NT) void k_sample(const SampleArgs a)
{
    extern __shared__ uint32_t lds[];   // keys [key_words(n)], then the history's bit set [(n + 31) / 32]
    __shared__ samp::Scratch S;
    const int n = a.n;
    uint32_t* keys = lds;
    uint32_t* seen = lds + samp::key_words(n);
    if (a.err && ld_uniform((const int*)a.err)) return;   // a rejected input: the state stays as it was
    const int pos = a.posp ? *a.posp : a.pos_value;   // read once: the position advances at the end
    const int rows = a.rows > 0 ? a.rows : 1;
    const bool pen = a.ch.penalty != 1.f;
    for (int r = 0; r < (a.cfg ? 1 : rows); ++r) {
        const int cur = a.cur ? a.cur[r] : -1;
        if (pen) samp::build_seen<NT>(seen, n, a.seq ? a.seq + r : nullptr, a.seq_stride, a.n_seq < 0 ? pos : a.n_seq, cur);
        const uint32_t* sp = pen ? seen : nullptr;
        const float* l = a.logits + (size_t)r * a.ld_logits;
        if (a.cfg) {
            for (int i = threadIdx.x; i < n; i += NT)
                keys[samp::key_at(i)] = samp::chain_key(guided(l, l + a.ld_logits, a.cfg_weight, i), i, a.ch, sp);
        } else {
            samp::load_keys<NT>(keys, l, n, a.ch, sp);
        }
        __syncthreads();
        const float u = samp::uniform24(a.seed, (uint32_t)(a.row + r), (uint32_t)pos, (uint32_t)a.pass);
        const int id = samp::chain_draw<NT>(keys, n, a.ch, u, S, sp);
        if (threadIdx.x == 0)
            for (int q = r; q < (a.cfg ? rows : r + 1); ++q) {   // guided: every row takes the id
                const int cq = a.cur ? a.cur[q] : -1;
                a.out[q] = id;
                if (a.posp) {
                    if (a.seq_out && a.cur) a.seq_out[(size_t)pos * a.seq_stride + q] = cq;
                    if (a.hist) a.hist[(size_t)pos * a.hist_stride + q] = id;
                }
            }
        __syncthreads();
    }
    if (threadIdx.x == 0 && a.posp) *a.posp = pos + 1;
}

}  // namespace

size_t sample_lds_bytes(int n)
{
    return (size_t)samp::key_words(n) * sizeof(uint32_t) + (size_t)((n + 31) / 32) * sizeof(uint32_t);
}

bool sample_supported(int n, int k)
{
    return n > 0 && k >= 1 && k <= n && k <= samp::KMAX && sample_lds_bytes(n) + sizeof(samp::Scratch) <= 64 * 1024;
}

hipError_t launch_sample(const SampleArgs& a, hipStream_t st)
{
    if (!sample_supported(a.n, a.ch.k) || !(a.ch.temperature > 0.f)) return hipErrorInvalidValue;
    if (a.rows > 1 && a.ld_logits < a.n) return hipErrorInvalidValue;
    if (a.cfg && a.rows != 2) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_sample, dim3(1), dim3(NT), sample_lds_bytes(a.n), st, a);
    return hipGetLastError();
}

}  // namespace tsd
