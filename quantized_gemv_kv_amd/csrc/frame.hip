// frame.hip — the batched operators of the Talker + code-predictor frame ("Every Frame Is a
// Memory Read", §1: a frame is one Talker step over the sum of 16 code embeddings, then 15
// sequential code-predictor passes; §3: 8-bit affine weights in groups of 64; §8: batches of
// rollouts, up to 16 rows here).
//
// With 16 rows every weight byte feeds 16 multiply-adds, a real (skinny) matrix product, so
// the linears run on the matrix cores (v_mfma_f32_16x16x32_f16) with fp32 accumulation, with
// the weights kept exact:
//   * a uint8 weight q enters the MFMA as the fp16 integer q - 128: a byte permute builds
//     1024 + q (bit pattern 0x6400 | q) for two weights at a time and one packed fp16 subtract
//     of 1152 centres them (centred weights keep the fp32 sums ~15x smaller than 1024 + q);
//   * an activation x enters as two fp16 numbers, hi = fp16(x) and lo = fp16(x - hi), two MFMAs
//     each, which carries about 22 bits of x;
//   * each group of 64 along K is scaled in fp32 after its MFMAs:
//       sum_k (s q_k + b) x_k = s P + (b + 128 s) X,   P = sum_k (q_k - 128) x_k,  X = sum_k x_k
//     with X computed once per row and group by the kernel that produced the operand.
// Operand roles: A = the 16 activation rows (lane l holds row l % 16), B = 16 weight rows (lane
// l holds row n0 + l % 16), so a lane's four results share one weight row and so one (s, b) per
// group.  Within a group, lane group j = l / 16 supplies K positions 16 j .. 16 j + 15 to two
// MFMAs (the same K permutation on both operands), i.e. one 16-byte load of weights per lane.
#include <math.h>

#include "gemv_core.h"
#include "kernels.h"

namespace tsd {
namespace {

using core::silu;

constexpr int NT = 256;
constexpr int PT = MM_MAX_K / NT;   // prep: elements per thread

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void put_hilo(const Act16& a, size_t idx, float y, float& sum)
{
    const _Float16 h = (_Float16)y;
    const _Float16 l = (_Float16)(y - (float)h);
    ((TSD_GLOBAL _Float16*)a.hi)[idx] = h;
    ((TSD_GLOBAL _Float16*)a.lo)[idx] = l;
    sum = (float)h + (float)l;
}

// ---- operand preparation: residual add, RMSNorm, fp16 hi/lo split, group sums --------------
// one workgroup per row; thread t holds elements t + 256 i, so wave w holds the whole group
// 4 i + w of its i-th element (K % 64 == 0): a group sum is a wave sum
__global__ __launch_bounds__(NT) void k_prep16(const PrepArgs p)
{
    const int b = blockIdx.x, t = threadIdx.x, K = p.K, G = K >> 6;
    TSD_GLOBAL float* xr = glb(p.x) + (size_t)b * p.ldx;
    __shared__ float red[NT / 64];
    float v[PT];
    float q2 = 0.f;
#pragma unroll
    for (int i = 0; i < PT; ++i) {
        const int k = t + i * NT;
        v[i] = 0.f;
        if (k < K) {
            float a = xr[k];
            for (int s = 0; s < p.n_part; ++s) a += glb(p.part)[((size_t)s * MM_ROWS + b) * p.ldx + k];
            if (p.n_part > 0) xr[k] = a;
            v[i] = a;
            q2 = fmaf(a, a, q2);
        }
    }
    float r = 1.f;
    if (p.g) {
        q2 = wave_sum(q2);
        if ((t & 63) == 0) red[t >> 6] = q2;
        __syncthreads();
        r = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)K + p.eps);
    }
#pragma unroll
    for (int i = 0; i < PT; ++i) {
        const int k0 = i * NT + (t & ~63);   // first element of this wave's group (uniform)
        if (k0 >= K) break;
        const int k = t + i * NT;
        const float y = p.g ? v[i] * r * glb(p.g)[k] : v[i];
        float s;
        put_hilo(p.a, (size_t)b * K + k, y, s);
        if (p.norm_out) glb(p.norm_out)[(size_t)b * K + k] = y;
        s = wave_sum(s);
        if ((t & 63) == 0) glb(p.a.gsum)[(size_t)b * G + (k0 >> 6)] = s;
    }
}

// ---- attention partials merged straight into the operand of the output projection ----------
// one 64-thread workgroup per group of 64 output elements (a head of 64 or half a head of 128)
__global__ __launch_bounds__(64) void k_merge_prep16(const float* __restrict__ part, int H, int hd, int max_split,
                                                     const int* posp, int n_keys_value, const Act16 a)
{
    const int e = blockIdx.x * 64 + threadIdx.x;
    const int i = e % hd, bh = e / hd, b = bh / H, h = bh - b * H;
    const int n_keys = posp ? ld_uniform(posp) + 1 : n_keys_value;
    const int n_split = (n_keys + ATTN_CHUNK - 1) / ATTN_CHUNK;
    const int PS = hd + 4;
    const TSD_GLOBAL float* pb = glb(part) + (size_t)bh * max_split * PS;
    float M = -INFINITY;
    for (int t = 0; t < n_split; ++t) M = fmaxf(M, pb[(size_t)t * PS + hd]);
    float L = 0.f, O = 0.f;
    for (int t = 0; t < n_split; ++t) {
        const float w = exp2f(pb[(size_t)t * PS + hd] - M);
        L = fmaf(pb[(size_t)t * PS + hd + 1], w, L);
        O = fmaf(pb[(size_t)t * PS + i], w, O);
    }
    const int K = H * hd;
    float s;
    put_hilo(a, (size_t)b * K + h * hd + i, O / L, s);
    s = wave_sum(s);
    if (threadIdx.x == 0) glb(a.gsum)[(size_t)b * (K >> 6) + ((h * hd + i) >> 6)] = s;
}

// ---- the skinny GEMM -------------------------------------------------------------------------
// byte q -> fp16 1024 + q for the four bytes of w: v_perm_b32 picks (q, 0x64) byte pairs
__device__ __forceinline__ void q4_to_h4(uint32_t w, uint32_t& lo2, uint32_t& hi2)
{
    lo2 = __builtin_amdgcn_perm(0x64646464u, w, 0x04010400u);   // (1024 + q0, 1024 + q1)
    hi2 = __builtin_amdgcn_perm(0x64646464u, w, 0x04030402u);   // (1024 + q2, 1024 + q3)
}
// bytes q of (w0, w1) -> the eight fp16 integers q - 128
__device__ __forceinline__ half8 q8_to_half8(uint32_t w0, uint32_t w1)
{
    u32x4 u;
    uint32_t a, b, c, d;
    q4_to_h4(w0, a, b);
    q4_to_h4(w1, c, d);
    u.x = a;
    u.y = b;
    u.z = c;
    u.w = d;
    return __builtin_bit_cast(half8, u) - (_Float16)1152.0f;   // q - 128, exact
}

constexpr int MM_U = 4;   // groups per wave whose loads are issued together

// Y = W X for the 16 operand rows: one workgroup per 16-row tile of W (blockIdx.x) and K slice
// (blockIdx.y of gridDim.y); the four waves take the slice's groups round robin, add their
// results in LDS, and wave 0 runs the epilogue.
template <int EPI>
__global__ __launch_bounds__(NT) void k_mm16(const PackedMat W, const Act16 a, const Mm16Out o)
{
    const int K = W.K, G = K >> 6, N = W.N;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, j = lane >> 4, c16 = lane & 15;
    const int n = blockIdx.x * 16 + c16;
    const int nl = n < N ? n : N - 1;   // rows past N load row N-1 and store nothing
    const int S = gridDim.y, sl = blockIdx.y;
    const int g_lo = (int)((long long)G * sl / S), g_hi = (int)((long long)G * (sl + 1) / S);
    const int gw = g_hi - g_lo > wave ? (g_hi - g_lo - wave + 3) >> 2 : 0;   // this wave's groups

    const TSD_GLOBAL uint8_t* wr = glb(W.q) + (size_t)nl * K + 16 * j;
    const TSD_GLOBAL _Float16* sr = (const TSD_GLOBAL _Float16*)glb(W.s) + (size_t)nl * G;
    const TSD_GLOBAL _Float16* br = (const TSD_GLOBAL _Float16*)glb(W.b) + (size_t)nl * G;
    const TSD_GLOBAL _Float16* ah = (const TSD_GLOBAL _Float16*)glb(a.hi) + (size_t)c16 * K + 16 * j;
    const TSD_GLOBAL _Float16* al = (const TSD_GLOBAL _Float16*)glb(a.lo) + (size_t)c16 * K + 16 * j;
    const TSD_GLOBAL float* gs = glb(a.gsum) + (size_t)(4 * j) * G;

    float4v acc = {0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < gw; c += MM_U) {
        u32x4 wq[MM_U];
        half8 h0[MM_U], h1[MM_U], l0[MM_U], l1[MM_U];
        float sc[MM_U], bi[MM_U], xs[MM_U][4];
#pragma unroll
        for (int u = 0; u < MM_U; ++u) {   // every load of the chunk first (clamped, masked below)
            const int gi = c + u < gw ? c + u : gw - 1;
            const int grp = g_lo + wave + 4 * gi, k0 = grp * 64;
            wq[u] = *(const TSD_GLOBAL u32x4*)(wr + k0);
            h0[u] = *(const TSD_GLOBAL half8*)(ah + k0);
            h1[u] = *(const TSD_GLOBAL half8*)(ah + k0 + 8);
            l0[u] = *(const TSD_GLOBAL half8*)(al + k0);
            l1[u] = *(const TSD_GLOBAL half8*)(al + k0 + 8);
            sc[u] = (float)sr[grp];
            bi[u] = (float)br[grp];
#pragma unroll
            for (int i = 0; i < 4; ++i) xs[u][i] = gs[(size_t)i * G + grp];
        }
#pragma unroll
        for (int u = 0; u < MM_U; ++u) {
            const half8 w0 = q8_to_half8(wq[u].x, wq[u].y), w1 = q8_to_half8(wq[u].z, wq[u].w);
            float4v pz = {0.f, 0.f, 0.f, 0.f};
            pz = __builtin_amdgcn_mfma_f32_16x16x32_f16(h0[u], w0, pz, 0, 0, 0);
            pz = __builtin_amdgcn_mfma_f32_16x16x32_f16(h1[u], w1, pz, 0, 0, 0);
            pz = __builtin_amdgcn_mfma_f32_16x16x32_f16(l0[u], w0, pz, 0, 0, 0);
            pz = __builtin_amdgcn_mfma_f32_16x16x32_f16(l1[u], w1, pz, 0, 0, 0);
            const bool valid = c + u < gw;
            const float s = valid ? sc[u] : 0.f;
            const float c0 = valid ? fmaf(128.f, sc[u], bi[u]) : 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = fmaf(s, pz[i], fmaf(c0, xs[u][i], acc[i]));
        }
    }

    __shared__ float4v red[3][64];
    if (wave > 0) red[wave - 1][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < 3; ++w) {
        const float4v r = red[w][lane];
        acc[0] += r[0];
        acc[1] += r[1];
        acc[2] += r[2];
        acc[3] += r[3];
    }
    // lane (j, c16) holds Y[4 j + i][n] for i < 4
    if constexpr (EPI == MM_STORE) {
        TSD_GLOBAL float* y = glb(o.y) + sl * o.slice;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * j + i < o.rows && n < N) y[(size_t)(4 * j + i) * o.ldy + n] = acc[i];
    } else if constexpr (EPI == MM_SWIGLU) {
        // rows (2m, 2m+1) = (gate_m, up_m): the up value sits in the neighbouring lane
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float up = __shfl_xor(acc[i], 1, 64);
            if ((c16 & 1) == 0 && 4 * j + i < o.rows && n < N)
                glb(o.y)[(size_t)(4 * j + i) * o.ldy + (n >> 1)] = silu(acc[i]) * up;
        }
    } else {
        const int pos = o.posp ? ld_uniform(o.posp) : o.pos_value;
        const int half = o.hd >> 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float partner = __shfl_xor(acc[i], 1, 64);
            const int b = 4 * j + i;
            if (b >= o.rows || n >= N) continue;
            if (n < o.qrows + o.krows) {
                if (c16 & 1) continue;
                const bool isk = n >= o.qrows;
                const int m = (isk ? n - o.qrows : n) >> 1;
                const int h = m / half, e = m - h * half;
                const float2 cs = o.rope[(size_t)pos * half + e];
                const float ra = acc[i] * cs.x - partner * cs.y, rb = acc[i] * cs.y + partner * cs.x;
                if (!isk) {
                    TSD_GLOBAL float* q = glb(o.q) + (size_t)b * o.qrows + h * o.hd;
                    q[e] = ra;
                    q[e + half] = rb;
                } else {
                    TSD_GLOBAL _Float16* kr =
                        (TSD_GLOBAL _Float16*)glb(o.kc) + (((size_t)b * o.Hkv + h) * o.n_ctx + pos) * o.hd;
                    kr[e] = (_Float16)ra;
                    kr[e + half] = (_Float16)rb;
                }
            } else {
                const int r = n - o.qrows - o.krows, h = r / o.hd, e = r - h * o.hd;
                ((TSD_GLOBAL _Float16*)glb(o.vc))[(((size_t)b * o.Hkv + h) * o.n_ctx + pos) * o.hd + e] = (_Float16)acc[i];
            }
        }
    }
}

// ---- embeddings ----------------------------------------------------------------------------
__global__ void k_embed_sum16(const EmbedTabs T, const int* __restrict__ codes, int ld_codes, int n_tab, int d,
                              float* __restrict__ x)
{
    const int b = blockIdx.y, k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= d) return;
    float s = 0.f;
    for (int c = 0; c < n_tab; ++c) {
        int id = codes[(size_t)b * ld_codes + c];
        id = id < 0 ? 0 : (id >= T.rows[c] ? T.rows[c] - 1 : id);
        s += T.tab[c][(size_t)id * d + k];
    }
    x[(size_t)b * d + k] = s;
}

// ---- per-row greedy pick ---------------------------------------------------------------------
__global__ __launch_bounds__(NT) void k_argmax_rows(const float* __restrict__ logits, int ld_l, int n, int* code,
                                                    int ld_code)
{
    const int b = blockIdx.x, t = threadIdx.x;
    const float* l = logits + (size_t)b * ld_l;
    unsigned long long best = 0ull;
    for (int i = t; i < n; i += NT) {
        const unsigned long long key = ((unsigned long long)float_order_key(l[i]) << 32) | (0xFFFFFFFFu - (uint32_t)i);
        best = key > best ? key : best;
    }
    best = wave_max_u64(best);
    __shared__ unsigned long long bk[NT / 64];
    if ((t & 63) == 0) bk[t >> 6] = best;
    __syncthreads();
    if (t == 0) {
        unsigned long long m = bk[0];
        for (int i = 1; i < NT / 64; ++i) m = bk[i] > m ? bk[i] : m;
        code[(size_t)b * ld_code] = (int)(0xFFFFFFFFu - (uint32_t)m);
    }
}

// y[b][n] = sum over s of part[s][b][n] (the standalone GEMM's split-K slices)
__global__ void k_sum_slices(const float* __restrict__ part, int S, long long slice, float* __restrict__ y, long long n)
{
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float a = 0.f;
    for (int s = 0; s < S; ++s) a += part[s * slice + i];
    y[i] = a;
}

// the frame's codes appended to the history at *pos, and the position advanced
__global__ void k_frame_done(const int* __restrict__ codes, int n, int* hist, int* pos)
{
    const int p = *pos;
    for (int i = threadIdx.x; i < n; i += blockDim.x) hist[(size_t)p * n + i] = codes[i];
    __syncthreads();
    if (threadIdx.x == 0) *pos = p + 1;
}

}  // namespace

bool mm16_supported(int fmt, int N, int K) { return fmt == FMT_AFF8 && N > 0 && K > 0 && K % 64 == 0 && K <= MM_MAX_K; }

hipError_t launch_prep16(const PrepArgs& p, hipStream_t st)
{
    if (p.K <= 0 || p.K % 64 || p.K > MM_MAX_K || p.rows <= 0 || p.rows > MM_ROWS || p.n_part < 0 ||
        p.n_part > MM_MAX_SPLIT || (p.n_part > 0 && !p.part))
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_prep16, dim3(p.rows), dim3(NT), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_mm16(int epi, const PackedMat& W, const Act16& a, int splits, const Mm16Out& o, hipStream_t st)
{
    if (!mm16_supported(FMT_AFF8, W.N, W.K) || !W.b || splits < 1 || splits > MM_MAX_SPLIT || splits > W.K / 64 ||
        o.rows < 1 || o.rows > MM_ROWS)
        return hipErrorInvalidValue;
    if (epi != MM_STORE && splits != 1) return hipErrorInvalidValue;   // nonlinear epilogues need the whole sum
    if ((epi == MM_SWIGLU || epi == MM_QKV_ROPE) && W.N % 2) return hipErrorInvalidValue;
    const dim3 grid((W.N + 15) / 16, splits);
    if (epi == MM_STORE) hipLaunchKernelGGL(k_mm16<MM_STORE>, grid, dim3(NT), 0, st, W, a, o);
    else if (epi == MM_SWIGLU) hipLaunchKernelGGL(k_mm16<MM_SWIGLU>, grid, dim3(NT), 0, st, W, a, o);
    else if (epi == MM_QKV_ROPE) hipLaunchKernelGGL(k_mm16<MM_QKV_ROPE>, grid, dim3(NT), 0, st, W, a, o);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_merge_prep16(const float* part, int B, int H, int hd, int max_split, const int* posp, int n_keys_value,
                               const Act16& a, hipStream_t st)
{
    if (hd % 64 || B < 1 || B > MM_ROWS) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_merge_prep16, dim3(B * H * hd / 64), dim3(64), 0, st, part, H, hd, max_split, posp, n_keys_value, a);
    return hipGetLastError();
}

hipError_t launch_embed_sum16(const EmbedTabs& T, const int* codes, int ld_codes, int n_tab, int d, float* x, int B,
                              hipStream_t st)
{
    if (n_tab < 1 || n_tab > 16 || B < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_embed_sum16, dim3((d + 255) / 256, B), dim3(256), 0, st, T, codes, ld_codes, n_tab, d, x);
    return hipGetLastError();
}

hipError_t launch_argmax_rows(const float* logits, int ld_l, int n, int* code, int ld_code, int B, hipStream_t st)
{
    if (n < 1 || B < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_argmax_rows, dim3(B), dim3(NT), 0, st, logits, ld_l, n, code, ld_code);
    return hipGetLastError();
}

hipError_t launch_sum_slices(const float* part, int S, long long slice, float* y, long long n, hipStream_t st)
{
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_sum_slices, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part, S, slice, y, n);
    return hipGetLastError();
}

hipError_t launch_frame_done(const int* codes, int n, int* hist, int* pos, hipStream_t st)
{
    hipLaunchKernelGGL(k_frame_done, dim3(1), dim3(256), 0, st, codes, n, hist, pos);
    return hipGetLastError();
}

}  // namespace tsd
