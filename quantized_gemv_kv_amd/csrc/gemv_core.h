// gemv_core.h — device building blocks of the fused dequant GEMV, shared by the per-operator
// GEMV kernels and the persistent step (internal).  NT is the workgroup size in threads.
#pragma once

#include <math.h>

#include "kernels.h"

namespace tsd {
namespace core {

constexpr int MAX_K = 4096;   // longest reduction dimension held in LDS

// byte i of v as float (v_cvt_f32_ubyteN), written out because the compiler otherwise folds the
// nibble masks into bit-field extracts and loses the one-instruction form
template <int I>
__device__ __forceinline__ float ubyte(uint32_t v)
{
    float r;
    if constexpr (I == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(v));
    else if constexpr (I == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(v));
    else if constexpr (I == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(v));
    else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(v));
    return r;
}

// bits 0..3 of v moved to bit 4 of bytes 0..3 (copies at shifts 0, 7, 14, 21 do not overlap,
// so one 24-bit multiply places every bit k at 8k; the mask keeps those)
__device__ __forceinline__ uint32_t spread4(uint32_t v) { return (__umul24(v & 0xFu, 0x00204081u) & 0x01010101u) << 4; }

// sum over the slot's elements of code * x: the codes as stored (Q8_0 offset by 128, Q4_0 and
// Q5_0 unsigned; h: the Q5_0 block's fifth bits, ignored by the other formats)
template <int F>
__device__ __forceinline__ float slot_dot(const uint4 w, const float* __restrict__ x, uint32_t h = 0u)
{
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    if constexpr (fmt_nibbles(F)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t lo = ws[j] & 0x0F0F0F0Fu, hi = (ws[j] >> 4) & 0x0F0F0F0Fu;
            if constexpr (F == FMT_Q5_0) {
                lo |= spread4(h >> (4 * j));
                hi |= spread4(h >> (16 + 4 * j));
            }
            float& al = (j & 1) ? a1 : a0;
            float& ah = (j & 1) ? a3 : a2;
            al = fmaf(ubyte<0>(lo), x[4 * j + 0], al);
            ah = fmaf(ubyte<0>(hi), x[16 + 4 * j + 0], ah);
            al = fmaf(ubyte<1>(lo), x[4 * j + 1], al);
            ah = fmaf(ubyte<1>(hi), x[16 + 4 * j + 1], ah);
            al = fmaf(ubyte<2>(lo), x[4 * j + 2], al);
            ah = fmaf(ubyte<2>(hi), x[16 + 4 * j + 2], ah);
            al = fmaf(ubyte<3>(lo), x[4 * j + 3], al);
            ah = fmaf(ubyte<3>(hi), x[16 + 4 * j + 3], ah);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float& a = j == 0 ? a0 : j == 1 ? a1 : j == 2 ? a2 : a3;
            a = fmaf(ubyte<0>(ws[j]), x[4 * j + 0], a);
            a = fmaf(ubyte<1>(ws[j]), x[4 * j + 1], a);
            a = fmaf(ubyte<2>(ws[j]), x[4 * j + 2], a);
            a = fmaf(ubyte<3>(ws[j]), x[4 * j + 3], a);
        }
    }
    return (a0 + a1) + (a2 + a3);
}

// one slot's contribution to its row: d = slot_dot, sx = the slot's sum of x, sc / sb the raw
// fp16 scale / bias of its group (zero scale for a slot outside the matrix)
template <int F>
__device__ __forceinline__ float slot_value(float d, float sx, float sc, float sb)
{
    if constexpr (F == FMT_Q4_0) return sc * fmaf(-8.f, sx, d);
    else if constexpr (F == FMT_Q8_0) return sc * fmaf(-128.f, sx, d);
    else if constexpr (F == FMT_Q5_0) return sc * fmaf(-16.f, sx, d);
    else return fmaf(sc, d, sb * sx);
}

// two sums in one pass (one pair of barriers)
template <int NT>
__device__ __forceinline__ float2 block_sum2(float a, float b, float* red)
{
    a = wave_sum(a);
    b = wave_sum(b);
    if ((threadIdx.x & 63) == 0) {
        red[2 * (threadIdx.x >> 6)] = a;
        red[2 * (threadIdx.x >> 6) + 1] = b;
    }
    lds_barrier();
    float2 r = make_float2(0.f, 0.f);
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
        r.x += red[2 * i];
        r.y += red[2 * i + 1];
    }
    lds_barrier();
    return r;
}

template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red)
{
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    lds_barrier();
    float r = 0.f;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) r += red[i];
    lds_barrier();
    return r;
}

__device__ __forceinline__ float4 f4add(float4 a, float4 b) { return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w); }

// x -> LDS, swizzled so that the lane owning slot s reads float4 e4 of its slice at
// index e4 * slots_per_row + s (consecutive lanes, consecutive addresses)
template <int E>
__device__ __forceinline__ int swz(int k, int lpr) { return ((k % E) >> 2) * lpr + k / E; }

// attention-merge prologue: per thread up to NJA float4 of the output, up to NSR chunks in
// registers (longer contexts take a slower loop)
constexpr int NJA = 2, NSR = 4;
struct AttnIn {
    float4 o[NJA][NSR];
    float m[NJA][NSR], l[NJA][NSR];
    int n_split;
};

template <int NT>
__device__ __forceinline__ void load_attn(const ProArgs& p, const int K, AttnIn& A)
{
    const int nch = K / 4, t = threadIdx.x, hd = p.a_hd, PS = hd + 4;
    const int n_keys = ld_uniform(p.pos) + 1 + p.pos_add;
    A.n_split = (n_keys + p.a_chunk - 1) / p.a_chunk;
#pragma unroll
    for (int j = 0; j < NJA; ++j) {
        const int c = t + j * NT;
#pragma unroll
        for (int s = 0; s < NSR; ++s) {
            A.o[j][s] = make_float4(0.f, 0.f, 0.f, 0.f);
            A.m[j][s] = -INFINITY;
            A.l[j][s] = 0.f;
            if (c < nch && s < A.n_split) {
                const int k = 4 * c, h = k / hd, i = k - h * hd;
                const float* pb = p.part + ((size_t)h * p.a_max_split + s) * PS;
                A.o[j][s] = *(const float4*)(pb + i);
                A.m[j][s] = pb[hd];
                A.l[j][s] = pb[hd + 1];
            }
        }
    }
}

template <int NT>
__device__ __forceinline__ void finish_attn(const ProArgs& p, const int K, const AttnIn& A, float4 (&v)[(MAX_K / 4 / NT)])
{
    const int nch = K / 4, t = threadIdx.x, hd = p.a_hd, PS = hd + 4;
#pragma unroll
    for (int j = 0; j < NJA; ++j) {
        const int c = t + j * NT;
        v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (c >= nch) continue;
        const int k = 4 * c, h = k / hd, i = k - h * hd;
        const float* ph = p.part + (size_t)h * p.a_max_split * PS;
        float M = -INFINITY;
#pragma unroll
        for (int s = 0; s < NSR; ++s) M = fmaxf(M, A.m[j][s]);
        for (int s = NSR; s < A.n_split; ++s) M = fmaxf(M, ph[(size_t)s * PS + hd]);
        float L = 0.f;
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int s = 0; s < NSR; ++s) {
            const float wgt = exp2f(A.m[j][s] - M);
            L = fmaf(A.l[j][s], wgt, L);
            o = make_float4(fmaf(A.o[j][s].x, wgt, o.x), fmaf(A.o[j][s].y, wgt, o.y), fmaf(A.o[j][s].z, wgt, o.z),
                            fmaf(A.o[j][s].w, wgt, o.w));
        }
        for (int s = NSR; s < A.n_split; ++s) {
            const float* pb = ph + (size_t)s * PS;
            const float wgt = exp2f(pb[hd] - M);
            const float4 os = *(const float4*)(pb + i);
            L = fmaf(pb[hd + 1], wgt, L);
            o = make_float4(fmaf(os.x, wgt, o.x), fmaf(os.y, wgt, o.y), fmaf(os.z, wgt, o.z), fmaf(os.w, wgt, o.w));
        }
        const float r = 1.0f / L;
        v[j] = make_float4(o.x * r, o.y * r, o.z * r, o.w * r);
    }
}

// phase 1 of the prologue: issue the input loads (the embedding rows for the first layer) and
// the norm's gain/bias
template <int PRO, int NT>
__device__ __forceinline__ void load_x(const ProArgs& p, const int K, float4 (&v)[MAX_K / 4 / NT],
                                       float4 (&g)[MAX_K / 4 / NT], float4 (&bt)[MAX_K / 4 / NT])
{
    constexpr bool EMB = PRO == PRO_LN_EMB || PRO == PRO_RMS_EMB;
    constexpr bool LN = PRO == PRO_LN || PRO == PRO_LN_EMB;
    const int nch = K / 4, t = threadIdx.x;
    if constexpr (PRO != PRO_LOAD) {
#pragma unroll
        for (int j = 0; j < (MAX_K / 4 / NT); ++j) {
            const int c = t + j * NT;
            g[j] = c < nch ? ((const float4*)p.g)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
            if constexpr (LN) bt[j] = c < nch ? ((const float4*)p.beta)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    if constexpr (PRO == PRO_ATTN) {
        return;
    } else if constexpr (EMB) {
        const int prow = p.pos_tab ? ld_uniform(p.pos) : 0;
#pragma unroll
        for (int j = 0; j < (MAX_K / 4 / NT); ++j) {
            const int c = t + j * NT;
            float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
            if (c < nch) {
                for (int i = 0; i < p.n_emb; ++i) {
                    int tk = ld_uniform(p.tok + i);
                    tk = tk < 0 ? 0 : (tk >= p.tab_rows[i] ? p.tab_rows[i] - 1 : tk);
                    a = f4add(a, ((const float4*)(p.tab[i] + (size_t)tk * K))[c]);
                }
                if (p.pos_tab) a = f4add(a, ((const float4*)(p.pos_tab + (size_t)prow * K))[c]);
            }
            v[j] = a;
        }
    } else {
#pragma unroll
        for (int j = 0; j < (MAX_K / 4 / NT); ++j) {
            const int c = t + j * NT;
            v[j] = c < nch ? ((const float4*)p.src)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
}

// phase 2: norm (if any) and the swizzled store into LDS
template <int F, int PRO, int NT>
__device__ __forceinline__ void finish_x(const ProArgs& p, const int K, float4 (&v)[MAX_K / 4 / NT],
                                         const float4 (&gg)[MAX_K / 4 / NT], const float4 (&bt)[MAX_K / 4 / NT],
                                         float4* xl4, float* red)
{
    constexpr int E = FmtT<F>::E;
    constexpr bool EMB = PRO == PRO_LN_EMB || PRO == PRO_RMS_EMB;
    constexpr bool LN = PRO == PRO_LN || PRO == PRO_LN_EMB;
    const int lpr = K / E, nch = K / 4, t = threadIdx.x;
    if (EMB && blockIdx.x == 0) {   // the first workgroup of each batch row (x_out is per row)
#pragma unroll
        for (int j = 0; j < (MAX_K / 4 / NT); ++j)
            if (t + j * NT < nch) ((float4*)p.x_out)[t + j * NT] = v[j];
    }
    if constexpr (PRO == PRO_LOAD || PRO == PRO_ATTN) {
#pragma unroll
        for (int j = 0; j < (MAX_K / 4 / NT); ++j) {
            const int c = t + j * NT;
            if (c < nch) xl4[swz<E>(4 * c, lpr)] = v[j];
        }
    } else {
        const float invK = 1.0f / (float)K;
        // LayerNorm: one pass over sums shifted by a value every thread knows (x[0] when x is
        // read from memory), which keeps E[(x-x0)^2] - E[x-x0]^2 free of cancellation when the
        // mean is large; RMSNorm needs only the sum of squares
        float x0 = 0.f;
        if constexpr (LN && !EMB) x0 = __int_as_float(ld_uniform((const int*)p.src));
        float s1 = 0.f, q2 = 0.f;
#pragma unroll
        for (int j = 0; j < (MAX_K / 4 / NT); ++j) {
            if (t + j * NT < nch) {
                const float dx = v[j].x - x0, dy = v[j].y - x0, dz = v[j].z - x0, dw = v[j].w - x0;
                s1 += (dx + dy) + (dz + dw);
                q2 += (dx * dx + dy * dy) + (dz * dz + dw * dw);
            }
        }
        float mean = 0.f, var;
        if constexpr (LN) {
            const float2 tot = block_sum2<NT>(s1, q2, red);
            const float ms = tot.x * invK;
            mean = x0 + ms;
            var = fmaxf(tot.y * invK - ms * ms, 0.f);
        } else {
            var = block_sum<NT>(q2, red) * invK;
        }
        const float r = 1.0f / sqrtf(var + p.eps);
#pragma unroll
        for (int j = 0; j < (MAX_K / 4 / NT); ++j) {
            const int c = t + j * NT;
            if (c < nch) {
                const float4 g = gg[j];
                float4 y = make_float4((v[j].x - mean) * r * g.x, (v[j].y - mean) * r * g.y,
                                       (v[j].z - mean) * r * g.z, (v[j].w - mean) * r * g.w);
                if constexpr (LN) y = f4add(y, bt[j]);
                xl4[swz<E>(4 * c, lpr)] = y;
            }
        }
    }
    lds_barrier();
}

__device__ __forceinline__ float gelu_tanh(float x)
{
    // tanh form of GELU (Hendrycks & Gimpel): 0.5 x (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3),
    // evaluated as x / (1 + e^(-2u)) (the same function: 0.5 (1 + tanh u) is the logistic of 2u)
    const float u = 0.7978845608028654f * fmaf(0.044715f * x, x * x, x);
    return __fdividef(x, 1.0f + __expf(-2.0f * u));
}

__device__ __forceinline__ float silu(float x) { return __fdividef(x, 1.0f + __expf(-x)); }

}  // namespace core
}  // namespace tsd
