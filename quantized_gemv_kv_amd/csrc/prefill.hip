// prefill.hip — the prompt pass: every prompt position of a GPT2/LLAMA decoder in one causal
// forward ([J] §3.2: prompt and decode graphs over one persistent KV cache; §3.11: the prompt
// graph's causal mask), instead of one decode step per position.
//
// The linears are matrix products on the matrix cores (v_mfma_f32_16x16x32_f16) straight from
// the packed GEMV layout, with the weights kept exact:
//   * every block of 32 weights enters as fp16 integers (its codes minus their zero point:
//     q - 8 for Q4_0 and 4-bit affine, q - 16 for Q5_0, the signed byte for Q8_0, q - 128 for
//     8-bit affine; a byte permute builds 1024 + code and one packed subtract removes the
//     offset), and one MFMA pair covers the block;
//   * an activation enters as two fp16 numbers, hi = fp16(x) and lo = fp16(x - hi);
//   * the block's (or group's) scale is applied in fp32 after its MFMAs:
//       sum_k w_k x_k = d P                     (Q4_0, Q5_0, Q8_0: w = d (q - zero))
//       sum_k w_k x_k = s P + (b + zero s) X    (affine: w = s q + b; X = sum_k x_k from the same
//                                                 operand fragments against a fragment of ones)
// Operand roles: A = 16 activation rows (lane l holds row l % 16), B = 16 weight rows (lane l
// holds row l % 16); lane group j = l / 16 supplies K positions 8 j .. 8 j + 7 of the block to
// both operands, so a lane's four results share one weight row (and so one scale).  A workgroup
// computes a 32 x 32 tile (2 x 2 MFMA tiles per wave); its four (eight, for reductions of 2048
// and more) waves each take a contiguous share of the scale groups along K, and the partial tiles
// are summed through LDS in wave order, so results do not depend on timing.  The small tile
// and the split keep ~1000 waves in flight for the 1024-wide projections of a 256-row prompt.
//
// Epilogues write what the next kernel consumes: queries (after RoPE) and the fp16 K/V cache
// entries at each row's position, the residual add, or the next product's hi/lo operand through
// GELU or SwiGLU.  Attention is causal over the cache (row r at position p reads keys 0..p) and
// runs on the matrix cores too, in the flash form (a running max and sum per query).
#include <math.h>

#include <type_traits>

#include "gemv_core.h"
#include "prefill.h"

namespace tsd {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// The operand of a product lives in fragment order: for each 16-row tile and 32-wide block of
// K, 1 KB in lane order (lane (j, c) holds row 16 t + c, K positions 32 blk + 8 j .. + 7), so one
// load instruction of a wave reads 1 KB of consecutive bytes.  Element (r, k) of an operand with
// K columns:
__device__ __forceinline__ size_t fl_index(int r, int k, int K)
{
    return ((((size_t)(r >> 4) * (K >> 5) + (k >> 5)) * 4 + ((k >> 3) & 3)) * 16 + (r & 15)) * 8 + (k & 7);
}

__device__ __forceinline__ void put_hilo(__half* hi, __half* lo, size_t idx, float y)
{
    const _Float16 h = (_Float16)y;
    ((TSD_GLOBAL _Float16*)hi)[idx] = h;
    ((TSD_GLOBAL _Float16*)lo)[idx] = (_Float16)(y - (float)h);
}

// the eight byte codes u of (w0, w1) (each < 2048 - 1024) as fp16 (1024 + u) - off: byte permutes
// put 0x64 above each code byte, which is the fp16 bit pattern of 1024 + u
__device__ __forceinline__ half8 codes_h8(uint32_t w0, uint32_t w1, _Float16 off)
{
    u32x4 u;
    u.x = __builtin_amdgcn_perm(0x64646464u, w0, 0x04010400u);
    u.y = __builtin_amdgcn_perm(0x64646464u, w0, 0x04030402u);
    u.z = __builtin_amdgcn_perm(0x64646464u, w1, 0x04010400u);
    u.w = __builtin_amdgcn_perm(0x64646464u, w1, 0x04030402u);
    return __builtin_bit_cast(half8, u) - off;
}

// per-format access to one 32-weight block of a packed row, for lane group j
// (PF_TILED8: the batched path's tiled 8-bit affine matrices, one 16-byte load per lane covering
// both blocks of a 64-group in the same lane order)
template <int F> struct PfFmt {
    static constexpr bool NIB = fmt_nibbles(F);
    static constexpr bool AFF = fmt_affine(F) || F == PF_TILED8;
    static constexpr int GB = (F == FMT_AFF8 || F == FMT_AFF4_G64 || F == PF_TILED8) ? 2 : 1;   // blocks per scale group
    // byte offset of lane group j's eight codes inside row n, and the stride between blocks
    __device__ static size_t row_off(int n, int K, int j)
    {
        return NIB ? (size_t)n * (K / 2) + 8 * (j & 1) : (size_t)n * K + 8 * j;
    }
    static constexpr int BLOCK_BYTES = NIB ? 16 : 32;
    // zero point entered with the code (w = scale (q - zero) [+ bias'])
    static constexpr float ZERO = F == FMT_Q4_0 || F == FMT_AFF4_G64 || F == FMT_AFF4_G32 ? 8.f
                                  : F == FMT_Q5_0                                         ? 16.f
                                                                                           : 128.f;
    // raw 8 bytes -> eight fp16 (q - zero); h: the block's Q5_0 fifth-bit word
    __device__ static half8 codes(u32x2 r, int j, uint32_t h)
    {
        uint32_t a = r.x, b = r.y;
        if constexpr (NIB) {
            const int sh = (j & 2) ? 4 : 0;   // lane groups 2, 3: elements 16..31 = high nibbles
            a = (a >> sh) & 0x0F0F0F0Fu;
            b = (b >> sh) & 0x0F0F0F0Fu;
            if constexpr (F == FMT_Q5_0) {
                const uint32_t hb = (h >> (8 * j)) & 0xFFu;   // fifth bits of elements 8j..8j+7
                a |= core::spread4(hb);
                b |= core::spread4(hb >> 4);
            }
        }
        return codes_h8(a, b, (_Float16)(1024.f + ZERO));
    }
};

__device__ __forceinline__ float4v mfma(half8 a, half8 b, float4v c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <int F, int EPI, int KS, int NU>
__global__ __launch_bounds__(64 * KS) void k_pf_gemm(const PfGemmArgs a)
{
    using T = PfFmt<F>;
    constexpr int GB = T::GB;
    __shared__ float red[KS][8 * NU][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int c = lane & 15, j = lane >> 4;
    const int m0 = blockIdx.y * PF_TILE;
    const int n0 = blockIdx.x * 16 * NU;
    const int N = a.W.N, K = a.W.K, M = a.M;
    const int ngrp = K / (32 * GB);
    // wave w reduces over scale groups [g_begin, g_end): the K range is split KS ways
    const int g_begin = ngrp * w / KS, g_end = ngrp * (w + 1) / KS;

    const TSD_GLOBAL half8* ah[2];
    const TSD_GLOBAL half8* al[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        // row tile (m0 + 16 s) / 16; the operand holds whole 32-row tiles (rows past M never stored)
        const size_t t0 = (size_t)((m0 + 16 * s) >> 4) * (K >> 5) * 64 + lane;
        ah[s] = (const TSD_GLOBAL half8*)glb(a.ahi) + t0;
        al[s] = (const TSD_GLOBAL half8*)glb(a.alo) + t0;
    }
    const TSD_GLOBAL uint8_t* wp[NU];
    const TSD_GLOBAL _Float16* sp[NU];
    const TSD_GLOBAL _Float16* bp[NU];
    const TSD_GLOBAL uint32_t* hp[NU];
    const TSD_GLOBAL u32x4* tq[NU];     // PF_TILED8: lane's 16 bytes of group 0 of its 16-row tile
    const TSD_GLOBAL uint32_t* tsb[NU]; // PF_TILED8: its (scale | bias << 16) word of group 0
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        if constexpr (F == PF_TILED8) {
            const int t = min((n0 + 16 * u) / 16, (N - 1) / 16);   // lane row c of tile t (rows past N never stored)
            tq[u] = (const TSD_GLOBAL u32x4*)glb(a.T.q) + (size_t)t * ngrp * 64 + lane;
            tsb[u] = glb(a.T.sb) + (size_t)t * ngrp * 16 + c;
        } else {
            const int n = min(n0 + 16 * u + c, N - 1);
            wp[u] = glb(a.W.q) + T::row_off(n, K, j);
            sp[u] = (const TSD_GLOBAL _Float16*)glb(a.W.s) + (size_t)n * ngrp;
            bp[u] = T::AFF ? (const TSD_GLOBAL _Float16*)glb(a.W.b) + (size_t)n * ngrp : nullptr;
            hp[u] = F == FMT_Q5_0 ? glb(a.W.h) + (size_t)n * (K / 32) : nullptr;
        }
    }

    half8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (_Float16)1.0f;

    float4v acc[2][NU];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int u = 0; u < NU; ++u) acc[s][u] = float4v{0.f, 0.f, 0.f, 0.f};

    // one stage: NG scale groups (NG * GB blocks), all loads issued before the first MFMA
    auto stage = [&](int g0, auto ng_tag) {
        constexpr int NG = decltype(ng_tag)::value;
        constexpr int NB = NG * GB;
        half8 xh[NB][2], xl[NB][2];
        u32x2 wr[NB][NU];
        uint32_t hb[NB][NU];
        float sc[NG][NU], bi[NG][NU];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int blk = g0 * GB + b;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                xh[b][s] = ah[s][(size_t)blk * 64];   // 1 KB (64 half8) per block of a row tile
                xl[b][s] = al[s][(size_t)blk * 64];
            }
            if constexpr (F != PF_TILED8) {
#pragma unroll
                for (int u = 0; u < NU; ++u) {
                    wr[b][u] = *(const TSD_GLOBAL u32x2*)(wp[u] + (size_t)blk * T::BLOCK_BYTES);
                    hb[b][u] = F == FMT_Q5_0 ? hp[u][blk] : 0u;
                }
            }
        }
        if constexpr (F == PF_TILED8) {   // one 16-byte load per group: bytes 0-7 block 2g, 8-15 block 2g+1
#pragma unroll
            for (int q = 0; q < NG; ++q)
#pragma unroll
                for (int u = 0; u < NU; ++u) {
                    const u32x4 v = tq[u][(size_t)(g0 + q) * 64];
                    wr[2 * q][u] = u32x2{v.x, v.y};
                    wr[2 * q + 1][u] = u32x2{v.z, v.w};
                    hb[2 * q][u] = hb[2 * q + 1][u] = 0u;
                }
        }
#pragma unroll
        for (int q = 0; q < NG; ++q)
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                if constexpr (F == PF_TILED8) {
                    const uint32_t sb = tsb[u][(size_t)(g0 + q) * 16];
                    sc[q][u] = (float)__builtin_bit_cast(_Float16, (uint16_t)(sb & 0xFFFFu));
                    bi[q][u] = (float)__builtin_bit_cast(_Float16, (uint16_t)(sb >> 16));
                } else {
                    sc[q][u] = (float)sp[u][g0 + q];
                    bi[q][u] = T::AFF ? (float)bp[u][g0 + q] : 0.f;
                }
            }
#pragma unroll
        for (int q = 0; q < NG; ++q) {
            float4v P[2][NU], X[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                X[s] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int u = 0; u < NU; ++u) P[s][u] = float4v{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int bb = 0; bb < GB; ++bb) {
                const int b = q * GB + bb;
                half8 wv[NU];
#pragma unroll
                for (int u = 0; u < NU; ++u) wv[u] = T::codes(wr[b][u], j, hb[b][u]);
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const half8 hi = xh[b][s];
                    const half8 lo = xl[b][s];
#pragma unroll
                    for (int u = 0; u < NU; ++u) {
                        P[s][u] = mfma(hi, wv[u], P[s][u]);
                        P[s][u] = mfma(lo, wv[u], P[s][u]);
                    }
                    if constexpr (T::AFF) {
                        X[s] = mfma(hi, ones, X[s]);
                        X[s] = mfma(lo, ones, X[s]);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const float d = sc[q][u];
                const float b2 = T::AFF ? fmaf(T::ZERO, d, bi[q][u]) : 0.f;   // b + zero * s
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float v = fmaf(d, P[s][u][i], acc[s][u][i]);
                        if constexpr (T::AFF) v = fmaf(b2, X[s][i], v);
                        acc[s][u][i] = v;
                    }
            }
        }
    };
    // groups per stage: four blocks of 32, or one 64-group for the group-64 formats (their
    // registers then leave room for four waves per SIMD, which the Talker's 512-row passes use)
    constexpr int SG = GB == 2 ? 1 : 4;
    int g = g_begin;
    for (; g + SG <= g_end; g += SG) stage(g, std::integral_constant<int, SG>{});
    for (; g < g_end; ++g) stage(g, std::integral_constant<int, 1>{});

    // the KS partial tiles summed in wave order (deterministic); wave w then finishes the
    // 16 x 16 sub-tiles st = w, w + KS, .. of the 2 x NU, (s, u) = (st & 1, st >> 1)
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[w][(u * 2 + s) * 4 + i][lane] = acc[s][u][i];
    __syncthreads();
    for (int st = w; st < 2 * NU; st += KS) {   // whole waves; no barrier follows
    const int s = st & 1, u = st >> 1;
    // epilogue: lane holds weight row n = n0 + 16u + c for activation rows m0 + 16s + 4j + i
    {
        const int n = n0 + 16 * u + c;
        const float bias = (a.bias && n < N) ? a.bias[n] : 0.f;
        {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float sum = red[0][st * 4 + i][lane];
#pragma unroll
                for (int q = 1; q < KS; ++q) sum += red[q][st * 4 + i][lane];
                const int r = m0 + 16 * s + 4 * j + i;
                const float v = sum + bias;
                float partner = 0.f;
                if constexpr (EPI == PF_SWIGLU || EPI == PF_QKV) partner = dpp_mov<0xB1>(v);   // column n ^ 1
                if (r >= M || n >= N) continue;
                if constexpr (EPI == PF_STORE) {
                    a.y[(size_t)r * a.ldy + n] = v;
                } else if constexpr (EPI == PF_RESID) {
                    a.y[(size_t)r * a.ldy + n] += v;
                } else if constexpr (EPI == PF_GELU) {
                    put_hilo(a.ohi, a.olo, fl_index(r, n, a.ldo), core::gelu_tanh(v));
                } else if constexpr (EPI == PF_SWIGLU) {
                    if ((n & 1) == 0) put_hilo(a.ohi, a.olo, fl_index(r, n >> 1, a.ldo), core::silu(v) * partner);
                } else {   // PF_QKV
                    const int b = r / a.n_pos, p = a.pos0 + (r - b * a.n_pos);
                    if (n < a.qrows + a.krows) {
                        const bool isk = n >= a.qrows;
                        const int nn = isk ? n - a.qrows : n, h = nn / a.hd, rr = nn - h * a.hd;
                        float out = v;
                        int e = rr;
                        if (a.rope) {
                            const int half = a.hd >> 1, ip = rr >> 1;
                            const float2 cs = a.rope_tab[(size_t)p * half + ip];
                            // row 2i holds element i, row 2i+1 element i + hd/2 (its partner lane)
                            out = (rr & 1) ? fmaf(partner, cs.y, v * cs.x) : fmaf(v, cs.x, -partner * cs.y);
                            e = (rr & 1) ? ip + half : ip;
                        }
                        if (!isk)
                            a.q[(size_t)r * a.ldq + h * a.hd + e] = out;
                        else
                            a.kc[b * a.kv_row + ((size_t)h * a.n_ctx + p) * a.hd + e] = __float2half_rn(out);
                    } else {
                        const int nn = n - a.qrows - a.krows, h = nn / a.hd, e = nn - h * a.hd;
                        a.vc[b * a.kv_row + ((size_t)h * a.n_ctx + p) * a.hd + e] = __float2half_rn(v);
                    }
                }
            }
        }
    }
    }
}

// ---- rows: embedding, norms, the standalone split ---------------------------------------------
constexpr int PF_NT = 256;
constexpr int PF_MAXV = core::MAX_K / PF_NT;   // row values per thread

__device__ __forceinline__ float row_sum(float v, float* red)
{
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return ((red[0] + red[1]) + red[2]) + red[3];
}

// The gain and bias of the thread's elements k = t + PF_NT i, each load issued unconditionally
// (clamped into the row) and before the row's reductions, so that they are in flight together with
// the row itself rather than one round trip each behind the reductions.
__device__ __forceinline__ void load_gain(const PfRowArgs& a, float (&gg)[PF_MAXV], float (&bb)[PF_MAXV])
{
    const int t = threadIdx.x, d = a.d;
    const float* bsrc = a.bn ? a.bn : a.g;
#pragma unroll
    for (int i = 0; i < PF_MAXV; ++i) {
        const int k = min(t + i * PF_NT, d - 1);
        gg[i] = a.g[k];
        bb[i] = bsrc[k];
    }
}

// LayerNorm (bn set) or RMSNorm of the row held in v, written to the operand row r
__device__ void norm_to_operand(const PfRowArgs& a, int r, const float (&v)[PF_MAXV], const float (&gg)[PF_MAXV],
                                const float (&bb)[PF_MAXV], float* red)
{
    const int t = threadIdx.x, d = a.d;
    const float invd = 1.0f / (float)d;
    float mean = 0.f, s2 = 0.f;
    if (a.bn) {
        float s1 = 0.f;
#pragma unroll
        for (int i = 0; i < PF_MAXV; ++i)
            if (t + i * PF_NT < d) s1 += v[i];
        mean = row_sum(s1, red) * invd;
    }
#pragma unroll
    for (int i = 0; i < PF_MAXV; ++i)
        if (t + i * PF_NT < d) s2 = fmaf(v[i] - mean, v[i] - mean, s2);
    const float rs = 1.0f / sqrtf(row_sum(s2, red) * invd + a.eps);
#pragma unroll
    for (int i = 0; i < PF_MAXV; ++i) {
        const int k = t + i * PF_NT;
        if (k < d) {
            float y = (v[i] - mean) * rs * gg[i];
            if (a.bn) y += bb[i];
            put_hilo(a.ahi, a.alo, fl_index(r, k, d), y);
        }
    }
}

__global__ __launch_bounds__(PF_NT) void k_pf_embed(const PfRowArgs a)
{
    __shared__ float red[4];
    __shared__ int ids[16];
    const int r = blockIdx.x, t = threadIdx.x, d = a.d;
    const int b = r / a.n_pos, tt = r - b * a.n_pos, p = a.pos0 + tt;
    const int* tr = a.tok + (b * a.tok_stride + a.t0 + tt) * a.n_tab;   // this position's ids
    if (t < a.n_tab) ids[t] = min(max(tr[t], 0), a.tab_rows[t] - 1);
    if (t == 0) {
        a.seq[(size_t)p * a.B + b] = min(max(tr[0], 0), a.tab_rows[0] - 1);
        // the history at a prompt position holds the id that follows it (the next prompt id)
        if (a.hist && a.t0 + tt + 1 < a.n_prompt) a.hist[(size_t)p * a.B + b] = min(max(tr[a.n_tab], 0), a.tab_rows[0] - 1);
    }
    float gg[PF_MAXV], bb[PF_MAXV];
    load_gain(a, gg, bb);
    __syncthreads();
    // the sum over the tables in table order, then the learned position; each table's loads are
    // issued together (clamped into the row; elements past it are dropped below)
    float v[PF_MAXV];
#pragma unroll
    for (int i = 0; i < PF_MAXV; ++i) v[i] = 0.f;
    for (int c = 0; c < a.n_tab; ++c) {
        const float* er = a.tab[c] + (size_t)ids[c] * d;
#pragma unroll
        for (int i = 0; i < PF_MAXV; ++i) v[i] += er[min(t + i * PF_NT, d - 1)];
    }
    if (a.wpe) {
        const float* pr = a.wpe + (size_t)p * d;
#pragma unroll
        for (int i = 0; i < PF_MAXV; ++i) v[i] += pr[min(t + i * PF_NT, d - 1)];
    }
#pragma unroll
    for (int i = 0; i < PF_MAXV; ++i) {
        const int k = t + i * PF_NT;
        if (k < d) a.x_out[(size_t)r * d + k] = v[i];
        else v[i] = 0.f;
    }
    norm_to_operand(a, r, v, gg, bb, red);
}

__global__ __launch_bounds__(PF_NT) void k_pf_norm(const PfRowArgs a)
{
    __shared__ float red[4];
    const int r = blockIdx.x, t = threadIdx.x, d = a.d;
    float v[PF_MAXV], gg[PF_MAXV], bb[PF_MAXV];
#pragma unroll
    for (int i = 0; i < PF_MAXV; ++i) {
        const int k = t + i * PF_NT;
        const float x = a.x[(size_t)r * d + min(k, d - 1)];
        v[i] = k < d ? x : 0.f;
    }
    load_gain(a, gg, bb);
    norm_to_operand(a, r, v, gg, bb, red);
}

// rows [M, Mpad) of the last tile are written as zeros
__global__ __launch_bounds__(256) void k_pf_split(const float* __restrict__ x, int M, int Mpad, int K, __half* hi, __half* lo)
{
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)Mpad * K) return;
    const int r = (int)(i / K), k = (int)(i - (size_t)r * K);
    put_hilo(hi, lo, fl_index(r, k, K), r < M ? x[i] : 0.f);
}

// ---- causal attention over the cache (matrix cores) -------------------------------------------
constexpr int PF_ATTN_WAVES = 4;
// One workgroup of PF_ATTN_WAVES waves per (batch row, 16 consecutive queries, head); wave w takes
// the key blocks w, w + PF_ATTN_WAVES, .. (so the last query tiles, which see the most keys, are
// not one long chain), and wave 0 merges the waves' running (max, sum, O^T).  Per block of 32 keys:
//   S^T = K Q^T          A = 16 keys (lane row = key), B = Q^T (lane column = query c), K-dim =
//                        head dims; q enters as fp16 hi/lo (scaled to the log2 domain), keys exact
//   running max / sum    per query c over its 8 keys in the lane and the 4 lane groups
//   O^T += V^T P^T       B = P^T is exactly the lane's 8 probabilities (hi/lo), A = V^T with row
//                        c of dim tile dt holding dim c * DT + dt, so a lane reads DT consecutive
//                        dims of each of its 8 keys
// The result O^T leaves the lane with query c's dims (4 j + i) DT + dt: 4 DT consecutive values.
__device__ __forceinline__ float group4_max(float v)   // over lanes c, c + 16, c + 32, c + 48
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float group4_sum(float v)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int HD, int NW>
__global__ __launch_bounds__(64 * NW) void k_pf_fattn(const PfAttnArgs a)
{
    constexpr int NC = HD / 32;   // K-dim chunks of S^T
    constexpr int DT = HD / 16;   // dim tiles of O^T
    typedef _Float16 halfDT __attribute__((ext_vector_type(DT)));
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, c = lane & 15, j = lane >> 4;
    const int ntile = (a.n_pos + 15) / 16;
    const int b = blockIdx.x / ntile, t0 = (blockIdx.x - b * ntile) * 16;
    const int h = blockIdx.y, g = h / (a.H / a.Hkv);
    const int tq = min(t0 + c, a.n_pos - 1);              // query of lane column c (clamped; never stored)
    const int r = b * a.n_pos + tq;
    const int pq = a.pos0 + tq;                            // it attends keys 0..pq
    const int plast = a.pos0 + min(t0 + 15, a.n_pos - 1);  // the tile's last position
    const TSD_GLOBAL _Float16* Kc = (const TSD_GLOBAL _Float16*)glb(a.kc) + b * a.kv_row + (size_t)g * a.n_ctx * HD;
    const TSD_GLOBAL _Float16* Vc = (const TSD_GLOBAL _Float16*)glb(a.vc) + b * a.kv_row + (size_t)g * a.n_ctx * HD;

    // Q^T fragments: lane (j, c) holds query c's dims 32 kk + 8 j .. + 7
    const float qscale = 1.4426950408889634f / sqrtf((float)HD);
    half8 qh[NC], ql[NC];
    const TSD_GLOBAL float* qr = glb(a.q) + (size_t)r * a.ldq + h * HD + 8 * j;
#pragma unroll
    for (int kk = 0; kk < NC; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = qr[32 * kk + e] * qscale;
            const _Float16 hi = (_Float16)x;
            qh[kk][e] = hi;
            ql[kk][e] = (_Float16)(x - (float)hi);
        }
    float4v o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = float4v{0.f, 0.f, 0.f, 0.f};
    float mx = -INFINITY, l = 0.f;   // query c's running max and sum (the same in its 4 lanes)

    for (int k0 = 32 * w; k0 <= plast; k0 += 32 * NW) {   // wave w: key blocks w, w + NW, ..
        // keys of this lane's operand rows / probability slots (clamped reads, masked below)
        float4v st[2];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int key = min(k0 + 16 * sub + c, plast);
            const TSD_GLOBAL half8* kr = (const TSD_GLOBAL half8*)(Kc + (size_t)key * HD) + j;
            st[sub] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < NC; ++kk) {
                const half8 kf = kr[4 * kk];
                st[sub] = mfma(kf, qh[kk], st[sub]);
                st[sub] = mfma(kf, ql[kk], st[sub]);
            }
        }
        halfDT vr[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int key = min(k0 + 16 * (e >> 2) + 4 * j + (e & 3), plast);
            vr[e] = *(const TSD_GLOBAL halfDT*)(Vc + (size_t)key * HD + c * DT);
        }
        // lane holds S^T[key k0 + 16 (e / 4) + 4 j + e % 4][query c] at slot e
        float sv[8];
        float ml = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int key = k0 + 16 * (e >> 2) + 4 * j + (e & 3);
            sv[e] = key <= pq ? st[e >> 2][e & 3] : -INFINITY;
            ml = fmaxf(ml, sv[e]);
        }
        const float mn = fmaxf(mx, group4_max(ml));
        // -inf while this wave has seen no key of query c (its blocks start past the query): a zero
        // reference keeps every weight at 0 instead of exp2(-inf + inf)
        const float mref = mn == -INFINITY ? 0.f : mn;
        const float alpha = exp2f(mx - mref);        // 0 on the wave's first block
        half8 ph, pl;
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p = exp2f(sv[e] - mref);
            ps += p;
            const _Float16 hi = (_Float16)p;
            ph[e] = hi;
            pl[e] = (_Float16)(p - (float)hi);
        }
        l = fmaf(l, alpha, group4_sum(ps));
        mx = mn;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            half8 va;
#pragma unroll
            for (int e = 0; e < 8; ++e) va[e] = vr[e][dt];
            o[dt] = o[dt] * alpha;
            o[dt] = mfma(va, ph, o[dt]);
            o[dt] = mfma(va, pl, o[dt]);
        }
    }
    if constexpr (NW > 1) {
        // the waves' (O^T, max, sum) merged by wave 0: every wave holds the same (query, dim) in the
        // same lane and register, so the merge is elementwise per lane
        __shared__ float xo[NW - 1][4 * DT + 2][64];
        if (w > 0) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) xo[w - 1][4 * dt + i][lane] = o[dt][i];
            xo[w - 1][4 * DT][lane] = mx;
            xo[w - 1][4 * DT + 1][lane] = l;
        }
        __syncthreads();
        if (w > 0) return;
        float M = mx;   // finite: wave 0's first block holds key 0
#pragma unroll
        for (int u = 0; u < NW - 1; ++u) M = fmaxf(M, xo[u][4 * DT][lane]);
        const float s0 = exp2f(mx - M);
        l *= s0;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] = o[dt] * s0;
#pragma unroll
        for (int u = 0; u < NW - 1; ++u) {
            const float su = exp2f(xo[u][4 * DT][lane] - M);   // 0 for a wave that saw no key
            l = fmaf(xo[u][4 * DT + 1][lane], su, l);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[dt][i] = fmaf(xo[u][4 * dt + i][lane], su, o[dt][i]);
        }
    }
    if (t0 + c >= a.n_pos) return;
    const float il = 1.0f / l;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) put_hilo(a.ohi, a.olo, fl_index(r, h * HD + (4 * j + i) * DT + dt, a.ldo), o[dt][i] * il);
}

template <int F, int KS, int NU>
hipError_t gemm_epi_ks(int epi, const PfGemmArgs& a, hipStream_t st)
{
    const dim3 grid((a.W.N + 16 * NU - 1) / (16 * NU), (a.M + PF_TILE - 1) / PF_TILE);
    switch (epi) {
    case PF_STORE: k_pf_gemm<F, PF_STORE, KS, NU><<<grid, 64 * KS, 0, st>>>(a); break;
    case PF_QKV: k_pf_gemm<F, PF_QKV, KS, NU><<<grid, 64 * KS, 0, st>>>(a); break;
    case PF_RESID: k_pf_gemm<F, PF_RESID, KS, NU><<<grid, 64 * KS, 0, st>>>(a); break;
    case PF_GELU: k_pf_gemm<F, PF_GELU, KS, NU><<<grid, 64 * KS, 0, st>>>(a); break;
    case PF_SWIGLU: k_pf_gemm<F, PF_SWIGLU, KS, NU><<<grid, 64 * KS, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// long reductions split eight ways, the rest four ways; very wide products (N >= 6144), and Q8_0
// products from 2048 rows, give each wave 64 columns (each activation fragment then feeds four MFMA
// tiles), the rest 32 (measured per format: the 4-bit and tiled 8-bit products lose parallelism
// there faster than they gain operand reuse)
template <int F>
hipError_t gemm_epi(int epi, const PfGemmArgs& a, hipStream_t st)
{
    if (a.W.K >= 2048) return gemm_epi_ks<F, 8, 2>(epi, a, st);
    const bool wide = a.W.N >= 6144 || (F == FMT_Q8_0 && a.W.N >= 2048);
    return wide ? gemm_epi_ks<F, 4, 4>(epi, a, st) : gemm_epi_ks<F, 4, 2>(epi, a, st);
}

}  // namespace

bool pf_gemm_ok(int fmt, int K)
{
    return fmt >= 0 && fmt < FMT_COUNT && K > 0 && K % fmt_group(fmt) == 0 && K % 32 == 0;
}

hipError_t launch_pf_gemm(int fmt, int epi, const PfGemmArgs& a, hipStream_t st)
{
    if (!pf_gemm_ok(fmt, a.W.K) || a.M <= 0 || a.W.N <= 0) return hipErrorInvalidValue;
    if ((epi == PF_SWIGLU || epi == PF_QKV) && a.W.N % 2) return hipErrorInvalidValue;
    switch (fmt) {
    case FMT_Q4_0: return gemm_epi<FMT_Q4_0>(epi, a, st);
    case FMT_Q8_0: return gemm_epi<FMT_Q8_0>(epi, a, st);
    case FMT_AFF8: return gemm_epi<FMT_AFF8>(epi, a, st);
    case FMT_Q5_0: return gemm_epi<FMT_Q5_0>(epi, a, st);
    case FMT_AFF4_G64: return gemm_epi<FMT_AFF4_G64>(epi, a, st);
    case FMT_AFF4_G32: return gemm_epi<FMT_AFF4_G32>(epi, a, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_pf_gemm_tiled(int epi, const PfGemmArgs& a, hipStream_t st)
{
    if (a.M <= 0 || a.W.N <= 0 || a.W.K <= 0 || a.W.K % 64 || a.T.N != a.W.N || a.T.K != a.W.K)
        return hipErrorInvalidValue;
    if ((epi == PF_SWIGLU || epi == PF_QKV) && a.W.N % 2) return hipErrorInvalidValue;
    return gemm_epi<PF_TILED8>(epi, a, st);
}

hipError_t launch_pf_embed(const PfRowArgs& a, hipStream_t st)
{
    if (a.M <= 0 || a.d > core::MAX_K || a.n_tab < 1 || a.n_tab > 16) return hipErrorInvalidValue;
    k_pf_embed<<<a.M, PF_NT, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_pf_norm(const PfRowArgs& a, hipStream_t st)
{
    if (a.M <= 0 || a.d > core::MAX_K) return hipErrorInvalidValue;
    k_pf_norm<<<a.M, PF_NT, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_pf_split(const float* x, int M, int K, __half* hi, __half* lo, hipStream_t st)
{
    if (M <= 0 || K <= 0 || K % 32) return hipErrorInvalidValue;
    const int Mpad = (M + PF_TILE - 1) / PF_TILE * PF_TILE;
    const size_t n = (size_t)Mpad * K;
    k_pf_split<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(x, M, Mpad, K, hi, lo);
    return hipGetLastError();
}

hipError_t launch_pf_attention(const PfAttnArgs& a, hipStream_t st)
{
    if (a.M <= 0 || a.Hkv <= 0 || a.H % a.Hkv) return hipErrorInvalidValue;
    if (a.M % a.n_pos) return hipErrorInvalidValue;
    const dim3 grid((a.M / a.n_pos) * ((a.n_pos + 15) / 16), a.H);
    if (a.hd == 64) k_pf_fattn<64, PF_ATTN_WAVES><<<grid, 64 * PF_ATTN_WAVES, 0, st>>>(a);
    else if (a.hd == 128) k_pf_fattn<128, PF_ATTN_WAVES><<<grid, 64 * PF_ATTN_WAVES, 0, st>>>(a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace tsd
