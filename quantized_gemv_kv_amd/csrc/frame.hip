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
//     and X comes from the same operand fragments multiplied by a fragment of ones (four more
//     MFMAs per group, shared by every weight tile of the workgroup).
// Operand roles: A = the 16 activation rows (lane l holds row l % 16), B = 16 weight rows (lane
// l holds row n0 + l % 16), so a lane's four results share one weight row and so one (s, b) per
// group.  Within a group, lane group j = l / 16 supplies K positions 16 j .. 16 j + 15 to two
// MFMAs (the same K permutation on both operands), i.e. one 16-byte load of weights per lane.
//
// Every operand is produced ready by the kernel before: the attention (or its merge) and the
// SwiGLU epilogue write fp16 hi/lo rows; the epilogue that adds a projection into the residual
// stream also writes the next norm's input, hi/lo of x * g, and per 16-column tile the rows'
// partial sums of x^2.  The GEMM that consumes a norm's input sums those partials in a fixed
// order and applies the RMSNorm's 1 / rms to its results, so no normalisation kernel runs
// between layers and the residual stream is never re-read to build an operand.
#include <math.h>

#include "exchange.h"
#include "gemv_core.h"
#include "frame.h"
#include "sampler.h"

namespace tsd {
namespace {

using core::silu;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void put_hilo(const Act16& a, size_t idx, float y)
{
    const _Float16 h = (_Float16)y;
    ((TSD_GLOBAL _Float16*)a.hi)[idx] = h;
    ((TSD_GLOBAL _Float16*)a.lo)[idx] = (_Float16)(y - (float)h);
}

// sum over the 256 threads of a workgroup in a fixed order; every thread gets it
__device__ __forceinline__ float block_sum256(float v, float* red)
{
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return ((red[0] + red[1]) + red[2]) + red[3];
}

// ---- attention partials merged into the operand of the output projection -------------------
// one thread per output element
__global__ __launch_bounds__(256) void k_merge16(const float* __restrict__ part, int H, int hd, int max_split,
                                                 const int* posp, int n_keys_value, int n, const Act16 a)
{
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= n) return;
    const int i = e % hd, bh = e / hd;
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
    const int b = bh / H, h = bh - b * H;
    put_hilo(a, il_act(b, h * hd + i), O / L);
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

// what an epilogue reads besides the results, loaded before the main loop so that its latency
// hides behind the weight stream: the residual values it adds to and the next norm's gain
// (RESID), the position and the lane's rotation (QKV_ROPE)
struct Pre {
    float xo[4];
    float gn;
    float2 cs;
};

template <int EPI>
__device__ __forceinline__ void prefetch(const Mm16Out& o, int tile, int N, int j, int c16, int pos, Pre& p)
{
    const int n = tile * 16 + c16;
    if constexpr (EPI == MM_RESID) {
#pragma unroll
        for (int i = 0; i < 4; ++i) p.xo[i] = (4 * j + i < o.rows && n < N) ? glb(o.y)[il_x(4 * j + i, n)] : 0.f;
        p.gn = (o.next.hi && n < N) ? glb(o.g_next)[n] : 0.f;
    } else if constexpr (EPI == MM_QKV_ROPE) {
        p.cs = make_float2(1.f, 0.f);
        if (n < o.qrows + o.krows && (c16 & 1) == 0) {
            const int half = o.hd >> 1;
            const int m = (n >= o.qrows ? n - o.qrows : n) >> 1;
            p.cs = o.rope[(size_t)pos * half + (m - (m / half) * half)];
        }
    }
}

// lane (j, c16) holds Y[4 j + i][n] for i < 4; tile = the 16-row tile of W
template <int EPI>
__device__ __forceinline__ void epilogue(const Mm16Out& o, int tile, int N, int j, int c16, int sl, int pos,
                                         const Pre& pre, const float4v& acc, uint32_t xep)
{
    const int n = tile * 16 + c16;
    if constexpr (EPI == MM_STORE) {
        TSD_GLOBAL float* y = glb(o.y) + sl * o.slice;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * j + i < o.rows && n < N) y[(size_t)(4 * j + i) * o.ldy + n] = acc[i];
    } else if constexpr (EPI == MM_RESID) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int b = 4 * j + i;
            float sq = 0.f;
            if (b < o.rows && n < N) {
                const float v = pre.xo[i] + acc[i];
                glb(o.y)[il_x(b, n)] = v;
                if (o.next.hi) put_hilo(o.next, il_act(b, n), v * pre.gn);
                sq = v * v;
            }
            if (o.ssq_out) {   // the tile's part of the row's sum of squares (same order every time)
                sq = group_sum(sq, 16);
                if (c16 == 0 && b < o.rows) glb(o.ssq_out)[(size_t)tile * MM_ROWS + b] = sq;
            }
        }
    } else if constexpr (EPI == MM_SWIGLU) {
        // rows (2m, 2m+1) = (gate_m, up_m): the up value sits in the neighbouring lane
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float up = __shfl_xor(acc[i], 1, 64);
            if ((c16 & 1) == 0 && 4 * j + i < o.rows && n < N) put_hilo(o.act, il_act(4 * j + i, n >> 1), silu(acc[i]) * up);
        }
    } else {
        const int half = o.hd >> 1;
        // the exchange copy for a fused attention (the words of row b at xq + b * ldx, epoch xep)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float partner = __shfl_xor(acc[i], 1, 64);
            const int b = 4 * j + i;
            if (b >= o.rows || n >= N) continue;
            uint64_t* xr = o.xq ? o.xq + (size_t)b * o.ldx : nullptr;
            if (n < o.qrows + o.krows) {
                if (c16 & 1) continue;
                const bool isk = n >= o.qrows;
                const int m = (isk ? n - o.qrows : n) >> 1;
                const int h = m / half, e = m - h * half;
                const float2 cs = pre.cs;
                const float ra = acc[i] * cs.x - partner * cs.y, rb = acc[i] * cs.y + partner * cs.x;
                if (!isk) {
                    TSD_GLOBAL float* qr = glb(o.q) + (size_t)b * o.qrows + h * o.hd;
                    qr[e] = ra;
                    qr[e + half] = rb;
                    if (xr) {
                        xchg::store(xr + h * o.hd + e, ra, xep);
                        xchg::store(xr + h * o.hd + e + half, rb, xep);
                    }
                } else {
                    TSD_GLOBAL _Float16* kr =
                        (TSD_GLOBAL _Float16*)glb(o.kc) + (((size_t)b * o.Hkv + h) * o.n_ctx + pos) * o.hd;
                    const _Float16 ka = (_Float16)ra, kb = (_Float16)rb;
                    kr[e] = ka;
                    kr[e + half] = kb;
                    if (xr) {
                        xchg::store(xr + o.qrows + h * o.hd + e, (float)ka, xep);
                        xchg::store(xr + o.qrows + h * o.hd + e + half, (float)kb, xep);
                    }
                }
            } else {
                const int rr = n - o.qrows - o.krows, h = rr / o.hd, e = rr - h * o.hd;
                const _Float16 v = (_Float16)acc[i];
                ((TSD_GLOBAL _Float16*)glb(o.vc))[(((size_t)b * o.Hkv + h) * o.n_ctx + pos) * o.hd + e] = v;
                if (xr) xchg::store(xr + n, (float)v, xep);
            }
        }
    }
}

// Y = W X for the 16 operand rows: a workgroup of NW waves takes T consecutive 16-row tiles of W
// (blockIdx.x) over one K slice (blockIdx.y of gridDim.y).  Each wave reduces a contiguous share
// of the slice's groups: per chunk of U groups it issues every load first (weights of the T
// tiles, then its operand fragment, which serves all T tiles), then converts and runs the MFMAs;
// the waves add their results in LDS and wave 0 runs the epilogue.
template <int EPI, int T, int NW, int U>
__device__ __forceinline__ void mm16_block(const TiledMat& W, const MmIn& in, const Mm16Out& o, const int bx, const int S,
                                           const int sl)
{
    const int K = W.K, G = K >> 6, N = W.N, tiles = (N + 15) >> 4;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, j = lane >> 4, c16 = lane & 15;
    const int g_lo = (int)((long long)G * sl / S), g_hi = (int)((long long)G * (sl + 1) / S);
    const int cnt = g_hi - g_lo, q = cnt / NW, r = cnt - q * NW;
    const int w_lo = g_lo + wave * q + (wave < r ? wave : r), w_n = q + (wave < r ? 1 : 0);

    const TSD_GLOBAL u32x4* wr[T];
    const TSD_GLOBAL uint32_t* sbr[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        int tile = bx * T + t;
        tile = tile < tiles ? tile : tiles - 1;   // tiles past the matrix reload the last one and store nothing
        wr[t] = (const TSD_GLOBAL u32x4*)glb(W.q) + (size_t)tile * G * 64 + lane;
        sbr[t] = glb(W.sb) + (size_t)tile * G * 16 + c16;
    }
    const TSD_GLOBAL half8* ah = (const TSD_GLOBAL half8*)glb(in.a.hi) + j * MM_ROWS + c16;
    const TSD_GLOBAL half8* al = (const TSD_GLOBAL half8*)glb(in.a.lo) + j * MM_ROWS + c16;
    // a norm's operand: the rows' partial sums of squares, loaded now, summed after the main loop
    const bool norm = in.ssq != nullptr;
    const int sb_row = threadIdx.x & 15, sb_part = threadIdx.x >> 4;   // 16 parts of 16 threads
    float sp[4] = {0.f, 0.f, 0.f, 0.f};
    if (norm && threadIdx.x < 256)
#pragma unroll
        for (int p = 0; p < 4; ++p)
            if (sb_part + 16 * p < in.n_ssq) sp[p] = glb(in.ssq)[(size_t)(sb_part + 16 * p) * MM_ROWS + sb_row];
    // the epilogue's own inputs (wave 0 runs it)
    const int pos = EPI == MM_QKV_ROPE ? (o.posp ? ld_uniform(o.posp) : o.pos_value) : 0;
    // a fused attention's epoch, read with the position (long before the epilogue needs it)
    const uint32_t xep = EPI == MM_QKV_ROPE && o.xq ? (uint32_t)ld_uniform((const int*)o.xctr) * (uint32_t)FUSE_EPOCHS + (uint32_t)o.xidx + 1u : 0u;
    // a head's logits are not written after a rejected input
    const bool skip = EPI == MM_STORE && o.err && ld_uniform((const int*)o.err);
    Pre pre[T];
    if (wave == 0)
#pragma unroll
        for (int t = 0; t < T; ++t) prefetch<EPI>(o, bx * T + t, N, j, c16, pos, pre[t]);
    half8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (_Float16)1.0f;

    float4v acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = (float4v){0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < w_n; c += U) {
        u32x4 wq[T][U];
        uint32_t sb[T][U];
        half8 h0[U], h1[U], l0[U], l1[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {   // clamped to the wave's last group, masked below
            const int grp = w_lo + (c + u < w_n ? c + u : w_n - 1);
#pragma unroll
            for (int t = 0; t < T; ++t) {
                wq[t][u] = wr[t][grp * 64];
                sb[t][u] = sbr[t][grp * 16];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // K offsets 8j .. 8j+7 (first MFMA) and 32 + 8j .. (second) of the group
            const int grp = w_lo + (c + u < w_n ? c + u : w_n - 1);
            h0[u] = ah[grp * 8 * MM_ROWS];
            h1[u] = ah[(grp * 8 + 4) * MM_ROWS];
            l0[u] = al[grp * 8 * MM_ROWS];
            l1[u] = al[(grp * 8 + 4) * MM_ROWS];
        }
        // every load of the chunk is in flight before the first use
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool valid = c + u < w_n;
            // X: the group sums of the operand rows, from the same fragments
            float4v xz = {0.f, 0.f, 0.f, 0.f};
            xz = __builtin_amdgcn_mfma_f32_16x16x32_f16(h0[u], ones, xz, 0, 0, 0);
            xz = __builtin_amdgcn_mfma_f32_16x16x32_f16(h1[u], ones, xz, 0, 0, 0);
            xz = __builtin_amdgcn_mfma_f32_16x16x32_f16(l0[u], ones, xz, 0, 0, 0);
            xz = __builtin_amdgcn_mfma_f32_16x16x32_f16(l1[u], ones, xz, 0, 0, 0);
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const half8 w0 = q8_to_half8(wq[t][u].x, wq[t][u].y), w1 = q8_to_half8(wq[t][u].z, wq[t][u].w);
                float4v pz = {0.f, 0.f, 0.f, 0.f};
                pz = __builtin_amdgcn_mfma_f32_16x16x32_f16(h0[u], w0, pz, 0, 0, 0);
                pz = __builtin_amdgcn_mfma_f32_16x16x32_f16(h1[u], w1, pz, 0, 0, 0);
                pz = __builtin_amdgcn_mfma_f32_16x16x32_f16(l0[u], w0, pz, 0, 0, 0);
                pz = __builtin_amdgcn_mfma_f32_16x16x32_f16(l1[u], w1, pz, 0, 0, 0);
                const float sv = (float)__builtin_bit_cast(_Float16, (uint16_t)(sb[t][u] & 0xFFFFu));
                const float bv = (float)__builtin_bit_cast(_Float16, (uint16_t)(sb[t][u] >> 16));
                const float s1 = valid ? sv : 0.f;
                const float c0 = valid ? fmaf(128.f, sv, bv) : 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[t][i] = fmaf(s1, pz[i], fmaf(c0, xz[i], acc[t][i]));
            }
        }
    }

    __shared__ float4v red[NW - 1][T][64];
    __shared__ float ssp[16][16];
    __shared__ float rrow[16];
    if (wave > 0)
#pragma unroll
        for (int t = 0; t < T; ++t) red[wave - 1][t][lane] = acc[t];
    if (norm && threadIdx.x < 256) {
        float v = ((sp[0] + sp[1]) + sp[2]) + sp[3];
        for (int p = sb_part + 64; p < in.n_ssq; p += 16) v += glb(in.ssq)[(size_t)p * MM_ROWS + sb_row];
        ssp[sb_part][sb_row] = v;
    }
    __syncthreads();
    if (wave != 0 || skip) return;
    if (norm) {
        if (lane < 16) {
            float tsum = 0.f;
#pragma unroll
            for (int p = 0; p < 16; ++p) tsum += ssp[p][lane];
            rrow[lane] = 1.0f / sqrtf(tsum / (float)K + in.eps);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);   // this wave's LDS writes (lgkmcnt 0) before reading rrow
        __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
#pragma unroll
        for (int w = 0; w < NW - 1; ++w) {
            const float4v v = red[w][t][lane];
            acc[t][0] += v[0];
            acc[t][1] += v[1];
            acc[t][2] += v[2];
            acc[t][3] += v[3];
        }
        if (norm)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[t][i] *= rrow[4 * j + i];
        epilogue<EPI>(o, bx * T + t, N, j, c16, sl, pos, pre[t], acc[t], xep);
    }
}

template <int EPI, int T, int NW, int U>
__global__ __launch_bounds__(64 * NW) void k_mm16(const TiledMat W, const MmIn in, const Mm16Out o)
{
    mm16_block<EPI, T, NW, U>(W, in, o, blockIdx.x, gridDim.y, blockIdx.y);
}

// ---- the QKV product fused with the attention --------------------------------------------------
// One workgroup (four waves) per (head h, row b): the split-KV attention of attention.hip with the
// whole cache in one item (n_ctx <= 512), each wave taking key tiles wave, wave + 4, ...  The rows
// of the positions before the new one were written by earlier launches; the new position's key
// and value, and the query, come from the exchange words the product's workgroups publish in the
// same launch.  The first tile of each wave is loaded before the wait, so it streams in while the
// product finishes elsewhere.
template <int HD, int TILE>
__device__ __forceinline__ void attn16_item(const AttnArgs& a, const int h, const int b, const uint64_t* xq, const int ldx,
                                            const uint32_t ep, const long long limit, uint32_t* abort_word)
{
    constexpr int NWV = 4;
    constexpr int LPK = HD / 8;           // lanes per key, 8 dims (16 bytes) each
    constexpr int KPI = 64 / LPK;         // keys per load instruction
    constexpr int R = TILE / KPI;         // load rounds per tile
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int pos = a.pos ? ld_uniform(a.pos) : a.n_keys - 1;   // the new position
    const int n_keys = pos + 1;
    const int g = h / (a.H / a.Hkv);
    const int c = lane % LPK, kq = lane / LPK;
    const size_t head_off = ((size_t)b * a.Hkv + g) * a.n_ctx * HD;
    __shared__ float ow[NWV][HD];
    __shared__ float mw[NWV], lw[NWV];
    __shared__ float qs[HD];
    __shared__ __align__(16) _Float16 kn[HD], vn[HD];
    __shared__ int bail;

    auto load_tile = [&](int tile, uint4 (&kr)[R], uint4 (&vr)[R]) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int key = min(tile * TILE + r * KPI + kq, pos);   // the slot of pos itself is replaced below
            kr[r] = *(const uint4*)(a.k + head_off + (size_t)key * HD + c * 8);
            vr[r] = *(const uint4*)(a.v + head_off + (size_t)key * HD + c * 8);
        }
    };
    uint4 kr[R], vr[R];
    int tile = wave;
    load_tile(tile, kr, vr);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // wave 0 polls the query of head h and the new key and value of kv head g (row b)
    if (wave == 0) {
        constexpr int NQ = 3 * HD / 64;
        const int qd = a.H * HD, kd = a.Hkv * HD;
        auto addr = [&](int i) -> const uint64_t* {
            const int e = lane + 64 * i, part = e / HD, d = e - part * HD;
            const int col = part == 0 ? h * HD + d : (part == 1 ? qd : qd + kd) + g * HD + d;
            return xq + (size_t)b * ldx + col;
        };
        uint64_t w[NQ];
#pragma unroll
        for (int i = 0; i < NQ; ++i) w[i] = xchg::load(addr(i));
        const bool ok = xchg::settle_n(w, NQ, addr, ep, limit, abort_word);
        const float qscale = 1.4426950408889634f / sqrtf((float)HD);   // log2(e) / sqrt(hd): exp2 softmax
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int e = lane + 64 * i, part = e / HD, d = e - part * HD;
            const float v = xchg::value(w[i]);
            if (part == 0) qs[d] = v * qscale;
            else if (part == 1) kn[d] = (_Float16)v;
            else vn[d] = (_Float16)v;
        }
        if (lane == 0) bail = ok ? 0 : 1;
        if (!ok && lane == 0) xchg::raise_abort(abort_word);
    }
    __syncthreads();
    if (bail) return;
    float q[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = qs[c * 8 + e];
    const uint4 knew = *(const uint4*)&kn[c * 8], vnew = *(const uint4*)&vn[c * 8];

    // online softmax over this wave's tiles (log2 domain)
    float m = -INFINITY, l = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (; tile * TILE < n_keys; tile += NWV) {
        if (tile != wave) load_tile(tile, kr, vr);
        float sc[R];
        float mt = -INFINITY;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int key = tile * TILE + r * KPI + kq;
            if (key == pos) {
                kr[r] = knew;
                vr[r] = vnew;
            }
            const __half2* kh = (const __half2*)&kr[r];
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float2 f = __half22float2(kh[e]);
                acc = fmaf(f.x, q[2 * e], acc);
                acc = fmaf(f.y, q[2 * e + 1], acc);
            }
            acc = group_sum(acc, LPK);
            sc[r] = key < n_keys ? acc : -INFINITY;
            mt = fmaxf(mt, sc[r]);
        }
        mt = wave_max(mt);
        const float mn = fmaxf(m, mt);
        const float rs = exp2f(m - mn);   // 0 for the first tile (m = -inf)
        l *= rs;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] *= rs;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const bool valid = tile * TILE + r * KPI + kq < n_keys;
            const float p = valid ? exp2f(sc[r] - mn) : 0.f;
            l += p;
            const uint4 vv = valid ? vr[r] : make_uint4(0u, 0u, 0u, 0u);
            const __half2* vh = (const __half2*)&vv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float2 f = __half22float2(vh[e]);
                o[2 * e] = fmaf(p, f.x, o[2 * e]);
                o[2 * e + 1] = fmaf(p, f.y, o[2 * e + 1]);
            }
        }
        m = mn;
    }
    // every key's p is held by its LPK lanes: the wave sum counts it LPK times (exact scaling)
    l = wave_sum(l) * (1.0f / LPK);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        if constexpr (LPK == 8) o[e] += dpp_mov<0x128>(o[e]);   // lanes i and i ^ 8 share dims
        o[e] = swap32_sum(swap16_sum(o[e]));
    }
    if (kq == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) ow[wave][c * 8 + e] = o[e];
    }
    if (lane == 0) {
        mw[wave] = m;
        lw[wave] = l;
    }
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWV; ++w) M = fmaxf(M, mw[w]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) L = fmaf(lw[w], exp2f(mw[w] - M), L);   // a wave without keys adds 0
    const float inv = 1.0f / L;
    for (int i = threadIdx.x; i < HD; i += 64 * NWV) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < NWV; ++w) acc = fmaf(ow[w][i], exp2f(mw[w] - M), acc);
        const float y = acc * inv;
        const _Float16 hi = (_Float16)y;
        const size_t idx = il_act(b, h * HD + i);
        ((TSD_GLOBAL _Float16*)a.act_hi)[idx] = hi;
        ((TSD_GLOBAL _Float16*)a.act_lo)[idx] = (_Float16)(y - (float)hi);
    }
}

// STACKED = false: workgroups [0, n_gemm) take the QKV product (one 16-row tile each), the ones
// after them one attention item per (head, row).  STACKED = true (short caches, whose items have
// little to preload): workgroup w takes product tile w, then item w, on a grid of
// max(n_gemm, items); the products never wait, so every item's words arrive once the grid's
// workgroups are resident together (one per compute unit here).
template <int U, int HD, int TILE, bool STACKED>
__global__ __launch_bounds__(256) void k_qkv_attn(const TiledMat W, const MmIn in, const Mm16Out o, const AttnArgs a,
                                                  const int n_gemm, const long long limit, uint32_t* abort_word)
{
    if ((int)blockIdx.x < n_gemm) {
        mm16_block<MM_QKV_ROPE, 1, 4, U>(W, in, o, blockIdx.x, 1, 0);
        if (!STACKED) return;
    }
    // the R = H / Hkv query heads of one (row, kv head) read the same cache rows: their items
    // are 8 workgroups apart, which puts them on one XCD and lets its L2 serve the second read
    // (when the (row, kv head) pairs come in multiples of 8; else items in (row, head) order)
    const int item = STACKED ? (int)blockIdx.x : (int)blockIdx.x - n_gemm, R = a.H / a.Hkv;
    if (STACKED && item >= a.H * a.B) return;
    int h, b;
    if ((a.B * a.Hkv) % 8 == 0) {
        const int pair = item / (8 * R) * 8 + item % 8, r = item / 8 % R;
        b = pair / a.Hkv;
        h = (pair - b * a.Hkv) * R + r;
    } else {
        h = item % a.H;
        b = item / a.H;
    }
    const uint32_t ep = (uint32_t)ld_uniform((const int*)o.xctr) * (uint32_t)FUSE_EPOCHS + (uint32_t)o.xidx + 1u;
    attn16_item<HD, TILE>(a, h, b, o.xq, o.ldx, ep, limit, abort_word);
}

// ---- repack a canonical 8-bit affine matrix into the tiled layout --------------------------
// one thread per (source row, group)
__global__ void k_pack_tiled(const uint8_t* __restrict__ src, int N, int K, uint8_t* __restrict__ dq,
                             uint32_t* __restrict__ dsb, int mode, int hd, int row0)
{
    const int G = K / 64;
    const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long long)N * G) return;
    const int r = (int)(idx / G), g = (int)(idx - (long long)r * G);
    const int dr = place_row(r, mode, hd, row0), t = dr >> 4, c = dr & 15;
    const uint8_t* qs = src + (size_t)r * K + (size_t)g * 64;
    uint8_t* blk = dq + ((size_t)t * G + g) * 1024;
    for (int kk = 0; kk < 64; ++kk) {
        const int jj = (kk & 31) >> 3, e = 8 * (kk >> 5) + (kk & 7);
        blk[(jj * 16 + c) * 16 + e] = qs[kk];
    }
    const uint8_t* s = src + (size_t)N * K + ((size_t)r * G + g) * 2;
    const uint8_t* b = src + (size_t)N * K + (size_t)N * G * 2 + ((size_t)r * G + g) * 2;
    dsb[((size_t)t * G + g) * 16 + c] = (uint32_t)(s[0] | (s[1] << 8)) | ((uint32_t)(b[0] | (b[1] << 8)) << 16);
}

// ---- a norm's input, one row per 256-thread workgroup ------------------------------------------
constexpr int RP = MM_MAX_K / 256;   // elements per thread

// id0 >= 0: the id of table 0 (ROW_EMB), else read from codes.  Rows b >= B write zeros.
// red: 4 floats of LDS; ids: 16 ints of LDS
// Every load is issued unconditionally (clamped into the row) ahead of its first use: the gains
// before the row's reduction, the embedding rows four tables at a time (summed in table order), so
// that a row costs a few memory round trips rather than one per element.
__device__ void row_prep(const RowPrep& p, int b, int id0, float* red, int* ids)
{
    const int t = threadIdx.x, K = p.K;
    const bool live = b < p.B;
    auto col = [&](int i) { return min(t + 256 * i, K - 1); };
    float gs[RP], ga[RP];   // the ROW_NORMED gain and the operand's gain
    if (p.src == ROW_NORMED) {
#pragma unroll
        for (int i = 0; i < RP; ++i) gs[i] = glb(p.g_src)[col(i)];
    }
    if (p.g) {
#pragma unroll
        for (int i = 0; i < RP; ++i) ga[i] = glb(p.g)[col(i)];
    }
    float v[RP];
#pragma unroll
    for (int i = 0; i < RP; ++i) v[i] = 0.f;
    if (p.src == ROW_EMB) {   // uniform over the workgroup
        if (live && t < p.n_tab) {
            const int id = (t == 0 && id0 >= 0) ? id0 : p.codes[(size_t)b * p.ld_codes + t];
            ids[t] = id < 0 ? 0 : (id >= p.tab_rows[t] ? p.tab_rows[t] - 1 : id);
        }
        __syncthreads();
    }
    if (live) {
        if (p.src == ROW_EMB) {
            constexpr int TG = 4;   // tables per round
            for (int c0 = 0; c0 < p.n_tab; c0 += TG) {
                float e[TG][RP];
#pragma unroll
                for (int u = 0; u < TG; ++u) {
                    const int c = min(c0 + u, p.n_tab - 1);
                    const auto row = glb(p.tab[c]) + (size_t)ids[c] * K;
#pragma unroll
                    for (int i = 0; i < RP; ++i) e[u][i] = row[col(i)];
                }
#pragma unroll
                for (int u = 0; u < TG; ++u)
                    if (c0 + u < p.n_tab)
#pragma unroll
                        for (int i = 0; i < RP; ++i) v[i] += e[u][i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < RP; ++i)
                v[i] = p.src == ROW_MAJOR ? glb(p.rows_src)[(size_t)b * K + col(i)] : glb(p.rows_src)[il_x(b, col(i))];
        }
#pragma unroll
        for (int i = 0; i < RP; ++i)
            if (t + 256 * i >= K) v[i] = 0.f;
    }
    if (p.src == ROW_NORMED) {   // uniform over the workgroup
        float q2 = 0.f;
#pragma unroll
        for (int i = 0; i < RP; ++i) q2 = fmaf(v[i], v[i], q2);
        const float r = 1.0f / sqrtf(block_sum256(q2, red) / (float)K + p.eps);
#pragma unroll
        for (int i = 0; i < RP; ++i) v[i] *= gs[i] * r;
    }
    float q2 = 0.f;
#pragma unroll
    for (int i = 0; i < RP; ++i) {
        const int k = t + 256 * i;
        if (k >= K) continue;
        if (p.x && live) glb(p.x)[il_x(b, k)] = v[i];
        put_hilo(p.act, il_act(b, k), p.g ? v[i] * ga[i] : v[i]);
        q2 = fmaf(v[i], v[i], q2);
    }
    if (p.ssq) {
        q2 = block_sum256(q2, red);
        if (t == 0 && live) glb(p.ssq)[b] = q2;
    }
}

__global__ __launch_bounds__(256) void k_row_prep(const RowPrep p)
{
    __shared__ float red[4];
    __shared__ int ids[16];
    row_prep(p, blockIdx.x, -1, red, ids);
}

// ---- the code of every row, then that row's next input ----------------------------------------
__global__ __launch_bounds__(256) void k_pick(const PickArgs a)
{
    extern __shared__ uint32_t keys[];   // draw only: the row's logits as ordered keys, then the
                                         // history's bit set
    __shared__ samp::Scratch S;
    __shared__ unsigned long long bk[4];
    __shared__ float red[4];
    __shared__ int ids[16];
    __shared__ int picked;
    const int b = blockIdx.x, t = threadIdx.x;
    if (a.err && ld_uniform((const int*)a.err)) return;   // a rejected input: the state stays as it was
    const float* l = a.logits + (size_t)b * a.ld_l;
    const int pos = *a.posp;
    const int cur = a.seq ? a.code[(size_t)b * a.ld_code] : -1;   // read before the pick overwrites it
    if (a.draw) {
        uint32_t* seen = keys + samp::key_words(a.n);
        const bool pen = a.seq && a.ch.penalty != 1.f;
        if (pen) samp::build_seen<256>(seen, a.n, a.seq + b, a.B, pos, cur);
        const uint32_t* sp = pen ? seen : nullptr;
        samp::load_keys<256>(keys, l, a.n, a.ch, sp);
        __syncthreads();
        const float u = samp::uniform24(a.seed, (uint32_t)b, (uint32_t)pos, (uint32_t)a.pass);
        const int id = samp::chain_draw<256>(keys, a.n, a.ch, u, S, sp);
        if (t == 0) picked = id;
    } else {
        // the loads of a round are all issued (clamped addresses) before the first is used
        constexpr int R = 8;
        unsigned long long best = 0ull;
        for (int base = 0; base < a.n; base += 256 * R) {
            float v[R];
#pragma unroll
            for (int j = 0; j < R; ++j) v[j] = l[min(base + j * 256 + t, a.n - 1)];
#pragma unroll
            for (int j = 0; j < R; ++j) {
                const int i = base + j * 256 + t;
                const unsigned long long key = ((unsigned long long)float_order_key(v[j]) << 32) | (0xFFFFFFFFu - (uint32_t)i);
                best = (i < a.n && key > best) ? key : best;
            }
        }
        best = wave_max_u64(best);
        if ((t & 63) == 0) bk[t >> 6] = best;
        __syncthreads();
        if (t == 0) {
            unsigned long long m = bk[0];
            for (int i = 1; i < 4; ++i) m = bk[i] > m ? bk[i] : m;
            picked = (int)(0xFFFFFFFFu - (uint32_t)m);
        }
    }
    __syncthreads();
    const int id = picked;
    if (t == 0) {
        if (a.seq) a.seq[(size_t)pos * a.B + b] = cur;
        a.code[(size_t)b * a.ld_code] = id;
    }
    if (a.prep.src >= 0) row_prep(a.prep, b, id, red, ids);
}

__global__ void k_il_to_rows(const float* __restrict__ src, int B, int K, float* __restrict__ dst)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= B * K) return;
    const int b = i / K, k = i - b * K;
    dst[i] = src[il_x(b, k)];
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
__global__ void k_frame_done(const int* __restrict__ codes, int n, int* hist, int* pos, int* seq, int B, int C,
                             const uint32_t* err, uint32_t* fctr)
{
    // the epoch counter of the fused launches advances every frame, a rejected one included, so
    // that no later launch can take a stale exchange word for its own
    if (fctr && threadIdx.x == 0) *fctr += 1u;
    if (err && ld_uniform((const int*)err)) return;   // a rejected input: the state stays as it was
    const int p = *pos;
    for (int i = threadIdx.x; i < n; i += blockDim.x) hist[(size_t)p * n + i] = codes[i];
    if (seq)
        for (int b = threadIdx.x; b < B; b += blockDim.x) seq[(size_t)p * B + b] = codes[(size_t)b * C];
    __syncthreads();
    if (threadIdx.x == 0) *pos = p + 1;
}

__global__ void k_bump_u32(uint32_t* p)
{
    if (threadIdx.x == 0) *p += 1u;
}

template <int EPI, int T, int NW, int U>
hipError_t go(const TiledMat& W, const MmIn& in, int splits, const Mm16Out& o, hipStream_t st)
{
    const int tiles = (W.N + 15) / 16;
    const dim3 grid((tiles + T - 1) / T, splits);
    hipLaunchKernelGGL((k_mm16<EPI, T, NW, U>), grid, dim3(64 * NW), 0, st, W, in, o);
    return hipGetLastError();
}

// The launch shape: a tall matrix takes four tiles per workgroup (its operand fragment serves
// all four; 131072 x 2048 streams at ~5.2 TB/s this way against 4.2 with eight waves of two
// groups); otherwise one tile, with enough waves (up to twelve) that each reduces at most four
// groups of its slice in one round of loads.
template <int EPI>
hipError_t launch_e(const TiledMat& W, const MmIn& in, int splits, const Mm16Out& o, hipStream_t st)
{
    const int tiles = (W.N + 15) / 16, gs = W.K / 64 / splits;
    if (tiles >= 1024) return go<EPI, 4, 4, 4>(W, in, splits, o, st);
    if (gs <= 16) return go<EPI, 1, 4, 4>(W, in, splits, o, st);
    if (gs <= 32) return go<EPI, 1, 8, 4>(W, in, splits, o, st);
    return go<EPI, 1, 12, 4>(W, in, splits, o, st);   // (beyond 48 groups a wave takes two rounds)
}

}  // namespace

bool mm16_supported(int N, int K) { return N > 0 && K > 0 && K % 64 == 0 && K <= MM_MAX_K; }

hipError_t launch_mm16(int epi, const TiledMat& W, const MmIn& in, int splits, const Mm16Out& o, hipStream_t st)
{
    if (!mm16_supported(W.N, W.K) || splits < 1 || splits > MM_MAX_SPLIT || splits > W.K / 64 || o.rows < 1 ||
        o.rows > MM_ROWS || in.rows < 1 || in.rows > MM_ROWS || !in.a.hi || !in.a.lo)
        return hipErrorInvalidValue;
    if (epi != MM_STORE && splits != 1) return hipErrorInvalidValue;       // the other epilogues need the whole sum
    if (in.ssq && (splits != 1 || in.n_ssq < 1 || in.n_ssq > MM_MAX_SSQ)) return hipErrorInvalidValue;
    if (epi == MM_RESID && o.next.hi && (!o.g_next || !o.next.lo)) return hipErrorInvalidValue;
    if ((epi == MM_SWIGLU || epi == MM_QKV_ROPE) && W.N % 2) return hipErrorInvalidValue;
    if (epi == MM_STORE) return launch_e<MM_STORE>(W, in, splits, o, st);
    if (epi == MM_RESID) return launch_e<MM_RESID>(W, in, splits, o, st);
    if (epi == MM_SWIGLU) return launch_e<MM_SWIGLU>(W, in, splits, o, st);
    if (epi == MM_QKV_ROPE) return launch_e<MM_QKV_ROPE>(W, in, splits, o, st);
    return hipErrorInvalidValue;
}

bool qkv_attention_fits(const TiledMat& W, const AttnArgs& a)
{
    const int qd = a.H * a.hd, kd = a.Hkv * a.hd;
    return (a.hd == 64 || a.hd == 128) && attn_direct_fits(a.n_ctx) && a.Hkv > 0 && a.H % a.Hkv == 0 &&
           W.N == qd + 2 * kd && W.K / 64 <= 16 && mm16_supported(W.N, W.K) && a.B >= 1 && a.B <= MM_ROWS;
}

hipError_t launch_qkv_attention(const TiledMat& W, const MmIn& in, const Mm16Out& o, const AttnArgs& a, long long limit,
                                uint32_t* abort_word, hipStream_t st)
{
    // the product's shape as launch_mm16 runs it for K <= 1024 (one tile, four waves, four groups per round)
    if (!qkv_attention_fits(W, a) || !o.xq || !o.xctr || o.xidx < 0 || o.xidx >= FUSE_EPOCHS - 1 || o.ldx != W.N ||
        !a.act_hi || !a.act_lo || !abort_word || o.rows < 1 || o.rows > MM_ROWS || in.rows < 1 || in.rows > MM_ROWS ||
        !in.a.hi || !in.a.lo || (in.ssq && (in.n_ssq < 1 || in.n_ssq > MM_MAX_SSQ)))
        return hipErrorInvalidValue;
    const int n_gemm = (W.N + 15) / 16, items = a.H * a.B;
    // short caches (the code predictor's): product and item stacked on one workgroup
    const dim3 grid(n_gemm + items), stacked(n_gemm > items ? n_gemm : items);
    if (a.hd == 64) {
        if (a.n_ctx <= 64) hipLaunchKernelGGL((k_qkv_attn<4, 64, 16, true>), stacked, dim3(256), 0, st, W, in, o, a, n_gemm, limit, abort_word);
        else hipLaunchKernelGGL((k_qkv_attn<4, 64, 64, false>), grid, dim3(256), 0, st, W, in, o, a, n_gemm, limit, abort_word);
    } else {
        if (a.n_ctx <= 64) hipLaunchKernelGGL((k_qkv_attn<4, 128, 16, true>), stacked, dim3(256), 0, st, W, in, o, a, n_gemm, limit, abort_word);
        else hipLaunchKernelGGL((k_qkv_attn<4, 128, 32, false>), grid, dim3(256), 0, st, W, in, o, a, n_gemm, limit, abort_word);
    }
    return hipGetLastError();
}

hipError_t launch_pack_tiled(const void* src, int N, int K, void* dst_base, int dst_N, int dst_row0, int mode, int hd,
                             hipStream_t st)
{
    if (K % 64 || N <= 0) return hipErrorInvalidValue;
    TiledMat T = tiled_view(dst_base, dst_N, K);
    const long long n = (long long)N * (K / 64);
    hipLaunchKernelGGL(k_pack_tiled, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, (const uint8_t*)src, N, K,
                       (uint8_t*)T.q, (uint32_t*)T.sb, mode, hd, dst_row0);
    return hipGetLastError();
}

static bool row_prep_ok(const RowPrep& p)
{
    return p.K > 0 && p.K % 64 == 0 && p.K <= MM_MAX_K && p.B >= 1 && p.B <= MM_ROWS && p.act.hi && p.act.lo &&
           (p.src != ROW_EMB || (p.n_tab >= 1 && p.n_tab <= 16)) && (p.src != ROW_NORMED || p.g_src) &&
           (p.src == ROW_EMB || p.rows_src);
}

hipError_t launch_row_prep(const RowPrep& p, hipStream_t st)
{
    if (!row_prep_ok(p)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_row_prep, dim3(MM_ROWS), dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_pick(const PickArgs& a, hipStream_t st)
{
    if (a.n < 1 || a.B < 1 || a.B > MM_ROWS || (a.prep.src >= 0 && (!row_prep_ok(a.prep) || a.prep.B != a.B)))
        return hipErrorInvalidValue;
    if (!a.posp || (a.draw && (!sample_supported(a.n, a.ch.k) || !(a.ch.temperature > 0.f)))) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_pick, dim3(a.B), dim3(256), a.draw ? sample_lds_bytes(a.n) : 0, st, a);
    return hipGetLastError();
}

hipError_t launch_il_to_rows(const float* src, int B, int K, float* dst, hipStream_t st)
{
    const int n = B * K;
    hipLaunchKernelGGL(k_il_to_rows, dim3((n + 255) / 256), dim3(256), 0, st, src, B, K, dst);
    return hipGetLastError();
}

hipError_t launch_merge16(const float* part, int B, int H, int hd, int max_split, const int* posp, int n_keys_value,
                          const Act16& a, hipStream_t st)
{
    if (B < 1 || B > MM_ROWS) return hipErrorInvalidValue;
    const int n = B * H * hd;
    hipLaunchKernelGGL(k_merge16, dim3((n + 255) / 256), dim3(256), 0, st, part, H, hd, max_split, posp, n_keys_value, n, a);
    return hipGetLastError();
}

hipError_t launch_sum_slices(const float* part, int S, long long slice, float* y, long long n, hipStream_t st)
{
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_sum_slices, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part, S, slice, y, n);
    return hipGetLastError();
}

hipError_t launch_frame_done(const int* codes, int n, int* hist, int* pos, int* seq, int B, int C, const uint32_t* err,
                             uint32_t* fctr, hipStream_t st)
{
    hipLaunchKernelGGL(k_frame_done, dim3(1), dim3(256), 0, st, codes, n, hist, pos, seq, B, C, err, fctr);
    return hipGetLastError();
}

hipError_t launch_bump_u32(uint32_t* p, hipStream_t st)
{
    hipLaunchKernelGGL(k_bump_u32, dim3(1), dim3(64), 0, st, p);
    return hipGetLastError();
}

}  // namespace tsd
