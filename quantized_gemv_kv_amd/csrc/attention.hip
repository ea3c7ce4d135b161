// attention.hip — split-KV flash-decode attention of one new token over an fp16 KV cache.
//
// What it computes: o_h = softmax(q_h K^T / sqrt(hd)) V for every query head h over cached
// positions 0..n_keys-1 of KV head h / (H/Hkv); a single new token sees every cached position,
// so there is no mask ("Chatterbox -> ggml Port: Development Journal", §3.13: flash attention
// over a cache stored the way it is read — head-dim fastest, then position, then head).
//
// Mapping onto CDNA4:
//   * the keys of a head are cut into chunks of 256 positions, one 4-wave workgroup per
//     (chunk, head, row), one 64-key tile per wave; a cache of at most 512 positions can instead
//     be covered by one workgroup (16-key tiles up to 64 positions, eight waves beyond 256);
//   * lane layout: hd/8 lanes share a key and each holds 8 of its dims (16 bytes), so every load
//     instruction reads 1 KB of consecutive K (or V) rows; the score is a DPP reduction inside
//     the key's lane group and the weighted sum stays in VGPRs, reduced across key groups with a
//     row rotation and the gfx950 row swaps at the end (no LDS per key);
//   * log2-domain online softmax: each wave keeps (running max m, sum l, unnormalised o); the
//     four waves merge in LDS and the workgroup writes one partial per chunk;
//   * the partials of a head are merged with the log-sum-exp rule
//       M = max m_i,  L = sum l_i 2^(m_i - M),  o = sum o_i 2^(m_i - M) / L
//     by whoever consumes the attention output: in the decode step that is the prologue of the
//     output-projection GEMV (so the merge costs neither a launch nor a device-wide fence);
//     the standalone operator runs a small merge kernel; when a cache fits one chunk (the code
//     predictor's) the workgroup normalises its own result and writes it as the fp16 hi/lo
//     operand of the batched output projection;
//   * the grid is sized for the full context and chunks past the current length exit at once,
//     so one launch configuration serves every position (the step is replayed from a graph).
#include <math.h>

#include "kernels.h"

namespace tsd {
namespace {


// sum over the lanes that hold the same dims of different keys (key groups of LPK lanes)
template <int LPK>
__device__ __forceinline__ float keygroup_sum(float v)
{
    if constexpr (LPK == 8) v += dpp_mov<0x128>(v);   // row_ror:8 (lane i and i^8 share dims)
    v = swap16_sum(v);
    v = swap32_sum(v);
    return v;
}

// NWAVE waves per workgroup, TILE keys per wave: one workgroup covers a chunk of NWAVE * TILE
// positions (ATTN_CHUNK for the split form; the whole cache for the operand-writing form)
template <int HD, int NWAVE, int TILE>
__global__ __launch_bounds__(64 * NWAVE) void k_attn(const AttnArgs a)
{
    constexpr int LPK = HD / 8;           // lanes per key, 8 dims (16 bytes) each
    constexpr int KPI = 64 / LPK;         // keys per load instruction (1 KB contiguous)
    constexpr int R = TILE / KPI;         // load rounds per tile
    constexpr int PS = HD + 4;            // partial stride (16-byte aligned)
    constexpr int CHUNK = NWAVE * TILE;
    const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n_keys = a.pos ? ld_uniform(a.pos) + 1 + a.pos_add : a.n_keys;
    if (s * CHUNK >= n_keys) return;
    const int g = h / (a.H / a.Hkv);
    const int k0 = s * CHUNK + wave * TILE;               // first key of this wave's tile
    const int c = lane % LPK, kq = lane / LPK;            // dims 8c..8c+7 of key k0 + r*KPI + kq
    const size_t head_off = ((size_t)b * a.Hkv + g) * a.n_ctx * HD;

    __shared__ float ow[NWAVE][HD];
    __shared__ float mw[NWAVE], lw[NWAVE];

    // the tile's K and V, coalesced: round r reads keys k0 + r*KPI .. +KPI-1 (1 KB each);
    // unconditional loads from clamped addresses, invalid keys masked after
    // (clamped to the last valid key, so that a partial tile fetches nothing beyond it)
    uint4 kr[R], vr[R];
    const int klast = n_keys - 1;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int key = min(k0 + r * KPI + kq, klast);
        kr[r] = *(const uint4*)(a.k + head_off + (size_t)key * HD + c * 8);
        vr[r] = *(const uint4*)(a.v + head_off + (size_t)key * HD + c * 8);
    }
    asm volatile("" ::: "memory");   // keep every load above: all of the tile in flight at once
    __builtin_amdgcn_sched_barrier(0);
    // this lane's 8 query dims, pre-scaled by log2(e)/sqrt(hd) so that the softmax runs on exp2
    const float qscale = 1.4426950408889634f / sqrtf((float)HD);
    const float4* qp = (const float4*)(a.q + (size_t)b * a.ldq + (size_t)h * HD + c * 8);
    const float4 qa = qp[0], qb = qp[1];
    const float q[8] = {qa.x * qscale, qa.y * qscale, qa.z * qscale, qa.w * qscale,
                        qb.x * qscale, qb.y * qscale, qb.z * qscale, qb.w * qscale};

    // scores: 8-dim partial dots, reduced over the key's LPK lanes
    float sc[R];
    float mloc = -INFINITY;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const __half2* kh = (const __half2*)&kr[r];
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float2 f = __half22float2(kh[e]);
            acc = fmaf(f.x, q[2 * e], acc);
            acc = fmaf(f.y, q[2 * e + 1], acc);
        }
        acc = group_sum(acc, LPK);
        sc[r] = k0 + r * KPI + kq < n_keys ? acc : -INFINITY;
        mloc = fmaxf(mloc, sc[r]);
    }
    const float m = wave_max(mloc);
    float lsum = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const bool valid = k0 + r * KPI + kq < n_keys;
        const float p = valid ? exp2f(sc[r] - m) : 0.f;
        lsum += p;
        const uint4 vv = valid ? vr[r] : make_uint4(0u, 0u, 0u, 0u);   // stale rows could hold NaN
        const __half2* vh = (const __half2*)&vv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float2 f = __half22float2(vh[e]);
            o[2 * e] = fmaf(p, f.x, o[2 * e]);
            o[2 * e + 1] = fmaf(p, f.y, o[2 * e + 1]);
        }
    }
    // every key's p is held by its LPK lanes: the wave sum counts it LPK times (exact scaling)
    const float l = wave_sum(lsum) * (1.0f / LPK);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = keygroup_sum<LPK>(o[e]);
    if (kq == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) ow[wave][c * 8 + e] = o[e];
    }
    if (lane == 0) {
        mw[wave] = k0 < n_keys ? m : -INFINITY;
        lw[wave] = l;
    }
    __syncthreads();

    // merge the four tiles of this chunk into one partial
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) M = fmaxf(M, mw[w]);
    if (a.act_hi) {   // the only chunk: normalise here and write the next GEMM's operand
        float L = 0.f;
#pragma unroll
        for (int w = 0; w < NWAVE; ++w) L = fmaf(lw[w], exp2f(mw[w] - M), L);
        const float inv = 1.0f / L;
        for (int i = threadIdx.x; i < HD; i += 64 * NWAVE) {
            float acc = 0.f;
#pragma unroll
            for (int w = 0; w < NWAVE; ++w) acc = fmaf(ow[w][i], exp2f(mw[w] - M), acc);
            const float y = acc * inv;
            const _Float16 hi = (_Float16)y;
            const size_t idx = il_act(b, h * HD + i);
            ((TSD_GLOBAL _Float16*)a.act_hi)[idx] = hi;
            ((TSD_GLOBAL _Float16*)a.act_lo)[idx] = (_Float16)(y - (float)hi);
        }
        return;
    }
    float* part = a.part + (((size_t)b * a.H + h) * attn_max_split(a.n_ctx) + s) * PS;
    for (int i = threadIdx.x; i < HD; i += 64 * NWAVE) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < NWAVE; ++w) acc = fmaf(ow[w][i], exp2f(mw[w] - M), acc);
        part[i] = acc;
    }
    if (threadIdx.x == 0) {
        float L = 0.f;
#pragma unroll
        for (int w = 0; w < NWAVE; ++w) L = fmaf(lw[w], exp2f(mw[w] - M), L);
        part[HD] = M;
        part[HD + 1] = L;
    }
}

// merge of the chunk partials for the standalone operator: one thread per output element
__global__ void k_attn_merge(const float* __restrict__ part, float* __restrict__ out, int B, int H, int hd,
                             int ldo, int max_split, int n_split)
{
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= B * H * hd) return;
    const int i = idx % hd, bh = idx / hd, b = bh / H, h = bh % H;
    const int PS = hd + 4;
    const float* pb = part + (size_t)bh * max_split * PS;
    float M = -INFINITY;
    for (int t = 0; t < n_split; ++t) M = fmaxf(M, pb[(size_t)t * PS + hd]);
    float L = 0.f, O = 0.f;
    for (int t = 0; t < n_split; ++t) {
        const float wgt = exp2f(pb[(size_t)t * PS + hd] - M);
        L = fmaf(pb[(size_t)t * PS + hd + 1], wgt, L);
        O = fmaf(pb[(size_t)t * PS + i], wgt, O);
    }
    out[(size_t)b * ldo + (size_t)h * hd + i] = O / L;
}

}  // namespace

size_t attn_part_bytes(int B, int H, int n_ctx, int hd)
{
    return (size_t)B * H * attn_max_split(n_ctx) * (hd + 4) * sizeof(float);
}

template <int HD>
hipError_t launch_hd(const AttnArgs& a, hipStream_t st)
{
    const dim3 one(1, a.H, a.B);
    if (a.act_hi) {   // one workgroup covers the whole cache
        if (a.n_ctx <= 64) hipLaunchKernelGGL((k_attn<HD, 4, 16>), one, dim3(256), 0, st, a);
        else if (a.n_ctx <= 256) hipLaunchKernelGGL((k_attn<HD, 4, 64>), one, dim3(256), 0, st, a);
        else hipLaunchKernelGGL((k_attn<HD, 8, 64>), one, dim3(512), 0, st, a);
    } else {
        hipLaunchKernelGGL((k_attn<HD, 4, 64>), dim3(attn_max_split(a.n_ctx), a.H, a.B), dim3(256), 0, st, a);
    }
    return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t st)
{
    if (a.act_hi && (!attn_direct_fits(a.n_ctx) || !a.act_lo)) return hipErrorInvalidValue;
    if (a.hd == 64) return launch_hd<64>(a, st);
    if (a.hd == 128) return launch_hd<128>(a, st);
    return hipErrorInvalidValue;
}

hipError_t launch_attention_merge(const AttnArgs& a, int n_keys, hipStream_t st)
{
    const int n = a.B * a.H * a.hd;
    const int n_split = (n_keys + ATTN_CHUNK - 1) / ATTN_CHUNK;
    hipLaunchKernelGGL(k_attn_merge, dim3((n + 255) / 256), dim3(256), 0, st, a.part, a.out, a.B, a.H, a.hd, a.ldo,
                       attn_max_split(a.n_ctx), n_split);
    return hipGetLastError();
}

}  // namespace tsd
