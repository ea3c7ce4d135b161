// attention.hip — split-KV flash-decode attention of one new token over an fp16 KV cache.
//
// What it computes: o_h = softmax(q_h K^T / sqrt(hd)) V for every query head h over cached
// positions 0..n_keys-1 of KV head h / (H/Hkv); a single new token sees every cached position,
// so there is no mask ("Chatterbox -> ggml Port: Development Journal", §3.13: flash attention
// over a cache stored the way it is read — head-dim fastest, then position, then head).
//
// Mapping onto CDNA4:
//   * the keys of a head are cut into tiles of 64 positions; one wave64 workgroup per
//     (tile, head, row): lane j scores key j of its tile (its 128/256-byte key row is read with
//     dwordx4 loads), while the whole V tile is fetched in the same burst, coalesced, and
//     staged in LDS for the weighted sum;
//   * each tile leaves an unnormalised partial (o, running max m, sum l) in log2 domain;
//   * the last workgroup of a head to finish (an atomic ticket) merges the partials with the
//     log-sum-exp rule  M = max m_i,  L = sum l_i 2^(m_i - M),  o = sum o_i 2^(m_i - M) / L,
//     so the merge costs no extra launch;
//   * the grid is sized for the full context and tiles past the current length exit at once,
//     so one launch configuration serves every position (the step is replayed from a graph).
#include <math.h>

#include "kernels.h"

namespace tsd {
namespace {

constexpr int TILE = 64;

template <int HD>
__global__ __launch_bounds__(64) void k_attn(const AttnArgs a)
{
    constexpr int NV = HD / 8;          // uint4 per key row
    constexpr int DPL = HD / 64;        // output dims per lane
    const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
    const int n_keys = a.pos ? *a.pos + 1 + a.pos_add : a.n_keys;
    const int n_split = (n_keys + TILE - 1) / TILE;
    if (s >= n_split) return;
    const int g = h / (a.H / a.Hkv);
    const size_t head_off = ((size_t)b * a.Hkv + g) * a.n_ctx * HD;
    const __half* Kt = a.k + head_off + (size_t)s * TILE * HD;
    const __half* Vt = a.v + head_off + (size_t)s * TILE * HD;
    const int nt = min(TILE, n_keys - s * TILE);   // keys in this tile

    __shared__ float qs[HD];
    __shared__ uint4 vt[TILE * NV];
    __shared__ float ps[TILE];

    // K row of this lane's key and the V tile, all in flight together
    uint4 kr[NV], vr[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        kr[i] = make_uint4(0u, 0u, 0u, 0u);
        if (lane < nt) kr[i] = ((const uint4*)(Kt + (size_t)lane * HD))[i];
        const int idx = i * 64 + lane;           // coalesced over the tile
        vr[i] = make_uint4(0u, 0u, 0u, 0u);
        if (idx / NV < nt) vr[i] = ((const uint4*)Vt)[idx];
    }
    // q, pre-scaled by log2(e)/sqrt(hd) so that the softmax runs on exp2
    const float qscale = 1.4426950408889634f / sqrtf((float)HD);
    const float* qh = a.q + (size_t)b * a.ldq + (size_t)h * HD;
#pragma unroll
    for (int i = 0; i < DPL; ++i) qs[lane + 64 * i] = qh[lane + 64 * i] * qscale;
    __syncthreads();

    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const __half2* kh = (const __half2*)&kr[i];
        const float4 q0 = *(const float4*)&qs[8 * i], q1 = *(const float4*)&qs[8 * i + 4];
        float2 f;
        f = __half22float2(kh[0]); acc = fmaf(f.x, q0.x, acc); acc = fmaf(f.y, q0.y, acc);
        f = __half22float2(kh[1]); acc = fmaf(f.x, q0.z, acc); acc = fmaf(f.y, q0.w, acc);
        f = __half22float2(kh[2]); acc = fmaf(f.x, q1.x, acc); acc = fmaf(f.y, q1.y, acc);
        f = __half22float2(kh[3]); acc = fmaf(f.x, q1.z, acc); acc = fmaf(f.y, q1.w, acc);
    }
    const float sc = lane < nt ? acc : -INFINITY;
    const float m = wave_max(sc);
    const float p = lane < nt ? exp2f(sc - m) : 0.f;
    const float l = wave_sum(p);

#pragma unroll
    for (int i = 0; i < NV; ++i) vt[i * 64 + lane] = vr[i];
    ps[lane] = p;
    __syncthreads();

    float o[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) o[i] = 0.f;
    const __half* vh = (const __half*)vt;
    for (int j = 0; j < nt; ++j) {
        const float pj = ps[j];
#pragma unroll
        for (int i = 0; i < DPL; ++i) o[i] = fmaf(pj, __half2float(vh[j * HD + lane + 64 * i]), o[i]);
    }

    const int max_split = (a.n_ctx + TILE - 1) / TILE;
    float* part = a.part + (((size_t)b * a.H + h) * max_split + s) * (HD + 2);
#pragma unroll
    for (int i = 0; i < DPL; ++i) part[lane + 64 * i] = o[i];
    if (lane == 0) {
        part[HD] = m;
        part[HD + 1] = l;
    }
    if (n_split == 1) {
        float* out = a.out + (size_t)b * a.ldo + (size_t)h * HD;
#pragma unroll
        for (int i = 0; i < DPL; ++i) out[lane + 64 * i] = o[i] / l;
        return;
    }

    // the last tile of this head to finish merges all partials
    __threadfence();
    unsigned int ticket = 0;
    if (lane == 0) ticket = atomicAdd(&a.cnt[b * a.H + h], 1u);
    ticket = __shfl(ticket, 0, 64);
    if (ticket != (unsigned)(n_split - 1)) return;
    __threadfence();
    const float* pb = a.part + ((size_t)b * a.H + h) * max_split * (HD + 2);
    float M = -INFINITY;
    for (int t = 0; t < n_split; ++t) M = fmaxf(M, pb[(size_t)t * (HD + 2) + HD]);
    float L = 0.f, O[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) O[i] = 0.f;
    for (int t = 0; t < n_split; ++t) {
        const float* pt = pb + (size_t)t * (HD + 2);
        const float wgt = exp2f(pt[HD] - M);
        L = fmaf(pt[HD + 1], wgt, L);
#pragma unroll
        for (int i = 0; i < DPL; ++i) O[i] = fmaf(pt[lane + 64 * i], wgt, O[i]);
    }
    float* out = a.out + (size_t)b * a.ldo + (size_t)h * HD;
#pragma unroll
    for (int i = 0; i < DPL; ++i) out[lane + 64 * i] = O[i] / L;
    if (lane == 0) atomicExch(&a.cnt[b * a.H + h], 0u);
}

}  // namespace

int attn_max_split(int n_ctx) { return (n_ctx + TILE - 1) / TILE; }

size_t attn_part_bytes(int B, int H, int n_ctx, int hd)
{
    return (size_t)B * H * attn_max_split(n_ctx) * (hd + 2) * sizeof(float);
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t st)
{
    dim3 grid(attn_max_split(a.n_ctx), a.H, a.B);
    if (a.hd == 64) hipLaunchKernelGGL(k_attn<64>, grid, dim3(64), 0, st, a);
    else if (a.hd == 128) hipLaunchKernelGGL(k_attn<128>, grid, dim3(64), 0, st, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace tsd
