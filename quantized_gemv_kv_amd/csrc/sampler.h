// sampler.h — the top-k draw of the decode step, as block-wide device code (internal).
//
// What it computes ("Chatterbox -> ggml Port: Development Journal", §3.2 and §3.9: temperature,
// then top-k, in that order; "Every Frame Is a Memory Read", §5.2: the random state stays on the
// device): keep the k largest of logits / T (equal logits: the lower index first), take
// z_r = exp(l_r / T - l_0 / T) in descending order, and return the first index whose running sum
// exceeds u * sum(z), where u is the top 24 bits of the first word of Philox4x64-10 (Salmon,
// Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011) with key
// (seed, 0) and counter (position, row, pass, 0).
//
// How, on one workgroup: logits arrive as monotone 32-bit keys in LDS; a four-pass radix select
// (8-bit digits, most significant first, LDS histograms) finds the k-th largest key; the
// survivors are gathered as 64-bit (key, ~index) words — the same ordering as the greedy
// argmax — bitonic-sorted in descending order, and an inclusive scan of their weights finds the
// crossing.
#pragma once

#include <math.h>

#include "common.h"

namespace tsd {
namespace samp {

constexpr int KMAX = 1024;   // largest k the draw supports

// Philox4x64-10: 64x64 -> 128-bit products (low half by multiply, high half by __umul64hi), ten
// rounds, the key bumped by the Weyl constants before each round after the first
__device__ __forceinline__ uint64_t philox4x64_10_word0(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3, uint64_t k0,
                                                        uint64_t k1)
{
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += W0;
            k1 += W1;
        }
        const uint64_t hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
        const uint64_t hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
        const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
    }
    return c0;
}

// u in [0, 1): exact in fp32
__device__ __forceinline__ float uniform24(uint64_t seed, uint32_t row, uint32_t pos, uint32_t pass)
{
    return (float)(philox4x64_10_word0(pos, row, pass, 0ull, seed, 0ull) >> 40) * 0x1p-24f;
}

__device__ __forceinline__ float key_to_float(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// LDS the draw needs besides the n keys
struct Scratch {
    uint32_t hist[256];
    uint32_t scan[256];
    unsigned long long cand[KMAX];
    float z[KMAX];
    int misc[4];
};

// inclusive scan over the NT threads' values (one per thread); every thread gets its prefix
template <int NT>
__device__ __forceinline__ uint32_t block_scan_u32(uint32_t v, uint32_t* buf)
{
    const int t = threadIdx.x;
    buf[t] = v;
    __syncthreads();
    for (int o = 1; o < NT; o <<= 1) {
        const uint32_t add = t >= o ? buf[t - o] : 0u;
        __syncthreads();
        buf[t] += add;
        __syncthreads();
    }
    const uint32_t r = buf[t];
    __syncthreads();
    return r;
}

template <int NT>
__device__ __forceinline__ float block_scan_f32(float v, float* buf)
{
    const int t = threadIdx.x;
    buf[t] = v;
    __syncthreads();
    for (int o = 1; o < NT; o <<= 1) {
        const float add = t >= o ? buf[t - o] : 0.f;
        __syncthreads();
        buf[t] += add;
        __syncthreads();
    }
    const float r = buf[t];
    __syncthreads();
    return r;
}

// The draw over keys[0..n) (LDS; float_order_key of the logits), 1 <= k <= min(n, KMAX).
// Every thread of the (NT = 256) workgroup calls it; every thread gets the index.
template <int NT>
__device__ int topk_draw(const uint32_t* keys, int n, int k, float temperature, float u, Scratch& S)
{
    static_assert(NT == 256, "one histogram bin per thread");
    const int t = threadIdx.x;
    const int per = (n + NT - 1) / NT;            // thread t owns elements [t*per, t*per + per)
    const int i0 = t * per, i1 = min(n, i0 + per);

    // 1. radix select of the k-th largest key
    uint32_t prefix = 0u, mask = 0u;
    int remaining = k;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        S.hist[t] = 0u;
        __syncthreads();
        for (int i = i0; i < i1; ++i) {
            const uint32_t key = keys[i];
            if ((key & mask) == prefix) atomicAdd(&S.hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        // running count from the highest digit down: thread t holds digit 255 - t
        const uint32_t c = S.hist[255 - t];
        const uint32_t cum = block_scan_u32<NT>(c, S.scan);
        if (cum >= (uint32_t)remaining && cum - c < (uint32_t)remaining) {
            S.misc[0] = 255 - t;              // the digit of the k-th largest
            S.misc[1] = (int)(cum - c);       // survivors with a larger digit
        }
        __syncthreads();
        const uint32_t d = (uint32_t)S.misc[0];
        remaining -= S.misc[1];
        prefix |= d << shift;
        mask |= 255u << shift;
        __syncthreads();
    }
    const uint32_t T = prefix;            // the k-th largest key
    const int n_eq = remaining;           // how many keys equal to T survive (the lowest indices)
    const int n_gt = k - n_eq;

    // 2. gather the survivors as (key, ~index)
    if (t == 0) S.misc[2] = 0;
    __syncthreads();
    uint32_t my_eq = 0u;
    for (int i = i0; i < i1; ++i) {
        const uint32_t key = keys[i];
        if (key > T) {
            const int p = atomicAdd(&S.misc[2], 1);
            S.cand[p] = ((unsigned long long)key << 32) | (0xFFFFFFFFu - (uint32_t)i);
        }
        my_eq += key == T;
    }
    const uint32_t eq_end = block_scan_u32<NT>(my_eq, S.scan);   // equal keys in index order
    uint32_t r = eq_end - my_eq;
    for (int i = i0; i < i1 && r < (uint32_t)n_eq; ++i)
        if (keys[i] == T) {
            S.cand[n_gt + r] = ((unsigned long long)T << 32) | (0xFFFFFFFFu - (uint32_t)i);
            ++r;
        }
    int P = 1;
    while (P < k) P <<= 1;
    for (int i = k + t; i < P; i += NT) S.cand[i] = 0ull;   // below every survivor
    __syncthreads();

    // 3. bitonic sort, descending
    for (int size = 2; size <= P; size <<= 1)
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = t; i < P / 2; i += NT) {
                const int lo = 2 * i - (i & (stride - 1)), hi = lo + stride;
                const bool desc = (lo & size) == 0;
                const unsigned long long a = S.cand[lo], b = S.cand[hi];
                if ((a < b) == desc) {
                    S.cand[lo] = b;
                    S.cand[hi] = a;
                }
            }
            __syncthreads();
        }

    // 4. weights in descending order, their running sum, the crossing
    const float l0 = key_to_float((uint32_t)(S.cand[0] >> 32)) / temperature;
    const int per_r = P / NT > 0 ? P / NT : 1;   // thread t owns ranks [t*per_r, t*per_r + per_r)
    float loc = 0.f;
    for (int q = 0; q < per_r; ++q) {
        const int rr = t * per_r + q;
        float zv = 0.f;
        if (rr < k) zv = expf(key_to_float((uint32_t)(S.cand[rr] >> 32)) / temperature - l0);
        if (rr < P) S.z[rr] = zv;
        loc += zv;
    }
    const float incl = block_scan_f32<NT>(loc, (float*)S.scan);
    if (t == NT - 1) ((float*)S.misc)[3] = incl;   // the total
    if (t == 0) S.misc[0] = (int)(0xFFFFFFFFu - (uint32_t)S.cand[k - 1]);   // if nothing crosses
    __syncthreads();
    const float thr = u * ((float*)S.misc)[3];
    float run = incl - loc;
    for (int q = 0; q < per_r; ++q) {
        const int rr = t * per_r + q;
        if (rr >= k) break;
        const float before = run;
        run += S.z[rr];
        if (run > thr && before <= thr) S.misc[0] = (int)(0xFFFFFFFFu - (uint32_t)S.cand[rr]);
    }
    __syncthreads();
    const int pick = S.misc[0];
    __syncthreads();
    return pick;
}

}  // namespace samp
}  // namespace tsd
