// sampler.h — the sampler chain's draw, as block-wide device code (internal).
//
// What it computes ("Chatterbox -> ggml Port: Development Journal", §3.2 and §3.9: temperature,
// then top-k, then top-p, then the repetition penalty; §3.19: the multilingual order, penalty,
// temperature, min-p, top-p, top-k; "Every Frame Is a Memory Read", §5.2 and §5.5: the random
// state and the penalty's history stay on the device):
//   * the penalty divides a positive logit by theta and multiplies a negative one, for every id
//     in the row's history (a bit set);
//   * top-k keeps the k largest (equal values: the lower index first); top-p keeps, in
//     descending order, every survivor whose preceding mass is below p; min-p keeps the
//     survivors whose probability is at least min_p times the largest;
//   * the draw takes z_r = exp(v_r - v_0) of the final values in descending order and returns
//     the first index whose running sum exceeds u * sum(z), where u is the top 24 bits of the
//     first word of Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
//     easy as 1, 2, 3", SC 2011) with key (seed, 0) and counter (position, row, pass, 0).
//
// How, on one workgroup: logits arrive as monotone 32-bit keys in LDS (penalized first in the
// multilingual order); a four-pass radix select (8-bit digits, most significant first, LDS
// histograms) finds the k-th largest key; the survivors are gathered as 64-bit (key, ~index)
// words, the same ordering as the greedy argmax, and bitonic-sorted in descending order; one
// scan of their weights gives the masses the top-p and min-p cuts compare against (in the
// multilingual order top-p is measured against the whole vocabulary's mass, a block sum);
// after a penalty that comes last the survivors are re-keyed and sorted again; a second scan
// finds the crossing.
#pragma once

#include <math.h>

#include "kernels.h"

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
constexpr int HIST_COPIES = 8;   // the radix histogram is kept 8 times (lane % 8 picks one):
                                 // logits cluster in a few digits, and one copy would serialise
                                 // their atomic adds
struct Scratch {
    union {
        uint32_t hist[256 * HIST_COPIES];   // digit d, copy c at d * HIST_COPIES + c (step 1 only)
        unsigned long long cand[KMAX];      // the survivors (from step 2 on)
    };
    float z[KMAX];                          // their weights
    uint32_t scan[8];                       // the scans' wave totals
    int misc[4];
};

// LDS position of key i: one word of padding after every 32, so that both the draw's per-thread
// ranges (thread t reads element t * per + j, per a multiple of 32 for the large vocabularies)
// and a writer's round-robin stores (element t + NT * q) spread over the 32 banks
__host__ __device__ constexpr int key_at(int i) { return i + (i >> 5); }
__host__ __device__ constexpr int key_words(int n) { return n + (n >> 5) + 1; }

// inclusive scans over the NT threads' values (one per thread): a shuffle scan inside each wave,
// then the wave totals through LDS; every thread gets its prefix
template <class T>
__device__ __forceinline__ T wave_incl_scan(T v)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const T u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    return v;
}

template <int NT, class T>
__device__ __forceinline__ T block_scan(T v, T* buf)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const T w = wave_incl_scan(v);
    if (lane == 63) buf[wave] = w;
    __syncthreads();
    T off = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) off += i < wave ? buf[i] : (T)0;
    __syncthreads();
    return w + off;
}

template <int NT>
__device__ __forceinline__ uint32_t block_scan_u32(uint32_t v, uint32_t* buf) { return block_scan<NT, uint32_t>(v, buf); }
template <int NT>
__device__ __forceinline__ float block_scan_f32(float v, float* buf) { return block_scan<NT, float>(v, buf); }

// the chain's parameters (kernels.h)
constexpr int ORDER_T3 = SAMP_ORDER_T3, ORDER_MTL = SAMP_ORDER_MTL;
using Chain = SampChain;

__device__ __forceinline__ float penalize(float l, float theta) { return l < 0.f ? l * theta : l / theta; }
__device__ __forceinline__ bool seen_bit(const uint32_t* seen, int i) { return (seen[i >> 5] >> (i & 31)) & 1u; }

// the history's ids as a bit set over [0, n) in LDS: entries hist[0], hist[stride], ...,
// hist[(count-1)*stride], then cur; ids outside [0, n) are ignored.  The loads of a round are
// all issued before the first is used (one memory round trip per 8 * NT entries).
template <int NT>
__device__ void build_seen(uint32_t* seen, int n, const int* hist, long long stride, int count, int cur)
{
    constexpr int R = 8;
    const int nw = (n + 31) >> 5;
    for (int i = threadIdx.x; i < nw; i += NT) seen[i] = 0u;
    __syncthreads();
    for (int base = 0; base <= count; base += NT * R) {
        int id[R];
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int p = base + j * NT + (int)threadIdx.x;
            id[j] = p < count ? hist[(long long)p * stride] : (p == count ? cur : -1);
        }
#pragma unroll
        for (int j = 0; j < R; ++j)
            if ((unsigned)id[j] < (unsigned)n) atomicOr(&seen[id[j] >> 5], 1u << (id[j] & 31));
    }
    __syncthreads();
}

// the key of logit l of id i, penalized first when the order asks for it
__device__ __forceinline__ uint32_t chain_key(float l, int i, const Chain& ch, const uint32_t* seen)
{
    if (seen && ch.order == ORDER_MTL && seen_bit(seen, i)) l = penalize(l, ch.penalty);
    return float_order_key(l);
}

// keys[key_at(i)] = chain_key(l[i], i) for i < n (l in global memory): the loads of a round
// are all issued (from clamped addresses) before the first is used
template <int NT>
__device__ void load_keys(uint32_t* keys, const float* __restrict__ l, int n, const Chain& ch, const uint32_t* seen)
{
    constexpr int R = 16;
    const int t = threadIdx.x;
    for (int base = 0; base < n; base += NT * R) {
        float v[R];
#pragma unroll
        for (int j = 0; j < R; ++j) v[j] = l[min(base + j * NT + t, n - 1)];
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int i = base + j * NT + t;
            if (i < n) keys[key_at(i)] = chain_key(v[j], i, ch, seen);
        }
    }
}

template <int NT>
__device__ __forceinline__ float block_sum_f32(float v, float* buf)
{
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) buf[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = 0.f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) r += buf[w];
    __syncthreads();
    return r;
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m)
{
    const uint32_t lo = __shfl_xor((uint32_t)v, m, 64), hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
    return ((unsigned long long)hi << 32) | lo;
}

// bitonic sort of cand[0..P) in descending order (P a power of two <= KMAX = 4 NT): thread t
// holds elements 4t..4t+3 in registers; partners inside a thread or a wave are reached by
// shuffles, only the strides that cross waves go through LDS.  Elements at P and beyond only
// ever meet each other.
template <int NT>
__device__ __forceinline__ void sort_desc(unsigned long long* cand, int P)
{
    static_assert(KMAX == 4 * NT, "four elements per thread");
    const int t = threadIdx.x;
    unsigned long long v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = 4 * t + e < P ? cand[4 * t + e] : 0ull;
    for (int size = 2; size <= P; size <<= 1)
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            unsigned long long o[4];
            if (stride >= 256) {   // partner in another wave
                __syncthreads();
#pragma unroll
                for (int e = 0; e < 4; ++e) cand[4 * t + e] = v[e];
                __syncthreads();
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = cand[(4 * t + e) ^ stride];
            } else if (stride >= 4) {
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = shfl_xor_u64(v[e], stride >> 2);
            } else if (stride == 2) {   // partners inside the thread (constant register indices)
                o[0] = v[2]; o[1] = v[3]; o[2] = v[0]; o[3] = v[1];
            } else {
                o[0] = v[1]; o[1] = v[0]; o[2] = v[3]; o[3] = v[2];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * t + e;
                const bool take_max = ((i & stride) == 0) == ((i & size) == 0);
                const bool gt = v[e] > o[e];
                v[e] = take_max == gt ? v[e] : o[e];
            }
        }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 4; ++e) cand[4 * t + e] = v[e];
    __syncthreads();
}

// The chain's draw over keys[0..n) (LDS, key i at key_at(i), chain_key of the logits); seen: the history's bit set
// in LDS, or null (no penalty).  Every thread of the (NT = 256) workgroup calls it; every thread
// gets the index.
template <int NT>
__device__ int chain_draw(const uint32_t* keys, int n, const Chain& ch, float u, Scratch& S, const uint32_t* seen)
{
    static_assert(NT == 256, "one histogram bin per thread");
    const int t = threadIdx.x;
    const int k = ch.k;
    const int per = (n + NT - 1) / NT;            // thread t owns elements [t*per, t*per + per)
    const int i0 = t * per, i1 = min(n, i0 + per);
    // the thread's keys KCH at a time, every read of a chunk issued before the first is used
    // (clamped: past the end a chunk rereads the last key, which the callers skip)
    constexpr int KCH = 8;
    auto load_chunk = [&](uint32_t* kk, int c) {
#pragma unroll
        for (int j = 0; j < KCH; ++j) kk[j] = keys[key_at(min(i0 + c + j, n - 1))];
    };

    // 1. radix select of the k-th largest key
    uint32_t prefix = 0u, mask = 0u;
    int remaining = k;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int i = t; i < 256 * HIST_COPIES; i += NT) S.hist[i] = 0u;
        __syncthreads();
        const uint32_t copy = (uint32_t)(t % HIST_COPIES);
        for (int c = 0; c < per; c += KCH) {
            uint32_t kk[KCH];
            load_chunk(kk, c);
#pragma unroll
            for (int j = 0; j < KCH; ++j)
                if (i0 + c + j < i1 && (kk[j] & mask) == prefix)
                    atomicAdd(&S.hist[((kk[j] >> shift) & 255u) * HIST_COPIES + copy], 1u);
        }
        __syncthreads();
        // running count from the highest digit down: thread t holds digit 255 - t
        uint32_t c = 0u;
#pragma unroll
        for (int r = 0; r < HIST_COPIES; ++r) c += S.hist[(255 - t) * HIST_COPIES + r];
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

    // 2. gather the survivors as (key, ~index), in index order: each thread counts its larger
    //    and its equal keys (packed: equal << 16 | larger), one scan gives its offsets
    uint32_t my = 0u;
    for (int c = 0; c < per; c += KCH) {
        uint32_t kk[KCH];
        load_chunk(kk, c);
#pragma unroll
        for (int j = 0; j < KCH; ++j)
            if (i0 + c + j < i1) my += kk[j] > T ? 1u : (kk[j] == T ? 0x10000u : 0u);
    }
    const uint32_t end = block_scan_u32<NT>(my, S.scan);
    uint32_t rg = (end - my) & 0xFFFFu, re = (end - my) >> 16;
    for (int c = 0; c < per && (my & 0xFFFFu) + (my >> 16) > 0u; c += KCH) {
        uint32_t kk[KCH];
        load_chunk(kk, c);
#pragma unroll
        for (int j = 0; j < KCH; ++j) {
            const int i = i0 + c + j;
            const unsigned long long cv = ((unsigned long long)kk[j] << 32) | (0xFFFFFFFFu - (uint32_t)i);
            if (i < i1 && kk[j] > T) S.cand[rg++] = cv;
            else if (i < i1 && kk[j] == T && re < (uint32_t)n_eq) S.cand[n_gt + re++] = cv;
        }
    }
    int P = 1;
    while (P < k) P <<= 1;
    for (int i = k + t; i < P; i += NT) S.cand[i] = 0ull;   // below every survivor
    __syncthreads();

    // 3. bitonic sort, descending
    sort_desc<NT>(S.cand, P);

    // 4. weights of the survivors (values / T, descending) and the cuts
    const float temp = ch.temperature;
    const float l0 = key_to_float((uint32_t)(S.cand[0] >> 32)) / temp;
    const int per_r = P / NT > 0 ? P / NT : 1;   // thread t owns ranks [t*per_r, t*per_r + per_r)
    const bool mtl = ch.order == ORDER_MTL;
    const bool use_p = ch.top_p > 0.f && ch.top_p < 1.f, use_min = mtl && ch.min_p > 0.f && ch.min_p < 1.f;
    int L = k;
    if (use_p || use_min) {
        float loc = 0.f;
        for (int q = 0; q < per_r; ++q) {
            const int rr = t * per_r + q;
            float zv = 0.f;
            if (rr < k) zv = expf(key_to_float((uint32_t)(S.cand[rr] >> 32)) / temp - l0);
            if (rr < P) S.z[rr] = zv;
            loc += zv;
        }
        // the mass top-p compares against: the k survivors (T3: top-k came first), or the whole
        // vocabulary's min-p survivors (MTL: top-k comes last)
        float Z;
        if (mtl) {
            float a = 0.f;
            for (int c = 0; c < per; c += KCH) {
                uint32_t kk[KCH];
                load_chunk(kk, c);
#pragma unroll
                for (int j = 0; j < KCH; ++j) {
                    const float zv = expf(key_to_float(kk[j]) / temp - l0);
                    a += (i0 + c + j < i1 && (!use_min || zv >= ch.min_p)) ? zv : 0.f;
                }
            }
            Z = block_sum_f32<NT>(a, (float*)S.scan);
        }
        const float incl = block_scan_f32<NT>(loc, (float*)S.scan);
        if (t == NT - 1) ((float*)S.misc)[3] = incl;
        __syncthreads();
        if (!mtl) Z = ((float*)S.misc)[3];
        const float cut = ch.top_p * Z;
        int kept = 0;
        float before = incl - loc;
        for (int q = 0; q < per_r; ++q) {
            const int rr = t * per_r + q;
            if (rr >= k) break;
            const float zv = S.z[rr];
            kept += (!use_p || before < cut) && (!use_min || zv >= ch.min_p);
            before += zv;
        }
        // both cuts keep a prefix of the descending order, so the count is its length
        L = (int)block_sum_f32<NT>((float)kept, (float*)S.scan);
        L = max(L, 1);
    }

    // 5. a penalty that comes last re-weights the survivors and can reorder them
    bool rekeyed = false;
    if (seen && !mtl && ch.penalty != 1.f) {
        int P2 = 1;
        while (P2 < L) P2 <<= 1;
        for (int rr = t; rr < P; rr += NT) {
            const unsigned long long c = S.cand[rr];
            unsigned long long nc = 0ull;
            if (rr < L) {
                const uint32_t lo = (uint32_t)c, idx = 0xFFFFFFFFu - lo;
                float v = key_to_float((uint32_t)(c >> 32)) / temp;
                if (seen_bit(seen, (int)idx)) v = penalize(v, ch.penalty);
                nc = ((unsigned long long)float_order_key(v) << 32) | lo;
            }
            S.cand[rr] = nc;
        }
        __syncthreads();
        sort_desc<NT>(S.cand, P2);
        rekeyed = true;
    }

    // 6. the draw over the first L: weights in descending order, their running sum, the crossing
    const float v0 = rekeyed ? key_to_float((uint32_t)(S.cand[0] >> 32)) : l0;
    float loc = 0.f;
    for (int q = 0; q < per_r; ++q) {
        const int rr = t * per_r + q;
        float zv = 0.f;
        if (rr < L) {
            const float v = key_to_float((uint32_t)(S.cand[rr] >> 32));
            zv = expf((rekeyed ? v : v / temp) - v0);
        }
        if (rr < P) S.z[rr] = zv;
        loc += zv;
    }
    const float incl = block_scan_f32<NT>(loc, (float*)S.scan);
    if (t == NT - 1) ((float*)S.misc)[3] = incl;   // the total
    if (t == 0) S.misc[0] = (int)(0xFFFFFFFFu - (uint32_t)S.cand[L - 1]);   // if nothing crosses
    __syncthreads();
    const float thr = u * ((float*)S.misc)[3];
    float run = incl - loc;
    for (int q = 0; q < per_r; ++q) {
        const int rr = t * per_r + q;
        if (rr >= L) break;
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
