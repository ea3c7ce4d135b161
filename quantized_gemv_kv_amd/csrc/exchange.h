// exchange.h — device-wide data exchange inside one persistent launch (internal).
//
// A value handed from one workgroup to others travels as one 64-bit word: the fp32 bits in the
// low half, the epoch of the phase that wrote it in the high half.  The word is written with a
// single relaxed agent-scope atomic store and read with single relaxed agent-scope atomic loads,
// which on gfx950 bypass the non-coherent per-XCD L2 (the sc1 bit), so a reader on any XCD
// either sees the old word or the new one, never a torn mix, and knows which by the epoch.
// No fence and no counter is needed: the data is its own flag, and one memory round trip
// delivers both.  Epochs are never reused within the life of the buffers, so a reader can
// never mistake data of another phase, layer or step for the one it waits on.
//
// Every wait is bounded: a reader that has not seen its epoch after `limit` ticks of the
// 100 MHz constant clock gives up, raises the sticky abort word and makes its workgroup leave
// the kernel, so a fault in the exchange ends the launch instead of hanging the device.
#pragma once

#include "common.h"

namespace tsd {
namespace xchg {

__device__ __forceinline__ uint64_t load(const uint64_t* p)
{
    return __hip_atomic_load(glb(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store(uint64_t* p, float v, uint32_t epoch)
{
    __hip_atomic_store(glb(p), ((uint64_t)epoch << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_bits(uint64_t* p, uint32_t bits, uint32_t epoch)
{
    __hip_atomic_store(glb(p), ((uint64_t)epoch << 32) | bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool ready(uint64_t w, uint32_t epoch) { return (uint32_t)(w >> 32) == epoch; }
__device__ __forceinline__ float value(uint64_t w) { return __uint_as_float((uint32_t)w); }

// 32-bit words, for a hand-over whose values are used once and never accumulated: the value
// rounded to nearest even at 15 mantissa bits (relative error <= 2^-16) in the high 24 bits, and
// in the low 8 bits a tag 1 + epoch mod 255 of its epoch, never 0, so zeroed words never match.
// Every launch rewrites each slot, and the epochs of two successive writes of one slot never
// differ by a multiple of 255 (a launch spans 5 L + 1 epochs, phases of one slot 5 apart), so a
// stale word cannot carry the tag a reader waits for.  Half the bytes of the 64-bit word.
__device__ __forceinline__ uint32_t tag8(uint32_t epoch) { return 1u + epoch % 255u; }
__device__ __forceinline__ uint32_t load(const uint32_t* p)
{
    return __hip_atomic_load(glb(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store32(uint32_t* p, float v, uint32_t epoch)
{
    uint32_t u = __float_as_uint(v);
    u = (u + 0x7Fu + ((u >> 8) & 1u)) & ~0xFFu;
    __hip_atomic_store(glb(p), u | tag8(epoch), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool ready(uint32_t w, uint32_t epoch) { return (w & 0xFFu) == tag8(epoch); }
__device__ __forceinline__ float value(uint32_t w) { return __uint_as_float(w & ~0xFFu); }

// the bounded-wait bookkeeping of one poll loop
struct Deadline {
    long long t0;
    long long limit;
    const uint32_t* abort_word;
    int iter;
    __device__ __forceinline__ Deadline(long long lim, const uint32_t* ab) : t0(wall_clock64()), limit(lim), abort_word(ab), iter(0) {}
    // true once this wait has run out of time, or another workgroup has already given up
    __device__ __forceinline__ bool expired()
    {
        if ((++iter & 31) != 0) return false;
        if (wall_clock64() - t0 > limit) return true;
        return __hip_atomic_load(glb(abort_word), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
    }
};

__device__ __forceinline__ void raise_abort(uint32_t* abort_word)
{
    __hip_atomic_store(glb(abort_word), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait for N words at p[0], p[stride], ... (all with the same epoch); out[i] = their values.
// Returns false on time-out.  Loads of a lane are all in flight before the first check.
template <int N>
__device__ __forceinline__ bool wait_words(const uint64_t* p, int stride, uint32_t epoch, float (&out)[N], long long limit,
                                           const uint32_t* abort_word)
{
    uint64_t w[N];
#pragma unroll
    for (int i = 0; i < N; ++i) w[i] = load(p + (size_t)i * stride);
    bool ok = true;
#pragma unroll
    for (int i = 0; i < N; ++i) ok &= ready(w[i], epoch);
    if (!ok) {
        Deadline dl(limit, abort_word);
        for (;;) {
#pragma unroll
            for (int i = 0; i < N; ++i)
                if (!ready(w[i], epoch)) w[i] = load(p + (size_t)i * stride);
            ok = true;
#pragma unroll
            for (int i = 0; i < N; ++i) ok &= ready(w[i], epoch);
            if (ok) break;
            if (dl.expired()) break;
        }
    }
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = value(w[i]);
    return ok;
}

// Wait until words w[0..n) (already loaded from addr(i)) all carry `epoch`, n uniform.  The
// loop is uniform over the wave: while any lane still sees a stale word, every lane re-loads
// all n (one memory round trip per round, no per-word or per-lane branch).  Returns false on
// time-out.
template <int N, class W, class Addr>
__device__ __forceinline__ bool settle_n(W (&w)[N], int n, Addr addr, uint32_t epoch, long long limit,
                                         const uint32_t* abort_word)
{
    auto lane_ready = [&]() {
        bool ok = true;
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (i < n) ok &= ready(w[i], epoch);
        return ok;
    };
    if (__builtin_amdgcn_ballot_w64(!lane_ready()) == 0) return true;
    Deadline dl(limit, abort_word);
    for (;;) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (i < n) w[i] = load(addr(i));
        if (__builtin_amdgcn_ballot_w64(!lane_ready()) == 0) return true;
        if (dl.expired()) return false;
    }
}

}  // namespace xchg
}  // namespace tsd
