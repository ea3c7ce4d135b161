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

// Two adjacent words in one 16-byte load, with the coherence of load() (sc1: served past the
// XCD's L2).  A buffer load: there is no 16-byte atomic load, and a volatile one waits for each
// load before the next is issued.  The compiler may treat it as loop-invariant, so a poll loop
// puts a compiler barrier before each round.  r spans the words; an offset past it reads zeros,
// which never carry an epoch.
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u64x2 load2(__amdgpu_buffer_rsrc_t r, uint32_t byte_off)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 16 /* sc1 */);
    u64x2 w;
    w.x = (uint64_t)v.x | ((uint64_t)v.y << 32);
    w.y = (uint64_t)v.z | ((uint64_t)v.w << 32);
    return w;
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t words_rsrc(const uint64_t* p, size_t n_words)
{
    return __builtin_amdgcn_make_buffer_rsrc((void*)p, 0, (int)(n_words * 8), 0x00020000);
}

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

// Wait until every word w[i] (already loaded from addr(i) for each i with use(i)) carries
// `epoch`: each round re-loads all words of the lane that are still stale at once, so a lane
// pays one memory round trip per round however many words it waits on.  Returns false on
// time-out.
template <int N, class Addr, class Use>
__device__ __forceinline__ bool settle_all(uint64_t (&w)[N], Addr addr, Use use, uint32_t epoch, long long limit,
                                           const uint32_t* abort_word)
{
    bool ok = true;
#pragma unroll
    for (int i = 0; i < N; ++i) ok &= !use(i) || ready(w[i], epoch);
    if (ok) return true;
    Deadline dl(limit, abort_word);
    for (;;) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (use(i) && !ready(w[i], epoch)) w[i] = load(addr(i));
        ok = true;
#pragma unroll
        for (int i = 0; i < N; ++i) ok &= !use(i) || ready(w[i], epoch);
        if (ok) return true;
        if (dl.expired()) return false;
    }
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

// the same for the words w[i] with use(i) (a uniform predicate)
template <int N, class Use, class Addr>
__device__ __forceinline__ bool settle_if(uint64_t (&w)[N], Use use, Addr addr, uint32_t epoch, long long limit,
                                          const uint32_t* abort_word)
{
    auto lane_ready = [&]() {
        bool ok = true;
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (use(i)) ok &= ready(w[i], epoch);
        return ok;
    };
    if (__builtin_amdgcn_ballot_w64(!lane_ready()) == 0) return true;
    Deadline dl(limit, abort_word);
    for (;;) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (use(i)) w[i] = load(addr(i));
        if (__builtin_amdgcn_ballot_w64(!lane_ready()) == 0) return true;
        if (dl.expired()) return false;
    }
}

// the same for one word w0 (loaded from p0) together with the words or word pairs w[i] with use(i)
// (each re-loaded as ld(i))
__device__ __forceinline__ bool ready2(uint64_t w, uint32_t epoch) { return ready(w, epoch); }
__device__ __forceinline__ bool ready2(u64x2 w, uint32_t epoch) { return (int)ready(w.x, epoch) & (int)ready(w.y, epoch); }
template <int N, class W, class Use, class Ld>
__device__ __forceinline__ bool settle_with(uint64_t& w0, const uint64_t* p0, W (&w)[N], Use use, Ld ld, uint32_t epoch,
                                            long long limit, const uint32_t* abort_word)
{
    auto lane_ready = [&]() {
        bool ok = ready(w0, epoch);
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (use(i)) ok &= ready2(w[i], epoch);
        return ok;
    };
    if (__builtin_amdgcn_ballot_w64(!lane_ready()) == 0) return true;
    Deadline dl(limit, abort_word);
    for (;;) {
        asm volatile("" ::: "memory");   // a new round of loads (see load2)
        w0 = load(p0);
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (use(i)) w[i] = ld(i);
        if (__builtin_amdgcn_ballot_w64(!lane_ready()) == 0) return true;
        if (dl.expired()) return false;
    }
}

}  // namespace xchg
}  // namespace tsd
