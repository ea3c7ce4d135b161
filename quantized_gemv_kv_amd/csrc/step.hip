// step.hip — the whole decode step (batch 1, or a pair of rows) as one persistent launch.
//
// What it computes is the step of the per-operator kernels (gemv.hip, attention.hip): for each
// layer norm -> fused QKV (+bias | +RoPE) -> K/V append -> split-KV attention -> output
// projection + residual -> norm -> FC + GELU | gate/up + SwiGLU -> down projection + residual,
// then the final norm, the head and the greedy sampler ("Chatterbox -> ggml Port: Development
// Journal", §3.2 the T3 step and §3.19 the Llama-shaped variant; "Every Frame Is a Memory Read",
// §3 and §4: the step is a chain of small matvecs whose cost is the bytes they read).
//
// Why one launch.  At batch 1 every operator moves only 0.5-5 MB, which the GPU streams in
// about a microsecond, while a kernel boundary inside a graph costs about as much again and the
// ramp of each new grid adds more; the journal measures the same effect as a step that is
// "dispatch-bound" (§3.14) and the frame post as a fixed cost per kernel (§4).  Here the grid
// is launched once, one workgroup per compute unit, and walks the step's phases in order:
//   * a phase's work is cut into tiles (rows of a matrix, or one head x 256- or 128-key chunk
//     of the cache); workgroup w takes tile w (and w + G, ... when there are more tiles);
//   * the attention output reaches the output projection through one writer per head, the item
//     of the head's last chunk, which merges the other chunks' partials;
//   * a phase's output is published as exchange words (exchange.h) carrying the phase's epoch,
//     and the next phase's workgroups poll exactly the words they need — there is no grid-wide
//     barrier, only data dependencies, each resolved by one round trip to the memory-side cache;
//   * each tile issues its weight, scale, bias and residual loads before it polls its input, so
//     they are in flight while the previous phase finishes elsewhere;
//   * a norm's scale (and a LayerNorm's mean) is applied to the finished dot products, so a
//     phase's input goes to LDS as soon as its words arrive, behind one barrier;
//   * no cache line is polled by two waves of one workgroup: polls of one line from one compute
//     unit merge, and a merged poll can return the words as they were when the first one left;
//   * the new token's key and value travel through the exchange (the attention of the same
//     launch reads them from there); the cache rows are written with plain stores and are read
//     by later launches, after the kernel boundary has made them visible on every XCD;
//   * the position, the input token and the epoch base are read at the start of the launch,
//     and workgroup 0 publishes the sampled id, the next position and the next epoch base at
//     the end, after every other workgroup has handed it its part of the argmax.
// The model's shape is a template parameter: every index, trip count and tile size is a
// compile-time constant, which keeps the per-phase instruction count (the step's critical path
// at batch 1) small.
// Epochs: launch n uses n * P + 1 .. n * P + P for its P = 5 * n_layer + 1 phases.
#include <math.h>
#include <type_traits>

#include "exchange.h"
#include "gemv_core.h"
#include "sampler.h"

namespace tsd {
namespace {

using namespace core;
constexpr int NT = 256;
constexpr int NWAVE = NT / 64;
static_assert(NWAVE <= STEP_SHIFT_COPIES, "a copy of the LayerNorm shift per wave");
constexpr int KTILE = 64;    // keys per wave in the attention phase (4 waves: one 256-key chunk), or half

enum { A_GPT2 = 0, A_LLAMA = 1 };
enum { IN_XCHG = 0, IN_NORM = 1, IN_EMB_NORM = 2, IN_XCHG32 = 3 };
enum { OUT_QKV = 0, OUT_QKV_ROPE = 1, OUT_RESID = 2, OUT_GELU = 3, OUT_SWIGLU = 4, OUT_HEAD = 5 };

constexpr int slices_for(int fmt_e, int K) { return K / fmt_e > 64 ? K / fmt_e / 64 : 1; }

// the model shape
template <int F_, int A_, int D_, int H_, int HK_, int HD_, int FF_, int V_, int B_>
struct Shape {
    static constexpr int F = F_, ARCH = A_, D = D_, H = H_, HK = HK_, HD = HD_, FF = FF_, V = V_;
    static constexpr int B = B_;   // batch rows: every weight is read once for all of them
    static constexpr bool GPT2 = A_ == A_GPT2;
    static constexpr int QD = H * HD, KD = HK * HD, QKV = QD + 2 * KD;
    static constexpr int FCN = GPT2 ? FF : 2 * FF;   // FC rows (gate/up interleaved for Llama)
    static constexpr int E = FmtT<F>::E;
    // loads per lane of each phase: two row slots (or, for rows wider than a wave, one row per
    // wave) for the K = d_model matrices, doubled for the interleaved gate/up rows and the head
    static constexpr int NL_D = fmt_nibbles(F) ? 2 : 4;
    static constexpr int NL_FC = GPT2 ? NL_D : 2 * NL_D;
    static constexpr int NL_HEAD = fmt_nibbles(F) ? 4 : 8;
    // the output projection: one row per lane for the 8-bit formats (every workgroup a tile: Llama-520M
    // 466.8 -> 452.1 us per step), two for the 4-bit ones (one or four were slower)
    static constexpr int NL_O = slices_for(E, QD) == 1 ? (fmt_nibbles(F) ? 2 : 1) : slices_for(E, QD);
    static constexpr int NL_F = slices_for(E, FF) == 1 ? 2 : slices_for(E, FF);
    static_assert(QD <= MAX_K && D <= MAX_K && FF <= MAX_K, "reduction dimension held in LDS");
    static_assert(slices_for(E, D) == 1, "d_model rows fit one wave");
};

// geometry of one GEMV phase: K-long rows, N of them, NL 16-byte loads per lane
template <int F, int K, int N, int NL>
struct Geo {
    static constexpr int E = FmtT<F>::E, SPS = FmtT<F>::SLOTS_PER_SCALE, GS = FmtT<F>::SCALE_GROUP;
    static constexpr int LPR = K / E;                       // 16-byte slots per row
    static constexpr bool WIDE = LPR > 64;                  // a row spans several loads per lane
    static constexpr int SPL = WIDE ? LPR / 64 : 1;         // loads per lane per row
    static constexpr int RG = WIDE ? 1 : 64 / LPR;          // row groups per wave
    static constexpr int NP = WIDE ? NL / SPL : NL;         // rows per lane
    static constexpr int RPW = NP * RG;                     // rows per wave
    static constexpr int RPT = NWAVE * RPW;                 // rows per tile
    static constexpr int TILES = (N + RPT - 1) / RPT;
    static constexpr int GW = WIDE ? 64 : LPR;              // lanes reduced per row
    static constexpr size_t RB = fmt_nibbles(F) ? (size_t)K / 2 : (size_t)K;   // payload bytes per row
    static constexpr int SPR = K / GS;                      // scales per row
    static_assert(K % E == 0 && (WIDE ? LPR % 64 == 0 : 64 % LPR == 0), "lanes map onto slots exactly");
    static_assert(!WIDE || NL % SPL == 0, "whole rows per wave");
};

struct Smem {
    float* xl;       // [B][MAX_K] phase input, swizzled for the weight format
    float* red;      // [4 * NWAVE]
    int* abort;      // a wait of this workgroup timed out
};

struct Ctx {
    int pos, tok[2], n_keys, S;   // tok: each batch row's input token; S attention chunks per head
    bool half_chunks;             // chunks of 128 keys (else 256)
    long long limit;
};

// ---- phase input -----------------------------------------------------------------------------
// x[0..K) of each batch row b < C::B into LDS (row b at xl + b * MAX_K) at the swizzled place of
// format F.  Thread t owns elements k = t + NT*j, j < ceil(K / NT); every load is issued
// unconditionally (an element past K, when K is not a multiple of NT, reads element K-1 and is
// discarded), and the words of all rows are polled together (one round trip for the batch).
//   IN_XCHG     exchange words src[b * xs + k] (epoch ep)
//   IN_NORM     the same, for a LayerNorm or RMSNorm with gain g: LDS gets g * (x - x0) and the
//               norm's scale and shift per row come back in rs / ms (applied after the dot products)
//   IN_EMB_NORM the embedding row of the row's input token (+ the learned position row), then the norm
//   IN_XCHG32   32-bit exchange words ((uint32_t*)(src + b * xs))[k] (the FC / SwiGLU output)
// NS sums over the workgroup with one barrier: every wave must have passed a barrier since the
// last readers of red (the gather's early barrier) before the first writer here
template <int NS>
__device__ __forceinline__ void block_sums(float (&v)[NS], float* red)
{
#pragma unroll
    for (int i = 0; i < NS; ++i) v[i] = wave_sum(v[i]);
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
        for (int i = 0; i < NS; ++i) red[NS * (threadIdx.x >> 6) + i] = v[i];
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        float r = 0.f;
#pragma unroll
        for (int w = 0; w < NWAVE; ++w) r += red[NS * w + i];
        v[i] = r;
    }
}

// X16: elements 16..31 of every 32 go to LDS divided by 16 (the high nibbles' weights are then
// taken as 16 q)
template <class C, int F, int K, int IN, bool LN, bool X16 = false>
__device__ __forceinline__ void gather_x(const StepArgs& a, const Ctx& cx, const uint64_t* src, const long long xs,
                                         const uint32_t ep, const float* g, Smem& sm, float (&rs)[C::B],
                                         float (&ms)[C::B])
{
    constexpr int B = C::B;
    constexpr int E = FmtT<F>::E, LPR = K / E, J = (K + NT - 1) / NT;
    constexpr bool NORM = IN == IN_NORM || IN == IN_EMB_NORM;
    const int t = threadIdx.x;
    auto elem = [&](int j) { return K % NT == 0 ? t + NT * j : min(t + NT * j, K - 1); };
    float v[B][J], gg[J];
    bool ok = true;
    // The early barrier: every wave passes one barrier after issuing its first round of polls and
    // before waiting on them, so that the previous phase's readers of xl and red are done before
    // anything here writes them, while the polls' round trip hides the barrier.
    bool early = false;
#pragma unroll
    for (int b = 0; b < B; ++b) {
        rs[b] = 1.f;
        ms[b] = 0.f;
    }
    if constexpr (NORM) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            gg[j] = glb(g)[elem(j)];
        }
    }
    float x0[B];   // LayerNorm shift per row (see finish_x in the GEMV core)
#pragma unroll
    for (int b = 0; b < B; ++b) x0[b] = 0.f;
    if constexpr (IN == IN_EMB_NORM) {
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const float* er = a.emb + (size_t)cx.tok[b] * K;
            const float* pr = a.wpe + (size_t)cx.pos * K;
#pragma unroll
            for (int j = 0; j < J; ++j) v[b][j] = glb(er)[elem(j)] + (C::GPT2 ? glb(pr)[elem(j)] : 0.f);
        }
        lds_barrier();   // the early barrier (see early above)
        early = true;
    } else if constexpr (IN == IN_XCHG32) {
        constexpr int NW = B * J;
        auto addr = [&](int q) -> const uint32_t* {
            const int b = q / J, j = q - b * J;
            return (const uint32_t*)(src + b * xs) + elem(j);
        };
        uint32_t w[NW];
#pragma unroll
        for (int q = 0; q < NW; ++q) w[q] = xchg::load(addr(q));
        lds_barrier();   // the early barrier (see early above)
        early = true;
        ok = xchg::settle_n(w, NW, addr, ep, cx.limit, a.abort_word);
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int j = 0; j < J; ++j) v[b][j] = xchg::value(w[b * J + j]);
    } else {
        // per row: words 0..J-1 this thread's elements, word J element 0 (the LayerNorm shift)
        constexpr int NR = J + (LN ? 1 : 0), NW = B * NR;
        auto addr = [&](int q) -> const uint64_t* {
            const int b = q / NR, qq = q - b * NR;
            // word 0 from this wave's copy at batch 1 (the pair, short of registers, was slower
            // with the copies than polling word 0 itself)
            return src + b * xs + (qq < J ? elem(qq) : B == 1 ? K + STEP_SHIFT_STRIDE * (t >> 6) : 0);
        };
        uint64_t w[NW];
#pragma unroll
        for (int q = 0; q < NW; ++q) w[q] = xchg::load(addr(q));
        lds_barrier();   // the early barrier (see early above)
        early = true;
        ok = xchg::settle_n(w, NW, addr, ep, cx.limit, a.abort_word);
#pragma unroll
        for (int b = 0; b < B; ++b) {
#pragma unroll
            for (int j = 0; j < J; ++j) v[b][j] = xchg::value(w[b * NR + j]);
            if constexpr (LN) x0[b] = xchg::value(w[b * NR + J]);
        }
    }
    if (!ok) *sm.abort = 1;
    if (!early) lds_barrier();   // the previous phase's readers of xl and red are done
    auto put = [&](int b, int j, float y) {
        const int k = t + NT * j;
        if (X16 && (k & 31) >= 16) y *= 0.0625f;   // exact
        if (K % NT == 0 || k < K) sm.xl[b * MAX_K + 4 * swz<E>(k, LPR) + (k & 3)] = y;
    };

    if constexpr (NORM) {
        constexpr float invK = 1.0f / (float)K;
        constexpr int NS = (LN ? 2 : 1) * B;   // per row: (sum, sum of squares) or the sum of squares
        float sums[NS];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            float s1 = 0.f, q2 = 0.f;
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const float dx = (K % NT == 0 || t + NT * j < K) ? v[b][j] - x0[b] : 0.f;
                s1 += dx;
                q2 = fmaf(dx, dx, q2);
            }
            if constexpr (LN) {
                sums[2 * b] = s1;
                sums[2 * b + 1] = q2;
            } else {
                sums[b] = q2;
            }
        }
        // The norm is applied after the dot products: g * (x - x0) goes to LDS at once (x0 the
        // LayerNorm shift, 0 for RMSNorm), and with the row's sums known the caller turns each
        // dot product p into rs (p - ms c) + d (LayerNorm: rs = 1 / sigma, ms = mean - x0, c = W g,
        // d = W beta + bias) or rs p (RMSNorm), so the sums' one barrier also publishes xl.
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int j = 0; j < J; ++j) put(b, j, (v[b][j] - x0[b]) * gg[j]);
        block_sums<NS>(sums, sm.red);
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if constexpr (LN) {
                const float m1 = sums[2 * b] * invK;
                rs[b] = 1.0f / sqrtf(fmaxf(sums[2 * b + 1] * invK - m1 * m1, 0.f) + a.eps);
                ms[b] = m1;
            } else {
                rs[b] = 1.0f / sqrtf(sums[b] * invK + a.eps);
            }
        }
        return;
    } else {
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int j = 0; j < J; ++j) put(b, j, v[b][j]);
    }
    lds_barrier();
}

// ---- one GEMV phase --------------------------------------------------------------------------
struct PhaseIO {
    const uint64_t* src;  // input words (IN_XCHG / IN_NORM); row b at src + b * src_xs
    long long src_xs;
    uint32_t src_ep;
    const float* g;       // norm gain
    const float* lc;      // LayerNorm-fed: W g and W beta + bias per output row (normalised after
    const float* ld;      // the dot products, see gather_x)
    const float* bias;    // linear bias or null
    uint64_t* dst;        // output words; row b at dst + b * dst_xs
    long long dst_xs;
    uint32_t dst_ep;
    const uint64_t* res;  // OUT_RESID: residual words, or null for the embedding row (first layer)
    long long res_xs;
    uint32_t res_ep;
    __half* kc;           // OUT_QKV*: this layer's cache (row b at kc + b * a.kv_row)
    __half* vc;
};

// 16-byte load through the global address space
__device__ __forceinline__ uint4 ld16(const void* p)
{
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    const v4u v = *(const TSD_GLOBAL v4u*)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}

// (cos, sin) pair load through the global address space
__device__ __forceinline__ float2 ld8f(const float2* p)
{
    typedef float v2f __attribute__((ext_vector_type(2)));
    const v2f v = *(const TSD_GLOBAL v2f*)p;
    return make_float2(v.x, v.y);
}

// fp16 store through the global address space
__device__ __forceinline__ void st_half(__half* p, __half v) { *glb((unsigned short*)p) = __half_as_ushort(v); }

// The partial sums of NU units of NV rows each (unit u = rows u NV .. u NV + NV - 1) reduced over
// aligned groups of GW lanes: lane s of a group ends with the NV totals of unit s % NU.  Each
// selecting stage halves the units a lane carries: the lane keeps the half that one bit of its
// slot names and adds that half as a partner lane (the bit flipped, the bits of earlier stages
// kept) held it, having sent the other half.  The stages after them add lanes that carry the same
// unit (rotations by 4 and 8 within a row of 16, then the 16- and 32-lane swaps).
template <int NU, int NV, int GW>
__device__ __forceinline__ void fold_units(const float (&p)[NU * NV], float (&t)[NV], int slot)
{
    static_assert(NU == 2 || NU == 4 || NU == 8, "two to eight units");
    static_assert(GW == 16 || GW == 32 || GW == 64, "groups of 16 to 64 lanes");
    float c[NU * NV];
#pragma unroll
    for (int i = 0; i < NU * NV; ++i) c[i] = p[i];
    auto stage = [&](auto ctrl, int half, bool k) {
#pragma unroll
        for (int i = 0; i < half * NV; ++i) {
            const float keep = k ? c[i + half * NV] : c[i], send = k ? c[i] : c[i + half * NV];
            c[i] = keep + dpp_mov<decltype(ctrl)::value>(send);
        }
    };
    if constexpr (NU >= 8) stage(std::integral_constant<int, 0x141>{}, 4, slot & 4);   // partner s ^ 7
    if constexpr (NU >= 4) stage(std::integral_constant<int, 0x4E>{}, 2, slot & 2);    // partner s ^ 2
    stage(std::integral_constant<int, 0xB1>{}, 1, slot & 1);                            // partner s ^ 1
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        float x = c[v];
        if constexpr (NU <= 2) x += dpp_mov<0x4E>(x);
        if constexpr (NU <= 4) x += dpp_mov<0x124>(x);   // row_ror:4
        x += dpp_mov<0x128>(x);                          // row_ror:8
        if constexpr (GW >= 32) x = swap16_sum(x);
        if constexpr (GW >= 64) x = swap32_sum(x);
        t[v] = x;
    }
}

typedef _Float16 h2t __attribute__((ext_vector_type(2)));

// v[i] for a runtime i < N: a tree of selects on the bits of i (the opaque intermediates keep
// the compiler from rebuilding it as an indexed load through scratch memory)
template <int N>
__device__ __forceinline__ float pick(const float (&v)[N], int i)
{
    static_assert((N & (N - 1)) == 0, "power of two");
    if constexpr (N == 1) {
        return v[0];
    } else {
        float lo[N / 2], hi[N / 2];
#pragma unroll
        for (int k = 0; k < N / 2; ++k) {
            lo[k] = v[k];
            hi[k] = v[k + N / 2];
        }
        float a = pick(lo, i & (N / 2 - 1)), b = pick(hi, i & (N / 2 - 1));
        asm volatile("" : "+v"(a), "+v"(b));
        return (i & (N / 2)) ? b : a;
    }
}

template <class C, int K, int N, int NL, int IN, int OUT, bool LN>
__device__ __forceinline__ bool gemv_phase(const StepArgs& a, const Ctx& cx, const PackedMat& W, const PhaseIO& io,
                                           Smem& sm)
{
    constexpr int F = C::F, HD = C::HD, B = C::B;
    using G = Geo<F, K, N, NL>;
    constexpr int E = G::E, NP = G::NP;
    constexpr bool PAIR = OUT == OUT_QKV_ROPE || OUT == OUT_SWIGLU;
    constexpr bool NORM = IN == IN_NORM || IN == IN_EMB_NORM;
    constexpr bool LNP = NORM && LN;   // LayerNorm applied after the dot products (the bias is in io.ld)
    constexpr bool PREH = F == FMT_Q4_0 && NL <= 2 && B == 2;   // weights as fp16 pairs (below)
    constexpr bool PRE8 = F == FMT_Q8_0 && B == 2;               // the same for Q8_0
    constexpr bool HAS_BIAS = C::GPT2 && !PAIR && OUT != OUT_HEAD && !LNP;
    constexpr int QD = C::QD, KD = C::KD;
    static_assert(!PAIR || NP % 2 == 0, "pair epilogues need an even number of rows per lane");

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int slot0 = G::WIDE ? lane : lane % G::LPR;   // this lane's slot (first slice)
    const int sub = G::WIDE ? 0 : lane / G::LPR;         // its row group within the wave
    // lane-parallel epilogue: lane `slot0` (< NOUT) of a row group finishes the group's output
    // slot0 (a row, or a pair of rows)
    constexpr int NOUT = PAIR ? NP / 2 : NP;
    const int er = slot0 < NOUT ? slot0 : NOUT - 1;
    const bool eon = slot0 < NOUT;
    // head: two rows guided by classifier-free guidance make one set of combined logits
    const bool guided = B == 2 && OUT == OUT_HEAD && a.cfg;

    unsigned long long best[B];
#pragma unroll
    for (int b = 0; b < B; ++b) best[b] = 0ull;
    bool have_x = false;
    float rs[B], ms[B];   // per row: the norm applied after the dot products (see gather_x)
    for (int tile = blockIdx.x; tile < G::TILES; tile += gridDim.x) {
        const int row0 = (tile * NWAVE + wave) * G::RPW + sub * NP;   // first row of this lane's group
        // epilogue operands of the lane's own output row(s), issued before the weights
        const int erow = row0 + (PAIR ? 2 * er : er);
        const int erc = min(erow, N - 1);
        float bv = 0.f, re[B];
        uint64_t rw[B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            re[b] = 0.f;
            rw[b] = 0ull;
        }
        if constexpr (HAS_BIAS) bv = glb(io.bias)[erc];
        float lcv = 0.f, ldv = 0.f;
        if constexpr (LNP) {
            lcv = glb(io.lc)[erc];
            ldv = glb(io.ld)[erc];
        }
        if constexpr (OUT == OUT_RESID) {
#pragma unroll
            for (int b = 0; b < B; ++b) {
                if (io.res) rw[b] = xchg::load(io.res + b * io.res_xs + erc);
                else re[b] = glb(a.emb)[(size_t)cx.tok[b] * N + erc] + (C::GPT2 ? glb(a.wpe)[(size_t)cx.pos * N + erc] : 0.f);
            }
        }
        // every weight and raw scale of this lane (unconditional, clamped rows)
        uint4 w[NL];
        uint32_t sc_raw[NL], sb_raw[NL], h_raw[NL];
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int row = min(G::WIDE ? row0 + i / G::SPL : row0 + i, N - 1);
            const int slot = G::WIDE ? (i % G::SPL) * 64 + lane : slot0;
            w[i] = ld16(W.q + (size_t)row * G::RB + (size_t)slot * 16);
            sc_raw[i] = *glb((const uint16_t*)W.s + (size_t)row * G::SPR + slot / G::SPS);
            sb_raw[i] = 0u;
            h_raw[i] = 0u;
            if constexpr (fmt_affine(F)) sb_raw[i] = *glb((const uint16_t*)W.b + (size_t)row * G::SPR + slot / G::SPS);
            if constexpr (F == FMT_Q5_0) h_raw[i] = *glb(W.h + (size_t)row * (K / 32) + slot);
        }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);

        // the pair in Q4_0 with at most two slots a lane: the weights as fp16 pairs, q - 8 for the
        // low nibbles and 16 (q - 8) for the high ones (against x / 16), each pair two elements two
        // apart, multiplied with one mixed fp16 x fp32 FMA per weight, the -8 offset needing no sum
        // of x (fewer live registers than the per-row decode; at batch 1 it measured slower)
        h2t wh[PREH || PRE8 ? NL : 1][PRE8 ? 8 : 16];
        auto pre = [&]() {
            if constexpr (PRE8) {
                // bytes q -> fp16 q - 128 in pairs (byte permutes build 1024 + q, a packed
                // subtract of 1152 centres them exactly)
#pragma unroll
                for (int i = 0; i < NL; ++i) {
                    const uint32_t ws[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        wh[i][2 * q + 0] = __builtin_bit_cast(h2t, __builtin_amdgcn_perm(0x64646464u, ws[q], 0x04010400u)) - h2t{1152.f, 1152.f};
                        wh[i][2 * q + 1] = __builtin_bit_cast(h2t, __builtin_amdgcn_perm(0x64646464u, ws[q], 0x04030402u)) - h2t{1152.f, 1152.f};
                    }
                }
            }
            if constexpr (PREH) {
#pragma unroll
                for (int i = 0; i < NL; ++i) {
                    const uint32_t ws[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t w8 = ws[q] >> 8;
                        wh[i][4 * q + 0] = __builtin_bit_cast(h2t, (ws[q] & 0x000F000Fu) | 0x64006400u) - h2t{1032.f, 1032.f};
                        wh[i][4 * q + 1] = __builtin_bit_cast(h2t, (ws[q] & 0x00F000F0u) | 0x64006400u) - h2t{1152.f, 1152.f};
                        wh[i][4 * q + 2] = __builtin_bit_cast(h2t, (w8 & 0x000F000Fu) | 0x64006400u) - h2t{1032.f, 1032.f};
                        wh[i][4 * q + 3] = __builtin_bit_cast(h2t, (w8 & 0x00F000F0u) | 0x64006400u) - h2t{1152.f, 1152.f};
                    }
                }
            }
        };
        if (!have_x) {
            gather_x<C, F, K, IN, LN, PREH>(a, cx, io.src, io.src_xs, io.src_ep, io.g, sm, rs, ms);
            have_x = true;
            if (*sm.abort) return false;
        }
        pre();

        // per row: this lane's x slices and their sums, then the dot products with the weights
        float part[B][NP];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            float xs[G::SPL][E];
            float sx[G::SPL];
            const float4* xl4 = (const float4*)(sm.xl + b * MAX_K);
#pragma unroll
            for (int j = 0; j < G::SPL; ++j) {
                const int slot = G::WIDE ? j * 64 + lane : slot0;
                float s = 0.f;
#pragma unroll
                for (int e4 = 0; e4 < E / 4; ++e4) {
                    const float4 v = xl4[e4 * G::LPR + slot];
                    xs[j][4 * e4 + 0] = v.x;
                    xs[j][4 * e4 + 1] = v.y;
                    xs[j][4 * e4 + 2] = v.z;
                    xs[j][4 * e4 + 3] = v.w;
                    s += (v.x + v.y) + (v.z + v.w);
                }
                sx[j] = s;
            }
#pragma unroll
            for (int r = 0; r < NP; ++r) part[b][r] = 0.f;
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                const int j = G::WIDE ? i % G::SPL : 0;
                const int r = G::WIDE ? i / G::SPL : i;
                const float sc = __half2float(__ushort_as_half((unsigned short)sc_raw[i]));
                if constexpr (PRE8) {
                    // word q: pairs (4q, 4q+1), (4q+2, 4q+3)
                    float a0 = 0.f, a1 = 0.f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        a0 = fmaf((float)wh[i][2 * q].x, xs[j][4 * q], a0);
                        a1 = fmaf((float)wh[i][2 * q + 1].x, xs[j][4 * q + 2], a1);
                        a0 = fmaf((float)wh[i][2 * q].y, xs[j][4 * q + 1], a0);
                        a1 = fmaf((float)wh[i][2 * q + 1].y, xs[j][4 * q + 3], a1);
                    }
                    part[b][r] = fmaf(sc, a0 + a1, part[b][r]);
                } else if constexpr (PREH) {
                    // word q: pairs (4q, 4q+2), (16+4q, 16+4q+2), (4q+1, 4q+3), (16+4q+1, 16+4q+3)
                    float a0 = 0.f, a1 = 0.f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        a0 = fmaf((float)wh[i][4 * q + 0].x, xs[j][4 * q], a0);
                        a1 = fmaf((float)wh[i][4 * q + 1].x, xs[j][16 + 4 * q], a1);
                        a0 = fmaf((float)wh[i][4 * q + 0].y, xs[j][4 * q + 2], a0);
                        a1 = fmaf((float)wh[i][4 * q + 1].y, xs[j][16 + 4 * q + 2], a1);
                        a0 = fmaf((float)wh[i][4 * q + 2].x, xs[j][4 * q + 1], a0);
                        a1 = fmaf((float)wh[i][4 * q + 3].x, xs[j][16 + 4 * q + 1], a1);
                        a0 = fmaf((float)wh[i][4 * q + 2].y, xs[j][4 * q + 3], a0);
                        a1 = fmaf((float)wh[i][4 * q + 3].y, xs[j][16 + 4 * q + 3], a1);
                    }
                    part[b][r] = fmaf(sc, a0 + a1, part[b][r]);
                } else {
                    const float d = slot_dot<F>(w[i], xs[j], h_raw[i]);
                    part[b][r] += slot_value<F>(d, sx[j], sc, __half2float(__ushort_as_half((unsigned short)sb_raw[i])));
                }
            }
        }
        // the lane's output row(s): fin[b][v] = row er * NV + v of the group
        constexpr int NV = PAIR ? 2 : 1;
        float fin[B][NV];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if constexpr (G::GW >= 16 && NOUT >= 2 && NOUT <= 8) {
                fold_units<NOUT, NV, G::GW>(part[b], fin[b], slot0);
            } else {
                float pv[NV][NOUT];
#pragma unroll
                for (int u = 0; u < NOUT; ++u)
#pragma unroll
                    for (int v = 0; v < NV; ++v) pv[v][u] = group_sum(part[b][u * NV + v], G::GW);
#pragma unroll
                for (int v = 0; v < NV; ++v) fin[b][v] = pick(pv[v], er);
            }
            if constexpr (LNP) {
#pragma unroll
                for (int v = 0; v < NV; ++v) fin[b][v] = fmaf(rs[b], fmaf(-ms[b], lcv, fin[b][v]), ldv);
            } else if constexpr (NORM) {
#pragma unroll
                for (int v = 0; v < NV; ++v) fin[b][v] *= rs[b];
            }
        }

        if constexpr (OUT == OUT_RESID) {
            if (io.res) {
                auto addr = [&](int q) { return io.res + q * io.res_xs + erc; };
                if (!xchg::settle_n(rw, B, addr, io.res_ep, cx.limit, a.abort_word)) *sm.abort = 1;
#pragma unroll
                for (int b = 0; b < B; ++b) re[b] = xchg::value(rw[b]);
            }
        }

        if constexpr (OUT == OUT_HEAD) {
            float tb[B];
#pragma unroll
            for (int b = 0; b < B; ++b) tb[b] = fin[b][0];
            if (eon && erow < N) {
#pragma unroll
                for (int b = 0; b < B; ++b) glb(a.logits)[(size_t)b * N + erow] = tb[b];
                if (guided) {
                    const float t = fmaf(a.cfg_weight, tb[0] - tb[B - 1], tb[0]);   // l0 + w (l0 - l1)
                    if (a.samp_mode) xchg::store(a.x_logit + erow, t, io.dst_ep);
                    const unsigned long long key =
                        ((unsigned long long)float_order_key(t) << 32) | (0xFFFFFFFFu - (uint32_t)erow);
                    best[0] = key > best[0] ? key : best[0];
                } else {
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        if (a.samp_mode) xchg::store(a.x_logit + b * a.xs_logit + erow, tb[b], io.dst_ep);
                        const unsigned long long key =
                            ((unsigned long long)float_order_key(tb[b]) << 32) | (0xFFFFFFFFu - (uint32_t)erow);
                        best[b] = key > best[b] ? key : best[b];
                    }
                }
            }
        } else if constexpr (PAIR) {
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const float t0 = fin[b][0], t1 = fin[b][NV - 1];
                uint64_t* dst = io.dst + b * io.dst_xs;
                if (eon && erow < N) {
                    if constexpr (OUT == OUT_SWIGLU) {
                        xchg::store32((uint32_t*)dst + (erow >> 1), silu(t0) * t1, io.dst_ep);
                    } else {
                        // rows (2m, 2m+1) = elements (i, i + hd/2) of a Q or K head, or (2m, 2m+1) of V
                        constexpr int half = HD / 2;
                        if (erow < QD + KD) {
                            const bool isk = erow >= QD;
                            const int m = (isk ? erow - QD : erow) >> 1;
                            const int h = m / half, i = m - h * half;
                            const float2 cs = ld8f(a.rope + (size_t)cx.pos * half + i);
                            const float ra = t0 * cs.x - t1 * cs.y, rb = t0 * cs.y + t1 * cs.x;
                            if (!isk) {
                                xchg::store(dst + h * HD + i, ra, io.dst_ep);
                                xchg::store(dst + h * HD + i + half, rb, io.dst_ep);
                            } else {
                                const __half ha = __float2half_rn(ra), hb = __float2half_rn(rb);
                                __half* c = io.kc + b * a.kv_row + ((size_t)h * a.n_ctx + cx.pos) * HD;
                                st_half(c + i, ha);
                                st_half(c + i + half, hb);
                                xchg::store(dst + QD + h * HD + i, __half2float(ha), io.dst_ep);
                                xchg::store(dst + QD + h * HD + i + half, __half2float(hb), io.dst_ep);
                            }
                        } else {
                            const int rv = erow - QD - KD;
                            const int h = rv / HD, i = rv - h * HD;
                            const __half ha = __float2half_rn(t0), hb = __float2half_rn(t1);
                            __half* c = io.vc + b * a.kv_row + ((size_t)h * a.n_ctx + cx.pos) * HD;
                            st_half(c + i, ha);
                            st_half(c + i + 1, hb);
                            xchg::store(dst + erow, __half2float(ha), io.dst_ep);
                            xchg::store(dst + erow + 1, __half2float(hb), io.dst_ep);
                        }
                    }
                }
            }
        } else {
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const float t = fin[b][0] + bv;
                uint64_t* dst = io.dst + b * io.dst_xs;
                if (eon && erow < N) {
                    if constexpr (OUT == OUT_QKV) {
                        if (erow < QD) {
                            xchg::store(dst + erow, t, io.dst_ep);
                        } else {
                            const bool isk = erow < QD + KD;
                            const int rv = isk ? erow - QD : erow - QD - KD;
                            const int h = rv / HD, i = rv - h * HD;
                            const __half hv = __float2half_rn(t);
                            st_half((isk ? io.kc : io.vc) + b * a.kv_row + ((size_t)h * a.n_ctx + cx.pos) * HD + i, hv);
                            xchg::store(dst + erow, __half2float(hv), io.dst_ep);
                        }
                    } else if constexpr (OUT == OUT_RESID) {
                        xchg::store(dst + erow, t + re[b], io.dst_ep);
                        if constexpr (C::GPT2 && B == 1) {
                            if (erow == 0) {   // the LayerNorm shift's copies (one per consuming wave)
#pragma unroll
                                for (int w = 0; w < STEP_SHIFT_COPIES; ++w)
                                    xchg::store(dst + N + STEP_SHIFT_STRIDE * w, t + re[b], io.dst_ep);
                            }
                        }
                    } else if constexpr (OUT == OUT_GELU) {
                        xchg::store32((uint32_t*)dst + erow, gelu_tanh(t), io.dst_ep);
                    }
                }
            }
        }
    }

    if constexpr (OUT == OUT_HEAD) {
        // this workgroup's best (ordered logit, ~index) key of each row (guided: of the combined
        // logits, row 0 only), published as two words
        if ((int)blockIdx.x < G::TILES) {
            __shared__ unsigned long long bkey[B][NWAVE];
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const unsigned long long m = wave_max_u64(best[b]);
                if (lane == 0) bkey[b][wave] = m;
            }
            lds_barrier();
            if (threadIdx.x == 0) {
                const int nrows = guided ? 1 : B;
                for (int b = 0; b < nrows; ++b) {
                    unsigned long long m = bkey[b][0];
#pragma unroll
                    for (int i = 1; i < NWAVE; ++i) m = bkey[b][i] > m ? bkey[b][i] : m;
                    xchg::store_bits(io.dst + b * io.dst_xs + 2 * blockIdx.x, (uint32_t)(m >> 32), io.dst_ep);
                    xchg::store_bits(io.dst + b * io.dst_xs + 2 * blockIdx.x + 1, (uint32_t)m, io.dst_ep);
                }
            }
        }
    }
    return true;
}

// ---- attention phase -------------------------------------------------------------------------
// Work item (row b, head h, chunk s) = keys [C s, C s + C) of query head h, C = NWAVE * KT (256
// or 128 keys: KT per wave); the same math as
// k_attn (attention.hip), with the query and the new position's key/value taken from the
// exchange.  Items go to the highest-numbered workgroups, which the QKV phase leaves idle when
// it has fewer tiles than the grid has workgroups.  One writer per head: the item of the head's
// last chunk merges the other chunks' (o, m, l) partials into its own and publishes the head's
// output o / l as plain exchange words (x_ao), so the output projection polls hd words per head
// like any other input instead of every chunk's partial.
template <class C, int KT>
__device__ __forceinline__ bool attn_phase(const StepArgs& a, const Ctx& cx, const __half* kcache, const __half* vcache,
                                           const uint32_t ep_qkv, const uint32_t ep_part, Smem& sm)
{
    constexpr int HD = C::HD, H = C::H, HK = C::HK, QD = C::QD, KD = C::KD;
    constexpr int LPK = HD / 8, KPI = 64 / LPK, R = KT / KPI, PS = HD + STEP_PART_PAD;
    __shared__ float ow[NWAVE][HD];
    __shared__ float mw[NWAVE], lw[NWAVE];
    __shared__ float qkv_l[3 * HD];   // the query, new key and new value of the item
    const int items = C::B * H * cx.S;
    const int last = cx.S - 1;                 // a head's last chunk
    const int n_first = C::B * H * last;       // the other chunks' items come first
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane % LPK, kq = lane / LPK;
    const int n_keys = cx.n_keys;
    const float qscale = 1.4426950408889634f / sqrtf((float)HD);

    for (int item = (int)gridDim.x - 1 - (int)blockIdx.x; item < items; item += gridDim.x) {
        // Items 0 .. n_first - 1 are the chunks before the last, then one item per (row, head) for
        // its last chunk, which waits for the others' partials.  A workgroup takes its items in
        // increasing order, so every item queued ahead of an awaited one never waits itself: the
        // waits always end.
        int h, s, b;
        if (item < n_first) {
            h = item % H;
            s = (item / H) % last;
            b = item / H / last;
        } else {
            h = (item - n_first) % H;
            b = (item - n_first) / H;
            s = last;
        }
        const int g = h / (H / HK);
        const int k0 = (s * NWAVE + wave) * KT;
        const size_t head_off = (size_t)b * a.kv_row + (size_t)g * a.n_ctx * HD;
        const int klast = n_keys - 1;
        uint4 kr[R], vr[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int key = min(k0 + r * KPI + kq, klast);
            kr[r] = ld16(kcache + head_off + (size_t)key * HD + c * 8);
            vr[r] = ld16(vcache + head_off + (size_t)key * HD + c * 8);
        }
        // The query of head h and the new key / value of kv head g (3 HD words) are polled by wave 0
        // alone, each lane its own words, and handed to the other waves through LDS: when every
        // wave polled the same words, the waves of one workgroup saw them up to a microsecond
        // apart (polls of one line from one compute unit merge, and a merged poll can return the
        // stale word).
        constexpr int NQ = 3 * HD / 64;   // words per lane of wave 0
        if (wave == 0) {
            const uint64_t* xq = a.x_qkv + b * a.xs_qkv;
            auto addr = [&](int i) {
                const int w = lane + 64 * i;
                return w < HD ? xq + h * HD + w : w < 2 * HD ? xq + QD + g * HD + (w - HD) : xq + QD + KD + g * HD + (w - 2 * HD);
            };
            uint64_t wx[NQ];
#pragma unroll
            for (int i = 0; i < NQ; ++i) wx[i] = xchg::load(addr(i));
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            if (!xchg::settle_n(wx, NQ, addr, ep_qkv, cx.limit, a.abort_word)) *sm.abort = 1;
#pragma unroll
            for (int i = 0; i < NQ; ++i) qkv_l[lane + 64 * i] = xchg::value(wx[i]);
        }
        lds_barrier();
        // the new position's row (exact fp16 values) replaces whatever the cache held there
        uint4 nk, nv;
        {
            __half2 hk[4], hv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                hk[e] = __floats2half2_rn(qkv_l[HD + c * 8 + 2 * e], qkv_l[HD + c * 8 + 2 * e + 1]);
                hv[e] = __floats2half2_rn(qkv_l[2 * HD + c * 8 + 2 * e], qkv_l[2 * HD + c * 8 + 2 * e + 1]);
            }
            nk = *(const uint4*)hk;
            nv = *(const uint4*)hv;
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (k0 + r * KPI + kq == cx.pos) {
                kr[r] = nk;
                vr[r] = nv;
            }
        float q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = qkv_l[c * 8 + e] * qscale;

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
            const uint4 vv = valid ? vr[r] : make_uint4(0u, 0u, 0u, 0u);
            const __half2* vh = (const __half2*)&vv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float2 f = __half22float2(vh[e]);
                o[2 * e] = fmaf(p, f.x, o[2 * e]);
                o[2 * e + 1] = fmaf(p, f.y, o[2 * e + 1]);
            }
        }
        const float l = wave_sum(lsum) * (1.0f / LPK);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = o[e];
            if constexpr (LPK == 8) v += dpp_mov<0x128>(v);
            v = swap16_sum(v);
            v = swap32_sum(v);
            o[e] = v;
        }
        lds_barrier();   // the previous item's readers of ow are done
        if (kq == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) ow[wave][c * 8 + e] = o[e];
        }
        if (lane == 0) {
            mw[wave] = k0 < n_keys ? m : -INFINITY;
            lw[wave] = l;
        }
        lds_barrier();
        if (*sm.abort) return false;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NWAVE; ++w) M = fmaxf(M, mw[w]);
        uint64_t* part = a.x_part + b * a.xs_part + ((size_t)h * a.max_split + s) * PS;
        const int tc = min((int)threadIdx.x, HD - 1);
        float acc = 0.f, L = 0.f;
#pragma unroll
        for (int w = 0; w < NWAVE; ++w) {
            const float f = exp2f(mw[w] - M);
            acc = fmaf(ow[w][tc], f, acc);
            L = fmaf(lw[w], f, L);
        }
        if (s != last) {   // a partial for the head's last chunk to merge
            if (threadIdx.x < HD) {
                xchg::store(part + threadIdx.x, acc, ep_part);
            } else if (threadIdx.x == HD) {
                xchg::store(part + HD, M, ep_part);
                xchg::store(part + HD + 1, L, ep_part);
            }
        } else {
            // the other chunks' partials, one per wave and round, through LDS
            for (int s0 = 0; s0 < last; s0 += NWAVE) {
                lds_barrier();   // every reader of ow, mw and lw is done
                const int sib = s0 + wave;
                if (sib < last) {
                    const uint64_t* ps = a.x_part + b * a.xs_part + ((size_t)h * a.max_split + sib) * PS;
                    constexpr int NO = HD / 64;   // output words per lane, then this lane's (m or l) word
                    auto addr = [&](int i) { return i < NO ? ps + lane + 64 * i : ps + HD + min(lane, 1); };
                    uint64_t wv[NO + 1];
#pragma unroll
                    for (int i = 0; i <= NO; ++i) wv[i] = xchg::load(addr(i));
                    if (!xchg::settle_n(wv, NO + 1, addr, ep_part, cx.limit, a.abort_word)) *sm.abort = 1;
#pragma unroll
                    for (int i = 0; i < NO; ++i) ow[wave][lane + 64 * i] = xchg::value(wv[i]);
                    if (lane == 0) mw[wave] = xchg::value(wv[NO]);
                    if (lane == 1) lw[wave] = xchg::value(wv[NO]);
                }
                lds_barrier();
                if (*sm.abort) return false;
                const int nw = min(NWAVE, last - s0);
                float Mn = M;
#pragma unroll
                for (int w = 0; w < NWAVE; ++w)
                    if (w < nw) Mn = fmaxf(Mn, mw[w]);
                const float sc = exp2f(M - Mn);
                acc *= sc;
                L *= sc;
#pragma unroll
                for (int w = 0; w < NWAVE; ++w)
                    if (w < nw) {
                        const float f = exp2f(mw[w] - Mn);
                        acc = fmaf(ow[w][tc], f, acc);
                        L = fmaf(lw[w], f, L);
                    }
                M = Mn;
            }
            if (threadIdx.x < HD)
                xchg::store(a.x_ao + b * a.xs_ao + h * HD + threadIdx.x, acc / L, ep_part);
        }
    }
    return true;
}

// ---- the step --------------------------------------------------------------------------------
template <class T>
__device__ __forceinline__ T* shift(T* p, long long bytes)
{
    return p ? (T*)((const char*)p + bytes) : nullptr;
}

__device__ __forceinline__ PackedMat shift(PackedMat m, long long bytes)
{
    m.q = shift(m.q, bytes);
    m.s = shift(m.s, bytes);
    m.b = shift(m.b, bytes);
    m.h = shift(m.h, bytes);
    return m;
}

// a workgroup that gave up tells every other one at once (their waits check the abort word)
__device__ __forceinline__ void give_up(const StepArgs& a)
{
    if (threadIdx.x == 0) xchg::raise_abort(a.abort_word);
}

// The arguments live in device memory and every phase re-reads the ones it uses through an
// opaque copy of their address (in the constant address space, so the fields are fetched with
// scalar loads, which hit the scalar cache): no phase keeps another phase's pointers alive,
// which held across the whole step would not fit the scalar registers.
using ArgsPtr = const __attribute__((address_space(4))) StepArgs*;
__device__ __forceinline__ const StepArgs& opaque(ArgsPtr p)
{
    asm volatile("" : "+s"(p));
    return *(const StepArgs*)p;
}

template <class C>
__global__ __launch_bounds__(NT) void k_step(const StepArgs* __restrict__ args)
{
    constexpr int OUT_QKV_K = C::GPT2 ? OUT_QKV : OUT_QKV_ROPE;
    constexpr int OUT_FC_K = C::GPT2 ? OUT_GELU : OUT_SWIGLU;
    constexpr int B = C::B;
    const ArgsPtr ap = (ArgsPtr)args;

    // the phase input buffer (one MAX_K slice per batch row); after the head, the drawing
    // workgroup reuses it for the chain's draw (keys, the history's bit set, the draw's scratch)
    constexpr size_t KEYS_BYTES = ((size_t)samp::key_words(C::V) * 4 + 15) & ~(size_t)15;
    constexpr size_t SEEN_BYTES = ((size_t)(C::V + 31) / 32 * 4 + 15) & ~(size_t)15;
    constexpr size_t SAMP_BYTES = KEYS_BYTES + SEEN_BYTES + sizeof(samp::Scratch);
    constexpr size_t RAW_BYTES = (size_t)B * MAX_K * 4 > SAMP_BYTES ? (size_t)B * MAX_K * 4 : SAMP_BYTES;
    static_assert(RAW_BYTES <= 56 * 1024, "LDS of one workgroup");
    __shared__ __align__(16) unsigned char raw[RAW_BYTES];
    __shared__ float red[4 * NWAVE];
    __shared__ int s_abort;
    Smem sm{(float*)raw, red, &s_abort};

    if (threadIdx.x == 0) s_abort = 0;
    Ctx cx;
    uint32_t ctr, ep0;
    int n_layer;
    {
        const StepArgs& a = opaque(ap);
        // a wait of an earlier launch timed out (the exchange state is not trusted), or an input id
        // was rejected (the state must stay as it was): do nothing
        if (ld_uniform((const int*)a.abort_word) | ld_uniform((const int*)a.bad_input)) return;
        cx.pos = ld_uniform(a.pos);
#pragma unroll
        for (int b = 0; b < B; ++b) {
            // ids enter through the checked input copy; the clamp only keeps every gather in bounds
            const int tok = ld_uniform(a.tok + b);
            cx.tok[b] = tok < 0 ? 0 : (tok >= C::V ? C::V - 1 : tok);
        }
        ctr = (uint32_t)ld_uniform((const int*)a.ctr);
        cx.n_keys = cx.pos + 1;
        // 128-key chunks halve each item's chain of dependent arithmetic, where that needs no
        // more merging (a context of at most 128 keys, or one already split) than one round
        // of the merging item, and the items still fit the workgroups the QKV phase leaves free
        {
            constexpr int CH = NWAVE * KTILE, QKV_TILES = Geo<C::F, C::D, C::QKV, C::NL_D>::TILES;
            const int s_full = (cx.n_keys + CH - 1) / CH, s_half = (cx.n_keys + CH / 2 - 1) / (CH / 2);
            cx.half_chunks = (s_full >= 2 || s_half == 1) && s_half - 1 <= NWAVE &&
                             B * C::H * s_half <= (int)gridDim.x - QKV_TILES;
            cx.S = cx.half_chunks ? s_half : s_full;
        }
        cx.limit = a.spin_limit;
        n_layer = a.n_layer;
        lds_barrier();
        if (cx.pos < 0 || cx.pos >= a.n_ctx) {   // never index the cache outside the context
            if (threadIdx.x == 0) xchg::raise_abort(a.abort_word);
            return;
        }
        ep0 = ctr * (5u * (uint32_t)n_layer + 1u) + 1u;
    }

    for (int l = 0; l < n_layer; ++l) {
        // this layer's tensors are layer 0's moved by l strides; each phase derives only its own
        const uint32_t e = ep0 + 5u * (uint32_t)l;   // qkv e, partials e+1, attn-out stream e+2, h e+3, layer out e+4
        {   // 1. norm + QKV (+bias | RoPE) + K/V append
            const StepArgs& a = opaque(ap);
            const long long o = a.lstride * l;
            PhaseIO io{};
            io.src = a.x_out;
            io.src_xs = a.xs_d;
            io.src_ep = e - 1u;
            io.g = shift(a.L0.n1g, o);
            io.lc = shift(a.L0.cqkv, o);
            io.ld = shift(a.L0.dqkv, o);
            io.bias = shift(a.L0.bqkv, o);
            io.dst = a.x_qkv;
            io.dst_xs = a.xs_qkv;
            io.dst_ep = e;
            io.kc = a.L0.kc + a.kvstride * l;
            io.vc = a.L0.vc + a.kvstride * l;
            const PackedMat W = shift(a.L0.qkv, o);
            const bool ok = l == 0
                ? gemv_phase<C, C::D, C::QKV, C::NL_D, IN_EMB_NORM, OUT_QKV_K, C::GPT2>(a, cx, W, io, sm)
                : gemv_phase<C, C::D, C::QKV, C::NL_D, IN_NORM, OUT_QKV_K, C::GPT2>(a, cx, W, io, sm);
            if (!ok) return give_up(a);
        }
        {   // 2. attention partials
            const StepArgs& a = opaque(ap);
            const __half* kc = a.L0.kc + a.kvstride * l;
            const __half* vc = a.L0.vc + a.kvstride * l;
            if (!(cx.half_chunks ? attn_phase<C, KTILE / 2>(a, cx, kc, vc, e, e + 1u, sm)
                                 : attn_phase<C, KTILE>(a, cx, kc, vc, e, e + 1u, sm)))
                return give_up(a);
        }
        {   // 3. merge + output projection + bias + residual
            const StepArgs& a = opaque(ap);
            const long long o = a.lstride * l;
            PhaseIO io{};
            io.src = a.x_ao;
            io.src_xs = a.xs_ao;
            io.src_ep = e + 1u;
            io.bias = shift(a.L0.bo, o);
            io.dst = a.x_attn;
            io.dst_xs = a.xs_d;
            io.dst_ep = e + 2u;
            io.res = l == 0 ? nullptr : a.x_out;
            io.res_xs = a.xs_d;
            io.res_ep = e - 1u;
            if (!gemv_phase<C, C::QD, C::D, C::NL_O, IN_XCHG, OUT_RESID, false>(a, cx, shift(a.L0.o, o), io, sm))
                return give_up(a);
        }
        {   // 4. norm + FC (+bias, GELU) | gate/up (SwiGLU)
            const StepArgs& a = opaque(ap);
            const long long o = a.lstride * l;
            PhaseIO io{};
            io.src = a.x_attn;
            io.src_xs = a.xs_d;
            io.src_ep = e + 2u;
            io.g = shift(a.L0.n2g, o);
            io.lc = shift(a.L0.cfc, o);
            io.ld = shift(a.L0.dfc, o);
            io.bias = shift(a.L0.bfc, o);
            io.dst = a.x_h;
            io.dst_xs = a.xs_h;
            io.dst_ep = e + 3u;
            if (!gemv_phase<C, C::D, C::FCN, C::NL_FC, IN_NORM, OUT_FC_K, C::GPT2>(a, cx, shift(a.L0.fc, o), io, sm))
                return give_up(a);
        }
        {   // 5. down projection + bias + residual
            const StepArgs& a = opaque(ap);
            const long long o = a.lstride * l;
            PhaseIO io{};
            io.src = a.x_h;
            io.src_xs = a.xs_h;
            io.src_ep = e + 3u;
            io.bias = shift(a.L0.bdown, o);
            io.dst = a.x_out;
            io.dst_xs = a.xs_d;
            io.dst_ep = e + 4u;
            io.res = a.x_attn;
            io.res_xs = a.xs_d;
            io.res_ep = e + 2u;
            if (!gemv_phase<C, C::FF, C::D, C::NL_F, IN_XCHG32, OUT_RESID, false>(a, cx, shift(a.L0.down, o), io, sm))
                return give_up(a);
        }
    }

    const StepArgs& a = opaque(ap);
    // final norm + head (logits, per-workgroup best)
    const uint32_t eh = ep0 + 5u * (uint32_t)n_layer;
    PhaseIO io{};
    io.src = a.x_out;
    io.src_xs = a.xs_d;
    io.src_ep = eh - 1u;
    io.g = a.nfg;
    io.lc = a.hc;
    io.ld = a.hdv;
    io.dst = a.x_best;
    io.dst_xs = a.xs_best;
    io.dst_ep = eh;
    if (!gemv_phase<C, C::D, C::V, C::NL_HEAD, IN_NORM, OUT_HEAD, C::GPT2>(a, cx, a.head, io, sm)) return give_up(a);

    // the rows' picks: guided pairs make one pick that both rows take.  Each row records the
    // token it consumed (read before the pick overwrites it) at seq[pos][row] for the repetition
    // penalty of later steps, and its id at hist[pos][row]
    const bool guided = B == 2 && a.cfg;
    const int npick = guided ? 1 : B;
    if (a.samp_mode) {
        // the chain's draw of pick r on workgroup r (all of them on workgroup 0 of a one-workgroup grid)
        for (int r = blockIdx.x; r < npick; r += gridDim.x) {
            const int t = threadIdx.x;
            uint32_t* keys = (uint32_t*)raw;
            uint32_t* seen = (uint32_t*)(raw + KEYS_BYTES);
            samp::Scratch& S = *(samp::Scratch*)(raw + KEYS_BYTES + SEEN_BYTES);
            int cur[B];
#pragma unroll
            for (int b = 0; b < B; ++b) cur[b] = glb(a.tok)[b];
            const bool pen = a.chain.penalty != 1.f;
            __syncthreads();   // the previous pick's readers of the scratch are done
            if (pen) samp::build_seen<NT>(seen, C::V, a.seq + r, B, cx.pos, cur[r]);
            const uint32_t* sp = pen ? seen : nullptr;
            constexpr int JV = (C::V + NT - 1) / NT;
            const uint64_t* xl = a.x_logit + r * a.xs_logit;
            auto addr = [&](int q) { return xl + min(t + NT * q, C::V - 1); };
            uint64_t w[JV];
#pragma unroll
            for (int q = 0; q < JV; ++q) w[q] = xchg::load(addr(q));
            if (!xchg::settle_n(w, JV, addr, eh, cx.limit, a.abort_word)) s_abort = 1;
#pragma unroll
            for (int q = 0; q < JV; ++q)
                if (t + NT * q < C::V)
                    keys[samp::key_at(t + NT * q)] = samp::chain_key(xchg::value(w[q]), t + NT * q, a.chain, sp);
            __syncthreads();
            if (s_abort) return give_up(a);
            const float u = samp::uniform24(a.seed, (uint32_t)r, (uint32_t)cx.pos, 0u);
            const int id = samp::chain_draw<NT>(keys, C::V, a.chain, u, S, sp);
            if (t == 0) {
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    if (!guided && b != r) continue;
                    glb(a.seq)[(size_t)cx.pos * B + b] = cur[b];
                    glb(a.tok)[b] = id;
                    glb(a.hist)[(size_t)cx.pos * B + b] = id;
                }
            }
        }
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            *glb(a.pos) = cx.pos + 1;
            *glb(a.ctr) = ctr + 1u;
        }
        return;
    }
    if (blockIdx.x != 0) return;
    // greedy sampler, last stage (workgroup 0): the best of the per-workgroup keys of each row;
    // ties go to the lowest index because the key's low word is the inverted index
    constexpr int HEAD_TILES = Geo<C::F, C::D, C::V, C::NL_HEAD>::TILES;
    const int nb = min((int)gridDim.x, HEAD_TILES);
    __shared__ unsigned long long fkey[B][NWAVE];
    bool ok = true;
    for (int r = 0; r < npick; ++r) {
        unsigned long long bk = 0ull;
        for (int w = threadIdx.x; w < nb; w += NT) {
            float hl[2];
            ok &= xchg::wait_words<2>(a.x_best + r * a.xs_best + 2 * w, 1, eh, hl, cx.limit, a.abort_word);
            const unsigned long long key = ((unsigned long long)__float_as_uint(hl[0]) << 32) | __float_as_uint(hl[1]);
            bk = key > bk ? key : bk;
        }
        bk = wave_max_u64(bk);
        if ((threadIdx.x & 63) == 0) fkey[r][threadIdx.x >> 6] = bk;
    }
    if (!ok) s_abort = 1;
    lds_barrier();
    if (threadIdx.x == 0) {
        if (s_abort) {
            xchg::raise_abort(a.abort_word);
            return;
        }
        int cur[B], id[B];
#pragma unroll
        for (int b = 0; b < B; ++b) cur[b] = glb(a.tok)[b];
        for (int r = 0; r < npick; ++r) {
            unsigned long long m = fkey[r][0];
#pragma unroll
            for (int i = 1; i < NWAVE; ++i) m = fkey[r][i] > m ? fkey[r][i] : m;
            id[r] = (int)(0xFFFFFFFFu - (uint32_t)m);
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const int v = id[guided ? 0 : b];
            glb(a.seq)[(size_t)cx.pos * B + b] = cur[b];
            glb(a.tok)[b] = v;
            glb(a.hist)[(size_t)cx.pos * B + b] = v;
        }
        *glb(a.pos) = cx.pos + 1;
        *glb(a.ctr) = ctr + 1u;
    }
}

// the shapes with a persistent kernel: the decoders of the pages at their real sizes, and the
// small shapes the parity tests use; any other shape runs one launch per operator
struct Entry {
    int fmt, arch, d, h, hk, hd, ff, v, b;
    const void* fn;
};
template <int F, int A, int D, int H, int HK, int HD, int FF, int V, int B = 1>
Entry entry()
{
    return Entry{F, A, D, H, HK, HD, FF, V, B, (const void*)k_step<Shape<F, A, D, H, HK, HD, FF, V, B>>};
}

const Entry* entries(int& n)
{
    static const Entry tab[] = {
        entry<FMT_Q4_0, A_GPT2, 1024, 16, 16, 64, 4096, 8192>(),    // GPT-2-Medium-shaped T3, Q4_0
        entry<FMT_Q8_0, A_GPT2, 1024, 16, 16, 64, 4096, 8192>(),    //   and Q8_0
        entry<FMT_Q8_0, A_LLAMA, 1024, 16, 16, 64, 4096, 8192>(),   // Llama-shaped ~520M T3, Q8_0
        entry<FMT_Q4_0, A_LLAMA, 1024, 16, 16, 64, 4096, 8192>(),   //   and Q4_0
        entry<FMT_Q5_0, A_GPT2, 1024, 16, 16, 64, 4096, 8192>(),    // the T3 in the journal's Q5_0
        // two rows: a guided pair (classifier-free guidance) or two streams
        entry<FMT_Q4_0, A_GPT2, 1024, 16, 16, 64, 4096, 8192, 2>(),
        entry<FMT_Q8_0, A_LLAMA, 1024, 16, 16, 64, 4096, 8192, 2>(),
        entry<FMT_Q4_0, A_GPT2, 128, 2, 2, 64, 256, 160, 2>(),
        entry<FMT_Q8_0, A_LLAMA, 128, 2, 2, 64, 256, 160, 2>(),
        // test shapes
        entry<FMT_Q4_0, A_GPT2, 128, 2, 2, 64, 256, 160>(),
        entry<FMT_Q8_0, A_GPT2, 128, 2, 2, 64, 256, 160>(),
        entry<FMT_AFF8, A_GPT2, 128, 2, 2, 64, 256, 160>(),
        entry<FMT_Q4_0, A_LLAMA, 128, 2, 2, 64, 256, 160>(),
        entry<FMT_Q8_0, A_LLAMA, 128, 2, 2, 64, 256, 160>(),
        entry<FMT_AFF8, A_LLAMA, 128, 2, 2, 64, 256, 160>(),
        entry<FMT_Q4_0, A_GPT2, 128, 2, 2, 64, 256, 1000>(),
        entry<FMT_Q8_0, A_LLAMA, 256, 4, 2, 128, 256, 160>(),
        entry<FMT_Q5_0, A_GPT2, 128, 2, 2, 64, 256, 160>(),
        entry<FMT_Q5_0, A_LLAMA, 128, 2, 2, 64, 256, 160>(),
        entry<FMT_AFF4_G64, A_GPT2, 128, 2, 2, 64, 256, 160>(),
        entry<FMT_AFF4_G64, A_LLAMA, 128, 2, 2, 64, 256, 160>(),
        entry<FMT_AFF4_G32, A_GPT2, 128, 2, 2, 64, 256, 160>(),
        entry<FMT_AFF4_G32, A_LLAMA, 128, 2, 2, 64, 256, 160>(),
    };
    n = (int)(sizeof(tab) / sizeof(tab[0]));
    return tab;
}

}  // namespace

const void* step_kernel_for(int fmt, int arch_llama, int d, int h, int hk, int hd, int ff, int vocab, int batch)
{
    int n = 0;
    const Entry* t = entries(n);
    const int arch = arch_llama ? A_LLAMA : A_GPT2;
    for (int i = 0; i < n; ++i)
        if (t[i].fmt == fmt && t[i].arch == arch && t[i].d == d && t[i].h == h && t[i].hk == hk && t[i].hd == hd &&
            t[i].ff == ff && t[i].v == vocab && t[i].b == batch)
            return t[i].fn;
    return nullptr;
}

hipError_t launch_step(const void* kernel, const StepArgs* d_args, int n_wg, hipStream_t st)
{
    void* args[] = {(void*)&d_args};
    return hipLaunchKernel(kernel, dim3(n_wg), dim3(NT), args, 0, st);
}

}  // namespace tsd
