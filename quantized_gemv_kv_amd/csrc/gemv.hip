// gemv.hip — fused block-dequant GEMV for batch-1 decode on gfx950.
//
// What it computes ("Chatterbox -> ggml Port: Development Journal", §3.15/§3.16: the quantized
// mat-vec with its bias, and then its residual, added in the same kernel; §3.14/§3.23: one fused
// Q/K/V matrix whose output rows are Q, K, V; §3.21: SwiGLU as one fused op):
//     y = epilogue( W . prologue(x) )
// with W in Q4_0 / Q8_0 / affine-8 blocks, fp32 accumulation.
//
// Mapping onto CDNA4:
//   * a workgroup is 4 wave64s; every lane owns one 16-byte slot of a row (one dwordx4 load:
//     32 Q4_0 weights or 16 Q8_0 / affine weights) and keeps the matching slice of x in VGPRs,
//     so x is read from LDS once per lane, never per weight;
//   * a wave covers 64/slots-per-row rows per load when a row is shorter than the wave, or one
//     row per ceil(slots/64) loads when it is longer;
//   * order of issue: the input-vector loads first, then every weight and scale load of the
//     lane (unconditional, clamped addresses), and only then the wait for the input.  Vector
//     memory counters retire in order, so this is the order that lets the weight stream stay
//     in flight while the norm prologue (LayerNorm / RMSNorm, or the first layer's embedding
//     gather) runs; the prologue is recomputed by every workgroup from the 4 KB input, which
//     costs no extra launch;
//   * per-row partials are reduced with DPP row moves and cross-row swaps, no LDS traffic;
//   * the block scale multiplies the integer-weighted sum once per slot; the Q4_0 "-8" and the
//     Q8_0 "+128" storage offset are applied through the slot's precomputed sum of x.
#include <math.h>

#include "gemv_core.h"

namespace tsd {
namespace {

using namespace core;
constexpr int WG = 256;
constexpr int NWAVE = WG / 64;
constexpr int NJ = MAX_K / 4 / WG;   // float4 of the input per thread

template <int EPI>
__device__ __forceinline__ void epi_single(const EpiArgs& e, int row, float t, int pos)
{
    if (e.bias) t += e.bias[row];
    if constexpr (EPI == EPI_STORE || EPI == EPI_HEAD_ARGMAX) {
        e.y[row] = t;
    } else if constexpr (EPI == EPI_RESID) {
        e.y[row] += t;
    } else if constexpr (EPI == EPI_GELU) {
        e.y[row] = gelu_tanh(t);
    } else if constexpr (EPI == EPI_QKV) {
        if (row < e.qrows) {
            e.q[row] = t;
        } else {
            const bool isk = row < e.qrows + e.krows;
            const int r = isk ? row - e.qrows : row - e.qrows - e.krows;
            const int h = r / e.hd, i = r - h * e.hd;
            __half* c = isk ? e.kc : e.vc;
            c[((size_t)h * e.n_ctx + pos) * e.hd + i] = __float2half_rn(t);
        }
    }
}

// rows (row, row+1), row even
template <int EPI>
__device__ __forceinline__ void epi_pair(const EpiArgs& e, int row, float t0, float t1, int pos)
{
    if constexpr (EPI == EPI_SWIGLU) {
        e.y[row >> 1] = silu(t0) * t1;
    } else if constexpr (EPI == EPI_QKV_ROPE) {
        const int half = e.hd >> 1;
        if (row < e.qrows + e.krows) {
            const bool isk = row >= e.qrows;
            const int m = (isk ? row - e.qrows : row) >> 1;   // pair index within Q or K
            const int h = m / half, i = m - h * half;
            const float2 cs = e.rope[(size_t)pos * half + i];
            const float a = t0 * cs.x - t1 * cs.y, bb = t0 * cs.y + t1 * cs.x;
            if (!isk) {
                e.q[h * e.hd + i] = a;
                e.q[h * e.hd + i + half] = bb;
            } else {
                __half* c = e.kc + ((size_t)h * e.n_ctx + pos) * e.hd;
                c[i] = __float2half_rn(a);
                c[i + half] = __float2half_rn(bb);
            }
        } else {
            const int r = row - e.qrows - e.krows;
            const int h = r / e.hd, i = r - h * e.hd;
            __half* c = e.vc + ((size_t)h * e.n_ctx + pos) * e.hd;
            c[i] = __float2half_rn(t0);
            c[i + 1] = __float2half_rn(t1);
        }
    }
}

template <int EPI> struct EpiIsPair { static constexpr bool v = EPI == EPI_SWIGLU || EPI == EPI_QKV_ROPE; };

// STREAM: the weight loads carry the non-temporal hint (a matrix read once, larger than the
// caches: the hint keeps it from displacing what stays resident and streams measurably faster)
template <int F, int SPL, int NLOAD, int PRO, int EPI, bool STREAM = false>
__global__ __launch_bounds__(WG) void k_gemv(const PackedMat W, const ProArgs pa0, const EpiArgs ea0)
{
    // batch row blockIdx.y: its input, output, cache and key pointers
    ProArgs pa = pa0;
    EpiArgs ea = ea0;
    if (blockIdx.y) {
        const long long b = blockIdx.y;
        if (pa.src) pa.src += b * pa.rs_src;
        if (pa.x_out) pa.x_out += b * pa.rs_src;
        if (pa.tok) pa.tok += b * pa.rs_tok;
        if (pa.part) pa.part += b * pa.rs_part;
        if (ea.y) ea.y += b * ea.rs_y;
        if (ea.q) ea.q += b * ea.rs_q;
        if (ea.kc) ea.kc += b * ea.rs_kv;
        if (ea.vc) ea.vc += b * ea.rs_kv;
        if (ea.best) ea.best += b * gridDim.x;
    }
    constexpr int E = FmtT<F>::E, SPS = FmtT<F>::SLOTS_PER_SCALE, G = FmtT<F>::SCALE_GROUP;
    constexpr int RWS = SPL == 1 ? 1 : NLOAD / SPL;       // rows per wave when rows span loads
    constexpr int NP = SPL == 1 ? NLOAD : RWS;             // partial sums per lane
    constexpr bool PAIR = EpiIsPair<EPI>::v;
    static_assert(SPL == 1 || NLOAD % SPL == 0, "whole rows per wave");
    static_assert(!PAIR || NP % 2 == 0, "pair epilogues need an even number of rows per lane");

    extern __shared__ float4 xl4[];   // [K / 4], sized at launch (a fixed MAX_K buffer would cost occupancy)
    __shared__ float red[2 * NWAVE];
    __shared__ unsigned long long bkey[NWAVE];

    const int K = W.K, N = W.N, lpr = K / E;
    const size_t rb = fmt_row_bytes(F, K);
    const int spr = K / G;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int slot0 = SPL == 1 ? (lane & (lpr - 1)) : lane;
    const int sub = SPL == 1 ? lane / lpr : 0;
    const int rpw = SPL == 1 ? NLOAD * (64 / lpr) : RWS;
    const int row0 = (blockIdx.x * NWAVE + wave) * rpw;

    // 1. the input vector's loads first ...
    float4 xv[NJ], xg[NJ], xb[NJ];
    AttnIn att;
    if constexpr (PRO == PRO_ATTN) load_attn<WG>(pa, K, att);
    else load_x<PRO, WG>(pa, K, xv, xg, xb);

    // 2. ... then every weight and raw scale of this lane, unconditionally (clamped address;
    //    out-of-range slots get a zero scale)
    uint4 w[NLOAD];
    uint32_t sc_raw[NLOAD], sb_raw[NLOAD];   // 32-bit: 16-bit elements would be packed, forcing a wait per load
    uint32_t h_raw[NLOAD];                   // Q5_0 fifth bits
    bool ok[NLOAD];
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) {
        const int row = SPL == 1 ? row0 + sub * NLOAD + i : row0 + i / SPL;
        const int slot = SPL == 1 ? slot0 : (i % SPL) * 64 + lane;
        ok[i] = row < N && slot < lpr;
        const int rr = row < N ? row : N - 1, ss = slot < lpr ? slot : lpr - 1;
        const uint4* wp = (const uint4*)(W.q + (size_t)rr * rb + (size_t)ss * 16);
        if constexpr (STREAM) {
            typedef unsigned int v4u __attribute__((ext_vector_type(4)));
            const v4u v = __builtin_nontemporal_load((const v4u*)wp);
            w[i] = make_uint4(v.x, v.y, v.z, v.w);
        } else {
            w[i] = *wp;
        }
        sc_raw[i] = __half_as_ushort(W.s[(size_t)rr * spr + ss / SPS]);
        sb_raw[i] = 0u;
        h_raw[i] = 0u;
        if constexpr (fmt_affine(F)) sb_raw[i] = __half_as_ushort(W.b[(size_t)rr * spr + ss / SPS]);
        if constexpr (F == FMT_Q5_0) h_raw[i] = W.h[(size_t)rr * (K / 32) + ss];
    }

    asm volatile("" ::: "memory");   // keep every load above: all in flight before any wait
    __builtin_amdgcn_sched_barrier(0);

    // 3. norm / embedding / attention merge into LDS (waits for the input only)
    if constexpr (PRO == PRO_ATTN) finish_attn<WG>(pa, K, att, xv);
    finish_x<F, PRO, WG>(pa, K, xv, xg, xb, xl4, red);

    // 4. this lane's x slices and their sums
    float xs[SPL][E];
    float sx[SPL];
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
        const int slot = SPL == 1 ? slot0 : j * 64 + lane;
        float s = 0.f;
#pragma unroll
        for (int e4 = 0; e4 < E / 4; ++e4) {
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (slot < lpr) v = xl4[e4 * lpr + slot];
            xs[j][4 * e4 + 0] = v.x;
            xs[j][4 * e4 + 1] = v.y;
            xs[j][4 * e4 + 2] = v.z;
            xs[j][4 * e4 + 3] = v.w;
            s += (v.x + v.y) + (v.z + v.w);
        }
        sx[j] = s;
    }

    // 5. dequantize-and-dot
    float part[NP];
#pragma unroll
    for (int r = 0; r < NP; ++r) part[r] = 0.f;
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) {
        const int j = SPL == 1 ? 0 : i % SPL;
        const int r = SPL == 1 ? i : i / SPL;
        const float d = slot_dot<F>(w[i], xs[j], h_raw[i]);
        const float sc = ok[i] ? __half2float(__ushort_as_half((unsigned short)sc_raw[i])) : 0.f;
        const float sb = ok[i] ? __half2float(__ushort_as_half((unsigned short)sb_raw[i])) : 0.f;
        part[r] += slot_value<F>(d, sx[j], sc, sb);
    }

    // 6. reduce over the lanes sharing a row
#pragma unroll
    for (int r = 0; r < NP; ++r) part[r] = group_sum(part[r], SPL == 1 ? lpr : 64);

    // 7. epilogue, one lane per row group (the head writes no logits after a rejected input)
    bool leader = SPL == 1 ? slot0 == 0 : lane == 0;
    if constexpr (EPI == EPI_HEAD_ARGMAX) {
        if (ea.err && ld_uniform((const int*)ea.err)) leader = false;
    }
    const int pos = (EPI == EPI_QKV || EPI == EPI_QKV_ROPE) ? ld_uniform(ea.pos) : 0;
    unsigned long long best = 0ull;
    if (leader) {
#pragma unroll
        for (int r = 0; r < NP; ++r) {
            const int row = SPL == 1 ? row0 + sub * NLOAD + r : row0 + r;
            if constexpr (PAIR) {
                if ((r & 1) == 0 && row < N) epi_pair<EPI>(ea, row, part[r], part[r + 1], pos);
            } else {
                if (row < N) {
                    epi_single<EPI>(ea, row, part[r], pos);
                    if constexpr (EPI == EPI_HEAD_ARGMAX) {
                        const unsigned long long key =
                            ((unsigned long long)float_order_key(part[r]) << 32) | (0xFFFFFFFFu - (uint32_t)row);
                        best = key > best ? key : best;
                    }
                }
            }
        }
    }
    if constexpr (EPI == EPI_HEAD_ARGMAX) {
        // greedy sampler, first stage: the workgroup's best key (ordered logit, ~index: ties go
        // to the lowest index); one plain store per workgroup, reduced by the finalize kernel
        best = wave_max_u64(best);
        if (lane == 0) bkey[wave] = best;
        lds_barrier();
        if (threadIdx.x == 0) {
            unsigned long long m = bkey[0];
#pragma unroll
            for (int i = 1; i < NWAVE; ++i) m = bkey[i] > m ? bkey[i] : m;
            ea.best[blockIdx.x] = m;
        }
    }
}

// ---- host dispatch ---------------------------------------------------------------------------

int spl_for(int fmt, int K)
{
    const int lpr = K / fmt_elems_per_slot(fmt);
    return lpr <= 64 ? 1 : (lpr + 63) / 64;
}

template <int SPL> constexpr int nload_for() { return SPL == 1 ? 2 : 2 * SPL; }

int rows_per_block_impl(int fmt, int K)
{
    const int spl = spl_for(fmt, K);
    const int lpr = K / fmt_elems_per_slot(fmt);
    const int rpw = spl == 1 ? 2 * (64 / lpr) : 2;
    return NWAVE * rpw;
}

template <int F, int PRO, int EPI, int SPL, bool STREAM = false>
hipError_t go(const PackedMat& W, const ProArgs& pa, const EpiArgs& ea, hipStream_t st, int B = 1)
{
    // a streamed matrix keeps twice the loads in flight per lane when a row fits one wave
    constexpr int NLOAD = STREAM && SPL == 1 ? 4 : nload_for<SPL>();
    const int lpr = W.K / FmtT<F>::E;
    const int rpb = NWAVE * (SPL == 1 ? NLOAD * (64 / lpr) : NLOAD / SPL);
    const int grid = (W.N + rpb - 1) / rpb;
    hipLaunchKernelGGL((k_gemv<F, SPL, NLOAD, PRO, EPI, STREAM>), dim3(grid, B), dim3(WG), (size_t)W.K * sizeof(float), st, W,
                       pa, ea);
    return hipGetLastError();
}

template <int F, int PRO, int EPI, bool STREAM = false>
hipError_t go_spl(const PackedMat& W, const ProArgs& pa, const EpiArgs& ea, hipStream_t st, int B = 1)
{
    switch (spl_for(F, W.K)) {
    case 1: return go<F, PRO, EPI, 1, STREAM>(W, pa, ea, st, B);
    case 2: return go<F, PRO, EPI, 2, STREAM>(W, pa, ea, st, B);
    case 3: return go<F, PRO, EPI, 3, STREAM>(W, pa, ea, st, B);
    case 4: return go<F, PRO, EPI, 4, STREAM>(W, pa, ea, st, B);
    default: return hipErrorInvalidValue;
    }
}

template <int F>
hipError_t go_fmt(int pro, int epi, const PackedMat& W, const ProArgs& pa, const EpiArgs& ea, hipStream_t st, int B)
{
#define TSD_CASE(PRO_, EPI_) \
    if (pro == PRO_ && epi == EPI_) return go_spl<F, PRO_, EPI_>(W, pa, ea, st, B);
    TSD_CASE(PRO_LOAD, EPI_STORE)
    TSD_CASE(PRO_LOAD, EPI_RESID)
    TSD_CASE(PRO_ATTN, EPI_RESID)
    TSD_CASE(PRO_LN, EPI_GELU)
    TSD_CASE(PRO_RMS, EPI_SWIGLU)
    TSD_CASE(PRO_LN, EPI_QKV)
    TSD_CASE(PRO_RMS, EPI_QKV_ROPE)
    TSD_CASE(PRO_LN_EMB, EPI_QKV)
    TSD_CASE(PRO_RMS_EMB, EPI_QKV_ROPE)
    TSD_CASE(PRO_LN, EPI_HEAD_ARGMAX)
    TSD_CASE(PRO_RMS, EPI_HEAD_ARGMAX)
    TSD_CASE(PRO_LN, EPI_STORE)
    TSD_CASE(PRO_RMS, EPI_STORE)
#undef TSD_CASE
    return hipErrorInvalidValue;
}

// ---- repack canonical blocks into the kernel layout ----------------------------------------
// one thread per (source row, scale group); `mode` places source row r at destination row
// place_row(r, mode, hd, row0) (kernels.h)
__global__ void k_pack(int fmt, const uint8_t* __restrict__ src, int N, int K, uint8_t* dq, __half* ds,
                       __half* db, uint32_t* dh, int mode, int hd, int row0)
{
    const int G = fmt_group(fmt), gpr = K / G;
    const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long long)N * gpr) return;
    const int r = (int)(idx / gpr), g = (int)(idx - (long long)r * gpr);
    const int dr = place_row(r, mode, hd, row0);
    if (fmt == FMT_Q4_0) {
        const uint8_t* blk = src + ((size_t)r * gpr + g) * 18;
        uint8_t* o = dq + (size_t)dr * (K / 2) + (size_t)g * 16;
        for (int j = 0; j < 16; ++j) o[j] = blk[2 + j];
        ds[(size_t)dr * gpr + g] = __ushort_as_half((unsigned short)(blk[0] | (blk[1] << 8)));
    } else if (fmt == FMT_Q8_0) {
        const uint8_t* blk = src + ((size_t)r * gpr + g) * 34;
        uint8_t* o = dq + (size_t)dr * K + (size_t)g * 32;
        for (int j = 0; j < 32; ++j) o[j] = (uint8_t)(blk[2 + j] ^ 0x80u);   // int8 q -> q + 128
        ds[(size_t)dr * gpr + g] = __ushort_as_half((unsigned short)(blk[0] | (blk[1] << 8)));
    } else if (fmt == FMT_Q5_0) {
        const uint8_t* blk = src + ((size_t)r * gpr + g) * 22;
        uint8_t* o = dq + (size_t)dr * (K / 2) + (size_t)g * 16;
        for (int j = 0; j < 16; ++j) o[j] = blk[6 + j];
        ds[(size_t)dr * gpr + g] = __ushort_as_half((unsigned short)(blk[0] | (blk[1] << 8)));
        dh[(size_t)dr * gpr + g] = (uint32_t)blk[2] | ((uint32_t)blk[3] << 8) | ((uint32_t)blk[4] << 16) | ((uint32_t)blk[5] << 24);
    } else if (fmt == FMT_AFF4_G64 || fmt == FMT_AFF4_G32) {
        // canonical: element 2i low / 2i+1 high nibble of byte i; packed: per 32-element slot,
        // byte b holds element b (low) and b + 16 (high)
        const uint8_t* q = src + (size_t)r * (K / 2) + (size_t)g * (G / 2);
        const uint8_t* s = src + (size_t)N * (K / 2) + ((size_t)r * gpr + g) * 2;
        const uint8_t* b = src + (size_t)N * (K / 2) + (size_t)N * gpr * 2 + ((size_t)r * gpr + g) * 2;
        uint8_t* o = dq + (size_t)dr * (K / 2) + (size_t)g * (G / 2);
        auto nib = [&](int e) { return (q[e >> 1] >> (4 * (e & 1))) & 15; };
        for (int sl = 0; sl < G / 32; ++sl)
            for (int j = 0; j < 16; ++j)
                o[sl * 16 + j] = (uint8_t)(nib(sl * 32 + j) | (nib(sl * 32 + j + 16) << 4));
        ds[(size_t)dr * gpr + g] = __ushort_as_half((unsigned short)(s[0] | (s[1] << 8)));
        db[(size_t)dr * gpr + g] = __ushort_as_half((unsigned short)(b[0] | (b[1] << 8)));
    } else {
        const uint8_t* q = src + (size_t)r * K + (size_t)g * 64;
        const uint8_t* s = src + (size_t)N * K + ((size_t)r * gpr + g) * 2;
        const uint8_t* b = src + (size_t)N * K + (size_t)N * gpr * 2 + ((size_t)r * gpr + g) * 2;
        uint8_t* o = dq + (size_t)dr * K + (size_t)g * 64;
        for (int j = 0; j < 64; ++j) o[j] = q[j];
        ds[(size_t)dr * gpr + g] = __ushort_as_half((unsigned short)(s[0] | (s[1] << 8)));
        db[(size_t)dr * gpr + g] = __ushort_as_half((unsigned short)(b[0] | (b[1] << 8)));
    }
}

}  // namespace

int gemv_rows_per_block(int fmt, int K, int) { return rows_per_block_impl(fmt, K); }

namespace {
__global__ __launch_bounds__(256) void k_argmax_finalize(const unsigned long long* __restrict__ best, int n, int B, int* tok,
                                                         int* hist, int* seq, int hist_stride, int* pos,
                                                         const uint32_t* err)
{
    __shared__ unsigned long long bk[NWAVE];
    if (err && ld_uniform((const int*)err)) return;   // a rejected input: the state stays as it was
    const int p = *pos;   // every row is read before the position advances (one workgroup)
    for (int r = 0; r < B; ++r) {
        unsigned long long m = 0ull;
        for (int i = threadIdx.x; i < n; i += WG) m = best[(size_t)r * n + i] > m ? best[(size_t)r * n + i] : m;
        m = wave_max_u64(m);
        if ((threadIdx.x & 63) == 0) bk[threadIdx.x >> 6] = m;
        __syncthreads();
        if (threadIdx.x == 0) {
            unsigned long long b = bk[0];
            for (int i = 1; i < NWAVE; ++i) b = bk[i] > b ? bk[i] : b;
            const int id = (int)(0xFFFFFFFFu - (uint32_t)(b & 0xFFFFFFFFull));
            if (seq) seq[(size_t)p * hist_stride + r] = tok[r];
            tok[r] = id;
            if (hist) hist[(size_t)p * hist_stride + r] = id;
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) *pos = p + 1;
}
}  // namespace

hipError_t launch_argmax_finalize(const unsigned long long* best, int n, int B, int* tok, int* hist, int* seq, int hist_stride,
                                  int* pos, const uint32_t* err, hipStream_t st)
{
    hipLaunchKernelGGL(k_argmax_finalize, dim3(1), dim3(WG), 0, st, best, n, B, tok, hist, seq, hist_stride, pos, err);
    return hipGetLastError();
}

hipError_t launch_gemv(int fmt, int pro, int epi, const PackedMat& W, const ProArgs& pa, const EpiArgs& ea,
                       hipStream_t st, int B)
{
    if (W.K > MAX_K || !gemv_shape_ok(fmt, W.K) || W.N <= 0 || B < 1 || B > 65535) return hipErrorInvalidValue;
    if (pro == PRO_ATTN && W.K > 4 * NJA * WG) return hipErrorInvalidValue;
    switch (fmt) {
    case FMT_Q4_0: return go_fmt<FMT_Q4_0>(pro, epi, W, pa, ea, st, B);
    case FMT_Q8_0: return go_fmt<FMT_Q8_0>(pro, epi, W, pa, ea, st, B);
    case FMT_AFF8: return go_fmt<FMT_AFF8>(pro, epi, W, pa, ea, st, B);
    case FMT_Q5_0: return go_fmt<FMT_Q5_0>(pro, epi, W, pa, ea, st, B);
    case FMT_AFF4_G64: return go_fmt<FMT_AFF4_G64>(pro, epi, W, pa, ea, st, B);
    case FMT_AFF4_G32: return go_fmt<FMT_AFF4_G32>(pro, epi, W, pa, ea, st, B);
    default: return hipErrorInvalidValue;
    }
}

namespace {
// sum over a slot of 32 four-bit codes in Q4_0's nibble order times x, where the x of the high
// nibbles (elements 16..31) has already been divided by 16: a high code is then used in place,
// as the byte value 16 q (one mask per word instead of a shift and a mask), and each product
// (16 q) (x / 16) is exactly q x
__device__ __forceinline__ float slot_dot_hi16(const uint4 w, const float* __restrict__ x)
{
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t lo = ws[j] & 0x0F0F0F0Fu, hi = ws[j] & 0xF0F0F0F0u;
        a0 = fmaf(ubyte<0>(lo), x[4 * j + 0], a0);
        a1 = fmaf(ubyte<0>(hi), x[16 + 4 * j + 0], a1);
        a0 = fmaf(ubyte<1>(lo), x[4 * j + 1], a0);
        a1 = fmaf(ubyte<1>(hi), x[16 + 4 * j + 1], a1);
        a0 = fmaf(ubyte<2>(lo), x[4 * j + 2], a0);
        a1 = fmaf(ubyte<2>(hi), x[16 + 4 * j + 2], a1);
        a0 = fmaf(ubyte<3>(lo), x[4 * j + 3], a0);
        a1 = fmaf(ubyte<3>(hi), x[16 + 4 * j + 3], a1);
    }
    return a0 + a1;
}

// y = W x (+bias) for a matrix streamed once, rows of at most one wave (slots per row a power of
// two <= 64): every lane issues its NL weight loads (non-temporal) and scale loads first, then x
// is staged in LDS, then the lane dots its slot with each of its rows.  With eight rows per lane
// the partial sums are reduced across the row group by a butterfly that halves them at each of
// its first three stages (each lane keeps one half and sends the other to its partner: seven
// lane moves and adds instead of eight full reductions), after which lane s holds the total of
// row s % 8; with four, each row is reduced on its own.  Lane s < NL stores row s.
template <int F, int NL>
__global__ __launch_bounds__(WG) void k_gemv_stream(const PackedMat W, const float* __restrict__ x,
                                                    const float* __restrict__ bias, float* __restrict__ y)
{
    constexpr int E = FmtT<F>::E, SPS = FmtT<F>::SLOTS_PER_SCALE, G = FmtT<F>::SCALE_GROUP;
    constexpr bool HI16 = fmt_nibbles(F) && F != FMT_Q5_0;   // Q5_0's fifth bit does not fit 16 q
    static_assert(NL == 4 || NL == 8, "four or eight rows per lane");
    extern __shared__ float4 xl4[];
    const int K = W.K, N = W.N, lpr = K / E, spr = K / G;
    const size_t rb = fmt_row_bytes(F, K);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lsh = __ffs(lpr) - 1;   // lpr is a power of two
    const int slot = lane & (lpr - 1), sub = lane >> lsh;
    const int row0 = ((blockIdx.x * NWAVE + wave) * (64 >> lsh) + sub) * NL;
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    // 32-bit byte offsets from the arrays' bases (the launcher keeps this kernel to matrices of
    // less than 4 GB) and 24-bit multiplies: no 64-bit or quarter-rate arithmetic per row; rows
    // past the matrix (j > lim) reload its last row, whose result no lane stores
    const int lim = N - 1 - row0;
    const uint32_t q0 = (uint32_t)row0 * (uint32_t)rb + (uint32_t)slot * 16u;
    const uint32_t s0 = (uint32_t)row0 * (uint32_t)spr + (uint32_t)(slot / SPS);
    const uint32_t h0 = (uint32_t)row0 * (uint32_t)(K / 32) + (uint32_t)slot;
    uint4 w[NL];
    uint32_t sc[NL], sb[NL], hb[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int j = min(i, lim);
        const uint32_t so = 2u * (s0 + (uint32_t)__mul24(j, spr));
        const v4u v = __builtin_nontemporal_load((const v4u*)(W.q + (q0 + (uint32_t)__mul24(j, (int)rb))));
        w[i] = make_uint4(v.x, v.y, v.z, v.w);
        sc[i] = *(const unsigned short*)((const uint8_t*)W.s + so);
        sb[i] = 0u;
        hb[i] = 0u;
        if constexpr (fmt_affine(F)) sb[i] = *(const unsigned short*)((const uint8_t*)W.b + so);
        if constexpr (F == FMT_Q5_0) hb[i] = *(const uint32_t*)((const uint8_t*)W.h + 4u * (h0 + (uint32_t)__mul24(j, K / 32)));
    }
    const int er = min(row0 + (slot < NL ? slot : NL - 1), N - 1);
    const float bv = bias ? bias[er] : 0.f;
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // x staged in LDS; for the nibble formats the high half of every 32-element block (elements
    // 16..31, the high nibbles) is stored divided by 16 (see slot_dot_hi16)
    for (int c = threadIdx.x; c < K / 4; c += WG) {
        float4 v = ((const float4*)x)[c];
        if (HI16 && (c & 7) >= 4) v = make_float4(v.x * 0.0625f, v.y * 0.0625f, v.z * 0.0625f, v.w * 0.0625f);
        xl4[swz<E>(4 * c, lpr)] = v;
    }
    __syncthreads();
    float xs[E];
    float sl = 0.f, sh = 0.f;   // the slot's sums of x over its low and high halves (high: / 16)
#pragma unroll
    for (int e4 = 0; e4 < E / 4; ++e4) {
        const float4 v = xl4[e4 * lpr + slot];
        xs[4 * e4] = v.x;
        xs[4 * e4 + 1] = v.y;
        xs[4 * e4 + 2] = v.z;
        xs[4 * e4 + 3] = v.w;
        if (HI16 && e4 >= 4) sh += (v.x + v.y) + (v.z + v.w);
        else sl += (v.x + v.y) + (v.z + v.w);
    }
    const float sx = HI16 ? fmaf(16.f, sh, sl) : sl;
    float p[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        float d;
        if constexpr (HI16) d = slot_dot_hi16(w[i], xs);
        else d = slot_dot<F>(w[i], xs, hb[i]);
        p[i] = slot_value<F>(d, sx, __half2float(__ushort_as_half((unsigned short)sc[i])),
                             __half2float(__ushort_as_half((unsigned short)sb[i])));
    }
    float t;
    if constexpr (NL == 8) {
        // stage 1: partner slot ^ 7 (half-row mirror), the half kept chosen by slot bit 2; then
        // partner slot ^ 2 by bit 1, and slot ^ 1 by bit 0: lane s keeps row s % 8
        const bool k2 = slot & 4, k1 = slot & 2, k0 = slot & 1;
        float q[4], r[2];
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = (k2 ? p[i + 4] : p[i]) + dpp_mov<0x141>(k2 ? p[i] : p[i + 4]);
#pragma unroll
        for (int i = 0; i < 2; ++i) r[i] = (k1 ? q[i + 2] : q[i]) + dpp_mov<0x4E>(k1 ? q[i] : q[i + 2]);
        t = (k0 ? r[1] : r[0]) + dpp_mov<0xB1>(k0 ? r[0] : r[1]);
        // the lanes 8, 16 and 32 apart hold the same row
        if (lpr >= 16) t += dpp_mov<0x128>(t);   // row_ror:8
        if (lpr >= 32) t = swap16_sum(t);
        if (lpr >= 64) t = swap32_sum(t);
    } else {
        float part[NL];
#pragma unroll
        for (int i = 0; i < NL; ++i) part[i] = group_sum(p[i], lpr);
        t = part[0];
#pragma unroll
        for (int i = 1; i < NL; ++i) t = slot == i ? part[i] : t;
    }
    if (slot < NL && row0 + slot < N) y[row0 + slot] = t + bv;
}
}  // namespace

hipError_t launch_gemv_stream(int fmt, const PackedMat& W, const ProArgs& pa, const EpiArgs& ea, hipStream_t st)
{
    if (W.K > MAX_K || !gemv_shape_ok(fmt, W.K) || W.N <= 0) return hipErrorInvalidValue;
    const int lpr = W.K / fmt_elems_per_slot(fmt);
    // rows fit one wave, a row group holds at least NL lanes and the payload is under 4 GB (the
    // kernel's 32-bit offsets); the 4-bit formats take eight rows per lane (their per-lane
    // overhead, spread over twice the codes)
    const int nl = fmt_nibbles(fmt) && lpr >= 8 ? 8 : 4;
    if (lpr <= 64 && lpr >= 4 && (size_t)W.N * fmt_row_bytes(fmt, W.K) < ((size_t)1 << 32)) {
        const int rpb = NWAVE * (64 / lpr) * nl;
        const dim3 grid((W.N + rpb - 1) / rpb);
        const size_t lds = (size_t)W.K * sizeof(float);
#define TSD_STREAM(F_, NL_) \
    if (fmt == F_ && nl == NL_) hipLaunchKernelGGL((k_gemv_stream<F_, NL_>), grid, dim3(WG), lds, st, W, pa.src, ea.bias, ea.y);
        TSD_STREAM(FMT_Q4_0, 4) TSD_STREAM(FMT_Q8_0, 4) TSD_STREAM(FMT_AFF8, 4) TSD_STREAM(FMT_Q5_0, 4)
        TSD_STREAM(FMT_AFF4_G64, 4) TSD_STREAM(FMT_AFF4_G32, 4)
        TSD_STREAM(FMT_Q4_0, 8) TSD_STREAM(FMT_Q5_0, 8) TSD_STREAM(FMT_AFF4_G64, 8) TSD_STREAM(FMT_AFF4_G32, 8)
#undef TSD_STREAM
        return hipGetLastError();
    }
    switch (fmt) {
    case FMT_Q4_0: return go_spl<FMT_Q4_0, PRO_LOAD, EPI_STORE, true>(W, pa, ea, st);
    case FMT_Q8_0: return go_spl<FMT_Q8_0, PRO_LOAD, EPI_STORE, true>(W, pa, ea, st);
    case FMT_AFF8: return go_spl<FMT_AFF8, PRO_LOAD, EPI_STORE, true>(W, pa, ea, st);
    case FMT_Q5_0: return go_spl<FMT_Q5_0, PRO_LOAD, EPI_STORE, true>(W, pa, ea, st);
    case FMT_AFF4_G64: return go_spl<FMT_AFF4_G64, PRO_LOAD, EPI_STORE, true>(W, pa, ea, st);
    case FMT_AFF4_G32: return go_spl<FMT_AFF4_G32, PRO_LOAD, EPI_STORE, true>(W, pa, ea, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_pack(int fmt, const void* src, int N, int K, void* dst_base, int dst_N, int dst_row0, int mode,
                       int hd, hipStream_t st)
{
    PackedLayout L = packed_layout(fmt, dst_N, K);
    uint8_t* base = (uint8_t*)dst_base;
    const long long n = (long long)N * (K / fmt_group(fmt));
    const int threads = 256;
    const long long blocks = (n + threads - 1) / threads;
    hipLaunchKernelGGL(k_pack, dim3((unsigned)blocks), dim3(threads), 0, st, fmt, (const uint8_t*)src, N, K,
                       base + L.q_off, (__half*)(base + L.s_off), fmt_affine(fmt) ? (__half*)(base + L.b_off) : nullptr,
                       fmt == FMT_Q5_0 ? (uint32_t*)(base + L.h_off) : nullptr,
                       mode, hd, dst_row0);
    return hipGetLastError();
}

}  // namespace tsd
