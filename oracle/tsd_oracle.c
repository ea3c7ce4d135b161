/*
 * tsd_oracle.c — the CPU oracle for the quantized speech-token decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Plain C, single-threaded, fp64 arithmetic, no blocking, no fusion.
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * nothing with the HIP library (no header, no helper, no table); the only thing both sides see
 * is the canonical byte layout of the weights, which each decodes with its own code.
 *
 * Pages followed:
 *   [J] "Chatterbox -> ggml Port: Development Journal"
 *   [F] "Every Frame Is a Memory Read: A Systems View of Speech Model Inference on Apple Silicon"
 *
 * Readings of points the pages leave open are marked READING and are the same as those listed
 * with the design notes (block field order, nibble order, affine layout, GELU variant, eps,
 * RoPE convention, head without bias, greedy tie-break, top-k draw, code-predictor wiring).
 *
 * Pinning: every function below is checked by the CPU tests against closed forms, library
 * routines, brute force or invariants (tests/test_oracle_*.py).  The whole-model functions are
 * pinned only through those invariants and through the sequence-vs-step identity; beyond that
 * their parity is unpinned, because the pages print no logits for synthetic weights.
 */
#include "tsd_oracle.h"

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static char g_err[512];
static void set_err(const char* m) { snprintf(g_err, sizeof g_err, "%s", m); }
const char* orc_last_error(void) { return g_err; }

/* ------------------------------------------------------------------------------------------ */
/* IEEE-754 binary16, written from the format definition (1 sign, 5 exponent, 10 fraction bits,
 * bias 15).  Pinned against numpy's float16 conversion on normals, subnormals, ties and
 * overflow. */
double orc_half_to_double(uint16_t h)
{
    int s = (h >> 15) & 1, e = (h >> 10) & 31, f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return s ? -v : v;
}

/* round half to even of a non-negative double that is exactly representable */
static double rne(double q)
{
    double fl = floor(q), diff = q - fl;
    if (diff > 0.5) return fl + 1.0;
    if (diff < 0.5) return fl;
    return fmod(fl, 2.0) == 0.0 ? fl : fl + 1.0;
}

uint16_t orc_double_to_half(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x)) return 0x7E00u;
    double a = fabs(x);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | 0x7C00u;
    if (a < ldexp(1.0, -14)) {                 /* subnormal range: units of 2^-24 */
        double r = rne(ldexp(a, 24));          /* r == 1024 is the smallest normal, 0x0400 */
        return (uint16_t)(sign | (uint16_t)r);
    }
    int e;
    double f = frexp(a, &e);                   /* a = f * 2^e, f in [0.5, 1) */
    int E = e - 1;                             /* a = (2f) * 2^E */
    double r = rne(ldexp(f, 11));              /* 2f * 1024 in [1024, 2048] */
    if (r == 2048.0) { r = 1024.0; E += 1; }
    if (E > 15) return sign | 0x7C00u;         /* >= 65520 rounds to infinity */
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(r - 1024.0));
}

/* ------------------------------------------------------------------------------------------ */
/* Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3",
 * SC 2011): ten rounds of two 64x64->128 multiplies with a Weyl key schedule.  Pinned against
 * numpy.random.Philox, which implements the same generator. */
void orc_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4])
{
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
    uint64_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint64_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) { k0 += W0; k1 += W1; }
        unsigned __int128 p0 = (unsigned __int128)M0 * c0;
        unsigned __int128 p1 = (unsigned __int128)M1 * c2;
        uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
        uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
        uint64_t n0 = hi1 ^ c1 ^ k0, n1 = lo1, n2 = hi0 ^ c3 ^ k1, n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* READING (top-k draw): one uniform per (row, position, pass), the top 24 bits of the first
 * Philox word, so that the value is exact in fp32 as well. counter = (pos, row, pass, 0),
 * key = (seed, 0). */
double orc_uniform24(uint64_t seed, uint32_t row, uint32_t pos, uint32_t pass)
{
    uint64_t ctr[4] = {pos, row, pass, 0}, key[2] = {seed, 0}, out[4];
    orc_philox4x64_10(ctr, key, out);
    return ldexp((double)(out[0] >> 40), -24);
}

/* ------------------------------------------------------------------------------------------ */
/* Weight formats.
 * [J] appendix A3 (quantize T3) and §3.23 (fused Q/K/V): legacy ggml blocks of 32 consecutive
 * values along the reduction axis K; a Q4_0 row of K=1024 is 32 blocks of 18 bytes.
 * READING (field order, nibble order): Q8_0 block = fp16 scale d, then 32 int8 q; w = d*q.
 * Q4_0 block = fp16 d, then 16 bytes; element j (j<16) is the low nibble of byte j and element
 * j+16 its high nibble; w = (q - 8) * d.
 * [F] §3 (counting the bytes): MLX affine quantization, group 64, ~8.5 bits/weight.
 * READING: q uint8, w = s*q + b with fp16 s and b per group of 64 along K; the matrix blob is
 * planar: q[N][K] bytes, then s[N][K/64] fp16, then b[N][K/64] fp16 (little endian). */
size_t orc_matrix_bytes(int fmt, int N, int K)
{
    if (N <= 0 || K <= 0) return 0;
    switch (fmt) {
    case ORC_Q4_0: return K % 32 ? 0 : (size_t)N * (K / 32) * 18;
    case ORC_Q8_0: return K % 32 ? 0 : (size_t)N * (K / 32) * 34;
    case ORC_AFF8: return K % 64 ? 0 : (size_t)N * K + (size_t)N * (K / 64) * 4;
    case ORC_Q5_0: return K % 32 ? 0 : (size_t)N * (K / 32) * 22;
    case ORC_AFF4_G64: return K % 64 ? 0 : (size_t)N * K / 2 + (size_t)N * (K / 64) * 4;
    case ORC_AFF4_G32: return K % 32 ? 0 : (size_t)N * K / 2 + (size_t)N * (K / 32) * 4;
    default: return 0;
    }
}

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

int orc_dequant_row(int fmt, const uint8_t* blob, int N, int K, int n, double* w)
{
    if (!orc_matrix_bytes(fmt, N, K) || n < 0 || n >= N) return -1;
    if (fmt == ORC_Q8_0) {
        const uint8_t* row = blob + (size_t)n * (K / 32) * 34;
        for (int b = 0; b < K / 32; ++b) {
            const uint8_t* blk = row + (size_t)b * 34;
            double d = orc_half_to_double(rd16(blk));
            for (int j = 0; j < 32; ++j) w[b * 32 + j] = d * (double)(int8_t)blk[2 + j];
        }
    } else if (fmt == ORC_Q4_0) {
        const uint8_t* row = blob + (size_t)n * (K / 32) * 18;
        for (int b = 0; b < K / 32; ++b) {
            const uint8_t* blk = row + (size_t)b * 18;
            double d = orc_half_to_double(rd16(blk));
            for (int j = 0; j < 16; ++j) {
                w[b * 32 + j] = ((double)(blk[2 + j] & 15) - 8.0) * d;
                w[b * 32 + j + 16] = ((double)(blk[2 + j] >> 4) - 8.0) * d;
            }
        }
    } else if (fmt == ORC_Q5_0) {
        /* READING (Q5_0, the GGUF block the journal's --quant q5_0 writes, [J] A3): fp16 d, a
         * 32-bit word of fifth bits (bit j for element j), then the 16 nibble bytes in Q4_0's
         * order; w = (q - 16) d with q = nibble | fifth bit << 4 */
        const uint8_t* row = blob + (size_t)n * (K / 32) * 22;
        for (int b = 0; b < K / 32; ++b) {
            const uint8_t* blk = row + (size_t)b * 22;
            double d = orc_half_to_double(rd16(blk));
            uint32_t qh = (uint32_t)blk[2] | ((uint32_t)blk[3] << 8) | ((uint32_t)blk[4] << 16) | ((uint32_t)blk[5] << 24);
            for (int j = 0; j < 16; ++j) {
                int lo = blk[6 + j] & 15, hi = blk[6 + j] >> 4;
                lo |= (int)((qh >> j) & 1u) << 4;
                hi |= (int)((qh >> (j + 16)) & 1u) << 4;
                w[b * 32 + j] = ((double)lo - 16.0) * d;
                w[b * 32 + j + 16] = ((double)hi - 16.0) * d;
            }
        }
    } else if (fmt == ORC_AFF4_G64 || fmt == ORC_AFF4_G32) {
        /* READING (4-bit affine, the MLX layout [F] §5.8 quantises to, groups of 64 or 32 along
         * K): q packed two per byte, element 2i in the low nibble of byte i and 2i+1 in the high
         * one (the little-endian uint32 words of eight); then fp16 scales, then fp16 biases, one
         * per group; w = s q + b */
        const int G = fmt == ORC_AFF4_G64 ? 64 : 32, ng = K / G;
        const uint8_t* q = blob + (size_t)n * (K / 2);
        const uint8_t* s = blob + (size_t)N * (K / 2) + (size_t)n * ng * 2;
        const uint8_t* bb = blob + (size_t)N * (K / 2) + (size_t)N * ng * 2 + (size_t)n * ng * 2;
        for (int g = 0; g < ng; ++g) {
            double sc = orc_half_to_double(rd16(s + 2 * g)), bi = orc_half_to_double(rd16(bb + 2 * g));
            for (int j = 0; j < G; ++j) {
                int k = g * G + j;
                int v = (k & 1) ? q[k >> 1] >> 4 : q[k >> 1] & 15;
                w[k] = sc * (double)v + bi;
            }
        }
    } else {
        const uint8_t* q = blob + (size_t)n * K;
        const uint8_t* s = blob + (size_t)N * K + (size_t)n * (K / 64) * 2;
        const uint8_t* bb = blob + (size_t)N * K + (size_t)N * (K / 64) * 2 + (size_t)n * (K / 64) * 2;
        for (int g = 0; g < K / 64; ++g) {
            double sc = orc_half_to_double(rd16(s + 2 * g)), bi = orc_half_to_double(rd16(bb + 2 * g));
            for (int j = 0; j < 64; ++j) w[g * 64 + j] = sc * (double)q[g * 64 + j] + bi;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Linear map y_n = sum_k w_nk x_k (+ b_n), fp64, one dequantized row at a time.
 * [J] §3.2 issue 5: weights stored so that each output row is contiguous along K;
 * §3.15/§3.16: the bias (and the residual) are added to the mat-vec result. */
int orc_gemv(int fmt, const uint8_t* blob, int N, int K, const double* x, const double* bias, double* y)
{
    double* w = (double*)malloc(sizeof(double) * (size_t)K);
    if (!w) return -1;
    for (int n = 0; n < N; ++n) {
        if (orc_dequant_row(fmt, blob, N, K, n, w)) { free(w); return -1; }
        double acc = 0.0;
        for (int k = 0; k < K; ++k) acc += w[k] * x[k];
        y[n] = acc + (bias ? bias[n] : 0.0);
    }
    free(w);
    return 0;
}

int orc_gemv_f32(int fmt, const uint8_t* blob, int N, int K, int B, const float* x, const float* bias, double* y)
{
    double* xd = (double*)malloc(sizeof(double) * (size_t)K);
    double* bd = bias ? (double*)malloc(sizeof(double) * (size_t)N) : NULL;
    if (!xd || (bias && !bd)) { free(xd); free(bd); return -1; }
    if (bias) for (int n = 0; n < N; ++n) bd[n] = bias[n];
    int rc = 0;
    for (int r = 0; r < B && !rc; ++r) {
        for (int k = 0; k < K; ++k) xd[k] = x[(size_t)r * K + k];
        rc = orc_gemv(fmt, blob, N, K, xd, bd, y + (size_t)r * N);
    }
    free(xd); free(bd);
    return rc;
}

/* ------------------------------------------------------------------------------------------ */
/* Normalisations.  LayerNorm with gain and bias (GPT-2 blocks, [J] §3.2 mirrors the ggml gpt-2
 * example); RMSNorm with gain only (Llama blocks, [J] §3.19; fused RMS_NORM+MUL in §3.21).
 * READING: eps is a configuration value (1e-5 by default). */
void orc_layernorm(const double* x, int n, const double* g, const double* b, double eps, double* y)
{
    double mu = 0.0, var = 0.0;
    for (int i = 0; i < n; ++i) mu += x[i];
    mu /= n;
    for (int i = 0; i < n; ++i) var += (x[i] - mu) * (x[i] - mu);
    var /= n;
    double inv = 1.0 / sqrt(var + eps);
    for (int i = 0; i < n; ++i) y[i] = (x[i] - mu) * inv * (g ? g[i] : 1.0) + (b ? b[i] : 0.0);
}

void orc_rmsnorm(const double* x, int n, const double* g, double eps, double* y)
{
    double ms = 0.0;
    for (int i = 0; i < n; ++i) ms += x[i] * x[i];
    ms /= n;
    double inv = 1.0 / sqrt(ms + eps);
    for (int i = 0; i < n; ++i) y[i] = x[i] * inv * (g ? g[i] : 1.0);
}

/* [J] §3.4 issue list: ggml's gelu is the tanh approximation (Hendrycks & Gimpel),
 * 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))); READING: T3 uses it (it mirrors ggml's
 * gpt-2 example, §3.2). */
double orc_gelu_tanh(double x)
{
    const double c = sqrt(2.0 / 3.14159265358979323846);
    return 0.5 * x * (1.0 + tanh(c * (x + 0.044715 * x * x * x)));
}

/* [J] §3.21 (SwiGLU kernel): silu(gate) * up, silu(g) = g / (1 + e^-g). */
double orc_silu(double x) { return x / (1.0 + exp(-x)); }

/* Rotary embedding, NEOX half-split convention ([J] §3.19 "RoPE (NEOX half-split)", and the
 * same convention in the S3Tokenizer port).  READING: plain RoPE, theta0 = 10000, no Llama-3
 * frequency scaling; pos is the absolute 0-based position.
 * For i < hd/2: t = pos * theta0^(-2i/hd); (a, b) = (v_i, v_{i+hd/2}) ->
 * (a cos t - b sin t, a sin t + b cos t). */
void orc_rope_neox(double* v, int hd, int pos, double theta)
{
    int h = hd / 2;
    for (int i = 0; i < h; ++i) {
        double t = (double)pos * pow(theta, -2.0 * (double)i / (double)hd);
        double a = v[i], b = v[i + h];
        v[i] = a * cos(t) - b * sin(t);
        v[i + h] = a * sin(t) + b * cos(t);
    }
}

/* max-subtracted softmax */
void orc_softmax(const double* s, int n, double* a)
{
    double m = -INFINITY, sum = 0.0;
    for (int i = 0; i < n; ++i) if (s[i] > m) m = s[i];
    for (int i = 0; i < n; ++i) { a[i] = exp(s[i] - m); sum += a[i]; }
    for (int i = 0; i < n; ++i) a[i] /= sum;
}

/* Attention of one query head over the cached keys, softmax(q K^T / sqrt(hd)) V
 * ([J] §3.8 attempt on flash attention; §3.13: at a single new token every cached position is
 * in the past, so no mask).  Keys/values are the fp16 rows of the cache. */
void orc_attend(const double* q, const uint16_t* kc, const uint16_t* vc, int n_keys, int hd, double* o)
{
    for (int i = 0; i < hd; ++i) o[i] = 0.0;
    if (n_keys <= 0) return;
    double* s = (double*)malloc(sizeof(double) * (size_t)n_keys);
    double* a = (double*)malloc(sizeof(double) * (size_t)n_keys);
    double scale = 1.0 / sqrt((double)hd);
    for (int j = 0; j < n_keys; ++j) {
        double dot = 0.0;
        for (int i = 0; i < hd; ++i) dot += q[i] * orc_half_to_double(kc[(size_t)j * hd + i]);
        s[j] = dot * scale;
    }
    orc_softmax(s, n_keys, a);
    for (int j = 0; j < n_keys; ++j)
        for (int i = 0; i < hd; ++i) o[i] += a[j] * orc_half_to_double(vc[(size_t)j * hd + i]);
    free(s); free(a);
}

/* READING (greedy tie-break): the lowest index among equal maxima. */
int orc_argmax(const double* v, int n)
{
    int best = 0;
    for (int i = 1; i < n; ++i) if (v[i] > v[best]) best = i;
    return best;
}

/* [J] §3.2 sampler order (temperature, then top-k); READING for the draw: keep the k largest
 * of logits/T (ties by lower index), softmax over them, and return the first index, in
 * descending order, whose cumulative unnormalised mass exceeds u times the total. */
int orc_sample_topk(const double* logits, int n, int k, double temperature, double u)
{
    if (n <= 0) return -1;
    if (k <= 0 || k > n) k = n;
    int* idx = (int*)malloc(sizeof(int) * (size_t)k);
    double* z = (double*)malloc(sizeof(double) * (size_t)k);
    char* taken = (char*)calloc((size_t)n, 1);
    for (int r = 0; r < k; ++r) {              /* selection, one maximum at a time */
        int best = -1;
        for (int i = 0; i < n; ++i)
            if (!taken[i] && (best < 0 || logits[i] > logits[best])) best = i;
        taken[best] = 1; idx[r] = best; z[r] = logits[best] / temperature;
    }
    double total = 0.0;
    for (int r = 0; r < k; ++r) { z[r] = exp(z[r] - logits[idx[0]] / temperature); total += z[r]; }
    double thr = u * total, c = 0.0;
    int pick = idx[k - 1];
    for (int r = 0; r < k; ++r) { c += z[r]; if (c > thr) { pick = idx[r]; break; } }
    free(idx); free(z); free(taken);
    return pick;
}

/* ------------------------------------------------------------------------------------------ */
/* The sampler chain, as processors on a full-vocabulary vector v[n] in which a removed entry is
 * -inf.  Two orders appear on the pages:
 *   [J] §3.2 (the T3 port, mirroring HF's processor list): temperature, top-k, top-p, then the
 *       repetition penalty;
 *   [J] §3.19 (the multilingual T3): repetition penalty, temperature, min-p, top-p, top-k, then
 *       the draw.
 * The repetition penalty ([J] §3.2 issue 7) divides a positive logit by theta and multiplies a
 * negative one, for every token id present in the history (once per id, however often it
 * occurs).  top-p keeps, in descending order, every entry whose preceding mass is below p
 * (HF's warper removes an entry whose ascending cumulative mass is <= 1 - p, which is the same
 * set); min-p keeps the entries whose probability is at least min_p times the largest.
 * READING (order of the draw): the survivors are walked in descending order of their final
 * values (ties by lower index), as in orc_sample_topk.  READING (greedy with a penalty): the
 * argmax of the penalized logits (HF applies processors, not warpers, when not sampling). */

typedef struct { double v; int i; } orc_vi;
static int cmp_desc(const void* a, const void* b)
{
    const orc_vi *x = (const orc_vi*)a, *y = (const orc_vi*)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return x->i < y->i ? -1 : (x->i > y->i);
}

/* the finite entries of v in descending order (ties by lower index); returns their count */
static int rank_desc(const double* v, int n, orc_vi* out)
{
    int m = 0;
    for (int i = 0; i < n; ++i) if (isfinite(v[i])) { out[m].v = v[i]; out[m].i = i; ++m; }
    qsort(out, (size_t)m, sizeof(orc_vi), cmp_desc);
    return m;
}

/* probabilities of the finite entries (softmax, max-subtracted); removed entries get 0 */
static void probs_of(const double* v, int n, double* p)
{
    double mx = -INFINITY, z = 0.0;
    for (int i = 0; i < n; ++i) if (v[i] > mx) mx = v[i];
    for (int i = 0; i < n; ++i) { p[i] = isfinite(v[i]) ? exp(v[i] - mx) : 0.0; z += p[i]; }
    for (int i = 0; i < n; ++i) p[i] /= z;
}

static void proc_penalty(double* v, int n, const char* seen, double theta)
{
    for (int i = 0; i < n; ++i)
        if (seen[i] && isfinite(v[i])) v[i] = v[i] < 0.0 ? v[i] * theta : v[i] / theta;
}

static void proc_temperature(double* v, int n, double T)
{
    for (int i = 0; i < n; ++i) v[i] /= T;
}

/* keep the k largest (ties by lower index); gap = distance between the k-th and (k+1)-th */
static void proc_top_k(double* v, int n, int k, orc_vi* r, double* gap)
{
    int m = rank_desc(v, n, r);
    if (k >= m) return;
    double g = r[k - 1].v - r[k].v;
    if (g < *gap) *gap = g;
    for (int j = k; j < m; ++j) v[r[j].i] = -INFINITY;
}

static void proc_top_p(double* v, int n, double top_p, orc_vi* r, double* p, double* margin)
{
    int m = rank_desc(v, n, r);
    probs_of(v, n, p);
    double before = 0.0;
    for (int j = 0; j < m; ++j) {
        double dist = fabs(before - top_p);
        if (j > 0 && dist < *margin) *margin = dist;
        if (before >= top_p) v[r[j].i] = -INFINITY;
        before += p[r[j].i];
    }
}

static void proc_min_p(double* v, int n, double min_p, double* p, double* margin)
{
    probs_of(v, n, p);
    double pmax = 0.0;
    for (int i = 0; i < n; ++i) if (p[i] > pmax) pmax = p[i];
    for (int i = 0; i < n; ++i) {
        if (!isfinite(v[i])) continue;
        double dist = fabs(p[i] / pmax - min_p);
        if (dist < *margin) *margin = dist;
        if (p[i] < min_p * pmax) v[i] = -INFINITY;
    }
}

/* margins (optional, 6 values): [0] distance of u from the nearest cumulative boundary of the
 * draw, relative to the total mass; [1] top-p: smallest |preceding mass - p|; [2] min-p:
 * smallest |p_i / p_max - min_p|; [3] top-k: gap between the k-th and (k+1)-th value at that
 * stage; [4] greedy: gap between the two largest penalized logits; [5] order: gap between the
 * drawn entry's final value and its neighbours' in the walk (two nearly equal values may be
 * walked in the other order by a computation that rounds differently, which moves the
 * crossing to the other id).  Unused ones are +inf. */
int orc_sample_chain(const double* logits, int n, const orc_sampling* s, const int32_t* hist, int n_hist,
                     double u, double* margins)
{
    if (n <= 0) return -1;
    double mg[6] = {INFINITY, INFINITY, INFINITY, INFINITY, INFINITY, INFINITY};
    double* v = (double*)malloc(sizeof(double) * (size_t)n);
    double* p = (double*)malloc(sizeof(double) * (size_t)n);
    char* seen = (char*)calloc((size_t)n, 1);
    orc_vi* r = (orc_vi*)malloc(sizeof(orc_vi) * (size_t)n);
    memcpy(v, logits, sizeof(double) * (size_t)n);
    for (int j = 0; j < n_hist; ++j) if (hist[j] >= 0 && hist[j] < n) seen[hist[j]] = 1;
    int pen = s->rep_penalty > 0.0 && s->rep_penalty != 1.0;
    int k = (s->top_k <= 0 || s->top_k > n) ? n : s->top_k;
    int use_p = s->top_p > 0.0 && s->top_p < 1.0, use_min = s->min_p > 0.0;
    int pick;
    if (s->mode == 0) {
        if (pen) proc_penalty(v, n, seen, s->rep_penalty);
        int m = rank_desc(v, n, r);
        pick = r[0].i;
        if (m > 1) mg[4] = r[0].v - r[1].v;
    } else {
        if (s->order == ORC_ORDER_MTL) {
            if (pen) proc_penalty(v, n, seen, s->rep_penalty);
            proc_temperature(v, n, s->temperature);
            if (use_min) proc_min_p(v, n, s->min_p, p, &mg[2]);
            if (use_p) proc_top_p(v, n, s->top_p, r, p, &mg[1]);
            proc_top_k(v, n, k, r, &mg[3]);
        } else {
            proc_temperature(v, n, s->temperature);
            proc_top_k(v, n, k, r, &mg[3]);
            if (use_p) proc_top_p(v, n, s->top_p, r, p, &mg[1]);
            if (pen) proc_penalty(v, n, seen, s->rep_penalty);
        }
        /* the draw: softmax over the survivors, walked in descending order */
        int m = rank_desc(v, n, r);
        double total = 0.0;
        for (int j = 0; j < m; ++j) total += exp(r[j].v - r[0].v);
        double thr = u * total, c = 0.0;
        pick = r[m - 1].i;
        int found = 0;
        int at = m - 1;
        for (int j = 0; j < m; ++j) {
            c += exp(r[j].v - r[0].v);
            double dist = fabs(c - thr) / total;
            if (dist < mg[0]) mg[0] = dist;
            if (!found && c > thr) { pick = r[j].i; at = j; found = 1; }
        }
        if (at > 0 && r[at - 1].v - r[at].v < mg[5]) mg[5] = r[at - 1].v - r[at].v;
        if (at + 1 < m && r[at].v - r[at + 1].v < mg[5]) mg[5] = r[at].v - r[at + 1].v;
    }
    if (margins) memcpy(margins, mg, sizeof(mg));
    free(v); free(p); free(seen); free(r);
    return pick;
}

/* ------------------------------------------------------------------------------------------ */
/* Models.
 * GPT-2-Medium-shaped T3 ([J] §3.2; appendix A3 lists the quantized linears c_attn, c_proj,
 * c_fc, mlp.c_proj and speech_head; biases, norms and embeddings stay fp32).
 * Llama-shaped T3 ([J] §3.19: RMSNorm, SwiGLU, separate Q/K/V without bias, RoPE).
 * Talker + code predictor ([F] §1 frame loop and §3 byte count: 28-layer Talker, 16 query / 8
 * KV heads of 128, 5-layer predictor of the same width running 15 passes; the sum of the
 * sixteen code embeddings is the next Talker input).
 *
 * Canonical weight order (all fp32 except the quantized matrices):
 *   GPT2 : wte[V][d], wpe[n_ctx][d], per layer {ln1_g, ln1_b, qkv_w[3d][d], qkv_b[3d],
 *          o_w[d][d], o_b[d], ln2_g, ln2_b, fc_w[ff][d], fc_b[ff], down_w[d][ff], down_b[d]},
 *          lnf_g, lnf_b, head_w[V][d]
 *   LLAMA: emb[V][d], per layer {rms1_g, q_w[H*hd][d], k_w[Hkv*hd][d], v_w[Hkv*hd][d],
 *          o_w[d][H*hd], rms2_g, gate_w[ff][d], up_w[ff][d], down_w[d][ff]}, rmsf_g, head_w[V][d]
 *   TALKER_CP: E_0[V][d], E_1..E_{C-1}[Vcp][d], Talker layers (as LLAMA), talker rmsf_g,
 *          talker head_w[V][d], predictor layers (as LLAMA), predictor rmsf_g,
 *          predictor heads 1..C-1 [Vcp][d]
 * READING (head): untied, no bias.  READING (code predictor): pass 1 consumes two positions,
 * the Talker's final-normed hidden state and E_0(c_0); pass j>1 consumes E_{j-1}(c_{j-1}); its
 * positions restart at 0 every frame; it has its own final RMSNorm and one head per codebook.
 */
#define LLAMA_PER_LAYER 9
#define GPT2_PER_LAYER 12

typedef struct {
    const double *n1g, *n1b, *n2g, *n2b;   /* norms (b NULL for RMS) */
    const uint8_t *wqkv, *wq, *wk, *wv, *wo, *wfc, *wgate, *wup, *wdown;
    const double *bqkv, *bo, *bfc, *bdown;
} orc_layer;

struct orc_model {
    orc_config c;
    int n_in;            /* tokens per position */
    void** own;          /* owned copies of all weights */
    int n_own;
    const double* emb[16];       /* embedding tables */
    const double* wpe;
    orc_layer* L;                /* main layers */
    orc_layer* Lc;               /* predictor layers */
    const double *nfg, *nfb, *cp_nfg;
    const uint8_t* head;
    const uint8_t* cp_head[16];
    uint16_t *kc, *vc;           /* [L][B][Hkv][n_ctx][hd] */
    uint16_t *ckc, *cvc;         /* predictor cache [Lc][B][Hkv][C][hd] */
    int n_past;
    int vmax;
    double* logits;              /* [B][C or 1][vmax] */
    int32_t* last;               /* [B][C or 1] last sampled */
    int32_t* seq;                /* [n_ctx][B] token consumed at each position (code 0 for
                                    TALKER_CP): the repetition penalty's history; -1 = unknown */
};

int orc_n_weights(const orc_config* c)
{
    switch (c->arch) {
    case ORC_GPT2: return 2 + GPT2_PER_LAYER * c->n_layer + 3;
    case ORC_LLAMA: return 1 + LLAMA_PER_LAYER * c->n_layer + 2;
    case ORC_TALKER_CP:
        return c->n_codebooks + LLAMA_PER_LAYER * c->n_layer + 2 + LLAMA_PER_LAYER * c->cp_n_layer + 1 +
               (c->n_codebooks - 1);
    default: return -1;
    }
}

/* expected byte size of every canonical tensor; fills kinds (0 fp32 vector/table, 1 matrix) */
static int expected_sizes(const orc_config* c, size_t* sz)
{
    int d = c->d_model, H = c->n_head, Hk = c->n_kv_head, hd = c->head_dim, ff = c->d_ff;
    int f = c->wfmt, i = 0;
#define F32(n) (sz[i++] = (size_t)(n) * 4)
#define MAT(N, K) (sz[i++] = orc_matrix_bytes(f, (N), (K)))
    if (c->arch == ORC_GPT2) {
        F32((size_t)c->vocab * d); F32((size_t)c->n_ctx * d);
        for (int l = 0; l < c->n_layer; ++l) {
            F32(d); F32(d); MAT(3 * d, d); F32(3 * d); MAT(d, d); F32(d);
            F32(d); F32(d); MAT(ff, d); F32(ff); MAT(d, ff); F32(d);
        }
        F32(d); F32(d); MAT(c->vocab, d);
    } else {
        int nl = c->n_layer;
        if (c->arch == ORC_LLAMA) F32((size_t)c->vocab * d);
        else {
            F32((size_t)c->vocab * d);
            for (int k = 1; k < c->n_codebooks; ++k) F32((size_t)c->cp_vocab * d);
        }
        for (int pass = 0; pass < (c->arch == ORC_TALKER_CP ? 2 : 1); ++pass) {
            int n = pass == 0 ? nl : c->cp_n_layer;
            for (int l = 0; l < n; ++l) {
                F32(d); MAT(H * hd, d); MAT(Hk * hd, d); MAT(Hk * hd, d); MAT(d, H * hd);
                F32(d); MAT(ff, d); MAT(ff, d); MAT(d, ff);
            }
            F32(d);
            if (pass == 0) MAT(c->vocab, d);
            else for (int k = 1; k < c->n_codebooks; ++k) MAT(c->cp_vocab, d);
        }
    }
#undef F32
#undef MAT
    return i;
}

void orc_model_destroy(orc_model* m)
{
    if (!m) return;
    for (int i = 0; i < m->n_own; ++i) free(m->own[i]);
    free(m->own); free(m->L); free(m->Lc); free(m->kc); free(m->vc); free(m->ckc); free(m->cvc);
    free(m->logits); free(m->last); free(m->seq); free(m);
}

static size_t cache_elems(const orc_config* c)
{
    return (size_t)c->n_layer * c->batch * c->n_kv_head * c->n_ctx * c->head_dim;
}

/* replace the owned fp32 copy of tensor idx by an fp64 copy */
static void widen(orc_model* m, int idx, size_t len)
{
    const float* src = (const float*)m->own[idx];
    double* dst = (double*)malloc(sizeof(double) * len);
    for (size_t t = 0; t < len; ++t) dst[t] = src[t];
    free(m->own[idx]);
    m->own[idx] = dst;
}

orc_model* orc_model_create(const orc_config* c, const void* const* w, const size_t* sizes, int n)
{
    g_err[0] = 0;
    int nw = orc_n_weights(c);
    if (nw < 0) { set_err("unknown arch"); return NULL; }
    if (c->n_layer <= 0 || c->d_model <= 0 || c->n_head <= 0 || c->n_kv_head <= 0 || c->head_dim <= 0 ||
        c->d_ff <= 0 || c->vocab <= 0 || c->n_ctx <= 0 || c->batch <= 0 || c->n_head % c->n_kv_head ||
        (c->cfg && (c->batch != 2 || c->arch == ORC_TALKER_CP)) ||
        c->head_dim % 2) { set_err("bad dimensions"); return NULL; }
    if (c->arch == ORC_GPT2 && (c->n_head * c->head_dim != c->d_model || c->n_kv_head != c->n_head)) {
        set_err("GPT2 needs n_head*head_dim == d_model and n_kv_head == n_head"); return NULL;
    }
    if (c->arch == ORC_TALKER_CP && (c->n_codebooks < 2 || c->n_codebooks > 16 || c->cp_n_layer <= 0 ||
                                     c->cp_vocab <= 0)) { set_err("bad code-predictor dims"); return NULL; }
    if (n != nw) { set_err("wrong number of weights"); return NULL; }
    size_t* exp_sz = (size_t*)calloc((size_t)nw, sizeof(size_t));
    expected_sizes(c, exp_sz);
    for (int i = 0; i < nw; ++i)
        if (!exp_sz[i] || sizes[i] != exp_sz[i] || !w[i]) {
            snprintf(g_err, sizeof g_err, "weight %d: %zu bytes, expected %zu", i, sizes[i], exp_sz[i]);
            free(exp_sz); return NULL;
        }
    orc_model* m = (orc_model*)calloc(1, sizeof *m);
    m->c = *c;
    m->n_in = c->arch == ORC_TALKER_CP ? c->n_codebooks : 1;
    m->own = (void**)calloc((size_t)nw, sizeof(void*));
    m->n_own = nw;
    for (int i = 0; i < nw; ++i) {
        m->own[i] = malloc(sizes[i]);
        memcpy(m->own[i], w[i], sizes[i]);
    }
    free(exp_sz);
    /* fp32 tensors are widened to fp64 once */
    int i = 0;
    const int d = c->d_model;
    m->L = (orc_layer*)calloc((size_t)c->n_layer, sizeof(orc_layer));
    {
        #define WIDEN(idx, len) widen(m, (idx), (size_t)(len))
        if (c->arch == ORC_GPT2) {
            WIDEN(0, (size_t)c->vocab * d); m->emb[0] = (double*)m->own[0];
            WIDEN(1, (size_t)c->n_ctx * d); m->wpe = (double*)m->own[1];
            i = 2;
            for (int l = 0; l < c->n_layer; ++l) {
                orc_layer* L = &m->L[l];
                WIDEN(i, d); L->n1g = (double*)m->own[i++];
                WIDEN(i, d); L->n1b = (double*)m->own[i++];
                L->wqkv = (uint8_t*)m->own[i++];
                WIDEN(i, 3 * d); L->bqkv = (double*)m->own[i++];
                L->wo = (uint8_t*)m->own[i++];
                WIDEN(i, d); L->bo = (double*)m->own[i++];
                WIDEN(i, d); L->n2g = (double*)m->own[i++];
                WIDEN(i, d); L->n2b = (double*)m->own[i++];
                L->wfc = (uint8_t*)m->own[i++];
                WIDEN(i, c->d_ff); L->bfc = (double*)m->own[i++];
                L->wdown = (uint8_t*)m->own[i++];
                WIDEN(i, d); L->bdown = (double*)m->own[i++];
            }
            WIDEN(i, d); m->nfg = (double*)m->own[i++];
            WIDEN(i, d); m->nfb = (double*)m->own[i++];
            m->head = (uint8_t*)m->own[i++];
        } else {
            WIDEN(0, (size_t)c->vocab * d); m->emb[0] = (double*)m->own[0];
            i = 1;
            if (c->arch == ORC_TALKER_CP)
                for (int k = 1; k < c->n_codebooks; ++k) { WIDEN(i, (size_t)c->cp_vocab * d); m->emb[k] = (double*)m->own[i++]; }
            int passes = c->arch == ORC_TALKER_CP ? 2 : 1;
            if (passes == 2) m->Lc = (orc_layer*)calloc((size_t)c->cp_n_layer, sizeof(orc_layer));
            for (int p = 0; p < passes; ++p) {
                int nl = p == 0 ? c->n_layer : c->cp_n_layer;
                orc_layer* LL = p == 0 ? m->L : m->Lc;
                for (int l = 0; l < nl; ++l) {
                    orc_layer* L = &LL[l];
                    WIDEN(i, d); L->n1g = (double*)m->own[i++];
                    L->wq = (uint8_t*)m->own[i++];
                    L->wk = (uint8_t*)m->own[i++];
                    L->wv = (uint8_t*)m->own[i++];
                    L->wo = (uint8_t*)m->own[i++];
                    WIDEN(i, d); L->n2g = (double*)m->own[i++];
                    L->wgate = (uint8_t*)m->own[i++];
                    L->wup = (uint8_t*)m->own[i++];
                    L->wdown = (uint8_t*)m->own[i++];
                }
                if (p == 0) {
                    WIDEN(i, d); m->nfg = (double*)m->own[i++];
                    m->head = (uint8_t*)m->own[i++];
                } else {
                    WIDEN(i, d); m->cp_nfg = (double*)m->own[i++];
                    for (int k = 1; k < c->n_codebooks; ++k) m->cp_head[k] = (uint8_t*)m->own[i++];
                }
            }
        }
        #undef WIDEN
    }
    m->kc = (uint16_t*)calloc(cache_elems(c), 2);
    m->vc = (uint16_t*)calloc(cache_elems(c), 2);
    if (c->arch == ORC_TALKER_CP) {
        size_t ce = (size_t)c->cp_n_layer * c->batch * c->n_kv_head * c->n_codebooks * c->head_dim;
        m->ckc = (uint16_t*)calloc(ce, 2);
        m->cvc = (uint16_t*)calloc(ce, 2);
    }
    m->vmax = c->vocab;
    if (c->arch == ORC_TALKER_CP && c->cp_vocab > m->vmax) m->vmax = c->cp_vocab;
    m->logits = (double*)calloc((size_t)c->batch * m->n_in * m->vmax, sizeof(double));
    m->last = (int32_t*)calloc((size_t)c->batch * m->n_in, sizeof(int32_t));
    m->seq = (int32_t*)malloc(sizeof(int32_t) * (size_t)c->n_ctx * c->batch);
    for (size_t i = 0; i < (size_t)c->n_ctx * c->batch; ++i) m->seq[i] = -1;
    if (!m->kc || !m->vc || !m->logits || !m->last) { set_err("out of memory"); orc_model_destroy(m); return NULL; }
    return m;
}

void orc_reset(orc_model* m) { m->n_past = 0; }
int orc_n_past(const orc_model* m) { return m->n_past; }
int orc_truncate(orc_model* m, int n_past)
{
    if (n_past < 0 || n_past > m->n_past) { set_err("truncate beyond n_past"); return -1; }
    m->n_past = n_past;
    return 0;
}

/* cache row pointer: [layer][row][kv_head][pos][hd] */
static uint16_t* cache_at(uint16_t* base, const orc_config* c, int nctx, int l, int b, int g, int pos)
{
    return base + ((((size_t)l * c->batch + b) * c->n_kv_head + g) * nctx + pos) * c->head_dim;
}

/* One decoder layer for one row at position pos, in place on x[d]. kc/vc/nctx select the main
 * or the predictor cache.  Attention reads positions 0..pos of that cache. */
static void layer_forward(const orc_model* m, const orc_layer* L, int l, int b, double* x, int pos,
                          uint16_t* kc, uint16_t* vc, int nctx)
{
    const orc_config* c = &m->c;
    int d = c->d_model, H = c->n_head, Hk = c->n_kv_head, hd = c->head_dim, ff = c->d_ff, f = c->wfmt;
    int qd = H * hd, kd = Hk * hd;
    double* nrm = (double*)malloc(sizeof(double) * (size_t)d);
    double* q = (double*)malloc(sizeof(double) * (size_t)qd);
    double* k = (double*)malloc(sizeof(double) * (size_t)kd);
    double* v = (double*)malloc(sizeof(double) * (size_t)kd);
    double* o = (double*)malloc(sizeof(double) * (size_t)qd);
    double* t = (double*)malloc(sizeof(double) * (size_t)(ff > d ? ff : d));
    double* g = (double*)malloc(sizeof(double) * (size_t)ff);
    double* u = (double*)malloc(sizeof(double) * (size_t)ff);
    int gpt2 = c->arch == ORC_GPT2;

    if (gpt2) {
        double* qkv = (double*)malloc(sizeof(double) * 3 * (size_t)d);
        orc_layernorm(x, d, L->n1g, L->n1b, c->norm_eps, nrm);
        orc_gemv(f, L->wqkv, 3 * d, d, nrm, L->bqkv, qkv);     /* fused QKV, [J] §3.14 offsets */
        memcpy(q, qkv, sizeof(double) * d);
        memcpy(k, qkv + d, sizeof(double) * d);
        memcpy(v, qkv + 2 * d, sizeof(double) * d);
        free(qkv);
    } else {
        orc_rmsnorm(x, d, L->n1g, c->norm_eps, nrm);
        orc_gemv(f, L->wq, qd, d, nrm, NULL, q);
        orc_gemv(f, L->wk, kd, d, nrm, NULL, k);
        orc_gemv(f, L->wv, kd, d, nrm, NULL, v);
        for (int h = 0; h < H; ++h) orc_rope_neox(q + h * hd, hd, pos, c->rope_theta);
        for (int h = 0; h < Hk; ++h) orc_rope_neox(k + h * hd, hd, pos, c->rope_theta);
    }
    /* KV append in fp16 at position pos ([J] §3.13: the cache is laid out the way attention
     * reads it, head-dim fastest, then position, then head) */
    for (int h = 0; h < Hk; ++h) {
        uint16_t* kr = cache_at(kc, c, nctx, l, b, h, pos);
        uint16_t* vr = cache_at(vc, c, nctx, l, b, h, pos);
        for (int i = 0; i < hd; ++i) { kr[i] = orc_double_to_half(k[h * hd + i]); vr[i] = orc_double_to_half(v[h * hd + i]); }
    }
    int grp = H / Hk;
    for (int h = 0; h < H; ++h)
        orc_attend(q + h * hd, cache_at(kc, c, nctx, l, b, h / grp, 0), cache_at(vc, c, nctx, l, b, h / grp, 0),
                   pos + 1, hd, o + h * hd);
    orc_gemv(f, L->wo, d, qd, o, gpt2 ? L->bo : NULL, t);
    for (int i = 0; i < d; ++i) x[i] += t[i];                   /* residual, [J] §3.16 */

    if (gpt2) {
        orc_layernorm(x, d, L->n2g, L->n2b, c->norm_eps, nrm);
        orc_gemv(f, L->wfc, ff, d, nrm, L->bfc, g);
        for (int i = 0; i < ff; ++i) g[i] = orc_gelu_tanh(g[i]);
        orc_gemv(f, L->wdown, d, ff, g, L->bdown, t);
    } else {
        orc_rmsnorm(x, d, L->n2g, c->norm_eps, nrm);
        orc_gemv(f, L->wgate, ff, d, nrm, NULL, g);
        orc_gemv(f, L->wup, ff, d, nrm, NULL, u);
        for (int i = 0; i < ff; ++i) g[i] = orc_silu(g[i]) * u[i];
        orc_gemv(f, L->wdown, d, ff, g, NULL, t);
    }
    for (int i = 0; i < d; ++i) x[i] += t[i];
    free(nrm); free(q); free(k); free(v); free(o); free(t); free(g); free(u);
}

static void final_norm(const orc_model* m, const double* x, const double* g, const double* b, double* y)
{
    if (m->c.arch == ORC_GPT2) orc_layernorm(x, m->c.d_model, g, b, m->c.norm_eps, y);
    else orc_rmsnorm(x, m->c.d_model, g, m->c.norm_eps, y);
}

/* READING (which heads the penalty covers): the main head (GPT2/LLAMA token, Talker code 0),
 * over the tokens the row consumed at positions 0..pos; the code predictor's heads use the rest
 * of the chain without it. */
static int pick(const orc_model* m, const double* logits, int n, int row, int pos, int pass)
{
    const orc_config* c = &m->c;
    orc_sampling s = {c->sample_mode, c->top_k, c->temperature, c->top_p, c->min_p, c->rep_penalty, c->sample_order};
    if (pass > 0) s.rep_penalty = 1.0;
    int pen = s.rep_penalty > 0.0 && s.rep_penalty != 1.0;
    if (s.mode == 0 && !pen) return orc_argmax(logits, n);
    int32_t* hist = (int32_t*)malloc(sizeof(int32_t) * (size_t)(pos + 1));
    for (int p = 0; p <= pos; ++p) hist[p] = m->seq[(size_t)p * c->batch + row];
    int id = orc_sample_chain(logits, n, &s, hist, pen ? pos + 1 : 0,
                              orc_uniform24(c->seed, (uint32_t)row, (uint32_t)pos, (uint32_t)pass), NULL);
    free(hist);
    return id;
}

/* the input embedding of one position */
static int embed(const orc_model* m, const int32_t* tok, int pos, double* x)
{
    const orc_config* c = &m->c;
    int d = c->d_model;
    if (c->arch == ORC_TALKER_CP) {
        for (int i = 0; i < d; ++i) x[i] = 0.0;
        for (int cb = 0; cb < c->n_codebooks; ++cb) {       /* [F] §1: sum of the 16 code embeddings */
            int lim = cb == 0 ? c->vocab : c->cp_vocab;
            if (tok[cb] < 0 || tok[cb] >= lim) return -1;
            const double* e = m->emb[cb] + (size_t)tok[cb] * d;
            for (int i = 0; i < d; ++i) x[i] += e[i];
        }
        return 0;
    }
    if (tok[0] < 0 || tok[0] >= c->vocab) return -1;
    const double* e = m->emb[0] + (size_t)tok[0] * d;
    for (int i = 0; i < d; ++i) x[i] = e[i];
    if (c->arch == ORC_GPT2) for (int i = 0; i < d; ++i) x[i] += m->wpe[(size_t)pos * d + i];  /* learned positions */
    return 0;
}

/* one position for every row; with_head = 0 skips the head and sampling (prefill positions
 * whose logits nobody reads) */
static int forward_position(orc_model* m, const int32_t* tok_in, int32_t* tok_out, int with_head)
{
    const orc_config* c = &m->c;
    int d = c->d_model, pos = m->n_past, C = m->n_in;
    if (pos >= c->n_ctx) { set_err("context full"); return -1; }
    double* x = (double*)malloc(sizeof(double) * (size_t)d);
    double* h = (double*)malloc(sizeof(double) * (size_t)d);
    double* lg = (double*)malloc(sizeof(double) * (size_t)m->vmax);
    /* validate every token before touching state */
    for (int b = 0; b < c->batch; ++b)
        if (embed(m, tok_in + (size_t)b * C, pos, x)) { set_err("token out of range"); free(x); free(h); free(lg); return -1; }
    for (int b = 0; b < c->batch; ++b) m->seq[(size_t)pos * c->batch + b] = tok_in[(size_t)b * C];
    for (int b = 0; b < c->batch; ++b) {
        embed(m, tok_in + (size_t)b * C, pos, x);
        for (int l = 0; l < c->n_layer; ++l) layer_forward(m, &m->L[l], l, b, x, pos, m->kc, m->vc, c->n_ctx);
        if (!with_head) continue;
        final_norm(m, x, m->nfg, m->nfb, h);
        orc_gemv(c->wfmt, m->head, c->vocab, d, h, NULL, lg);
        double* dst = m->logits + (size_t)b * C * m->vmax;
        memcpy(dst, lg, sizeof(double) * c->vocab);
        if (c->cfg) continue;                   /* guided: one pick after both rows, below */
        int c0 = pick(m, lg, c->vocab, b, pos, 0);
        m->last[(size_t)b * C] = c0;
        if (c->arch != ORC_TALKER_CP) continue;
        /* code-predictor frame: 15 sequential passes, its own cache restarted every frame */
        int cpos = 0, prev = c0;
        for (int j = 1; j < C; ++j) {
            if (j == 1) {
                memcpy(x, h, sizeof(double) * d);                  /* Talker final-normed hidden */
                for (int l = 0; l < c->cp_n_layer; ++l)
                    layer_forward(m, &m->Lc[l], l, b, x, cpos, m->ckc, m->cvc, C);
                ++cpos;
            }
            const double* e = m->emb[j - 1] + (size_t)prev * d;   /* E_{j-1}(c_{j-1}) */
            memcpy(x, e, sizeof(double) * d);
            for (int l = 0; l < c->cp_n_layer; ++l) layer_forward(m, &m->Lc[l], l, b, x, cpos, m->ckc, m->cvc, C);
            ++cpos;
            orc_rmsnorm(x, d, m->cp_nfg, c->norm_eps, h);
            orc_gemv(c->wfmt, m->cp_head[j], c->cp_vocab, d, h, NULL, lg);
            memcpy(dst + (size_t)j * m->vmax, lg, sizeof(double) * c->cp_vocab);
            prev = pick(m, lg, c->cp_vocab, b, pos, j);
            m->last[(size_t)b * C + j] = prev;
        }
    }
    if (c->cfg && with_head) {
        /* READING (classifier-free guidance, [J] §3.19: cond and uncond forwards combined at the
         * logits before the rest of the chain): l = l_cond + w (l_cond - l_uncond), row 0 the
         * conditioned one; the pick uses row 0's counter and history and both rows take it */
        const double* l0 = m->logits;
        const double* l1 = m->logits + (size_t)C * m->vmax;
        for (int i = 0; i < c->vocab; ++i) lg[i] = l0[i] + c->cfg_weight * (l0[i] - l1[i]);
        int id = pick(m, lg, c->vocab, 0, pos, 0);
        m->last[0] = id;
        m->last[C] = id;
    }
    free(x); free(h); free(lg);
    m->n_past = pos + 1;
    if (tok_out && with_head) memcpy(tok_out, m->last, sizeof(int32_t) * (size_t)c->batch * C);
    return 0;
}

int orc_step(orc_model* m, const int32_t* tok_in, int32_t* tok_out)
{
    return forward_position(m, tok_in ? tok_in : m->last, tok_out, 1);
}

/* Prefill: the decode step at every prompt position (exact prefill/decode consistency).  Only
 * the last position's head and sampler are evaluated; the cached K/V do not depend on them.
 * tokens are [batch][n][tokens per position]. */
int orc_prefill(orc_model* m, const int32_t* toks, int n, int32_t* tok_out)
{
    const orc_config* c = &m->c;
    if (n <= 0 || m->n_past + n > c->n_ctx) { set_err("context full"); return -1; }
    int C = m->n_in;
    int32_t* buf = (int32_t*)malloc(sizeof(int32_t) * (size_t)c->batch * C);
    for (int t = 0; t < n; ++t) {
        for (int b = 0; b < c->batch; ++b)
            memcpy(buf + (size_t)b * C, toks + ((size_t)b * n + t) * C, sizeof(int32_t) * C);
        if (forward_position(m, buf, tok_out, t == n - 1)) { free(buf); return -1; }
    }
    free(buf);
    return 0;
}

int orc_get_logits(const orc_model* m, double* out, size_t n_out)
{
    size_t need = (size_t)m->c.batch * m->n_in * m->vmax;
    if (n_out < need) return -1;
    memcpy(out, m->logits, sizeof(double) * need);
    return 0;
}

/* Replace the main cache contents by k/v given as [L][B][Hkv][n_pos][hd] fp16, n_past = n_pos. */
int orc_load_kv(orc_model* m, const uint16_t* k, const uint16_t* v, int n_pos)
{
    const orc_config* c = &m->c;
    if (n_pos < 0 || n_pos > c->n_ctx) { set_err("n_pos out of range"); return -1; }
    size_t hd = c->head_dim;
    for (int l = 0; l < c->n_layer; ++l)
        for (int b = 0; b < c->batch; ++b)
            for (int g = 0; g < c->n_kv_head; ++g)
                for (int p = 0; p < n_pos; ++p) {
                    size_t src = ((((size_t)l * c->batch + b) * c->n_kv_head + g) * n_pos + p) * hd;
                    memcpy(cache_at(m->kc, c, c->n_ctx, l, b, g, p), k + src, hd * 2);
                    memcpy(cache_at(m->vc, c, c->n_ctx, l, b, g, p), v + src, hd * 2);
                }
    for (size_t i = 0; i < (size_t)n_pos * c->batch; ++i) m->seq[i] = -1;   /* tokens unknown */
    m->n_past = n_pos;
    return 0;
}

/* Copy the main cache of positions 0..n_pos-1 out as [L][B][Hkv][n_pos][hd] fp16 (read-out only). */
int orc_get_kv(const orc_model* m, uint16_t* k, uint16_t* v, int n_pos)
{
    const orc_config* c = &m->c;
    if (n_pos < 0 || n_pos > m->n_past) { set_err("n_pos out of range"); return -1; }
    size_t hd = c->head_dim;
    for (int l = 0; l < c->n_layer; ++l)
        for (int b = 0; b < c->batch; ++b)
            for (int g = 0; g < c->n_kv_head; ++g)
                for (int p = 0; p < n_pos; ++p) {
                    size_t dst = ((((size_t)l * c->batch + b) * c->n_kv_head + g) * n_pos + p) * hd;
                    memcpy(k + dst, cache_at(m->kc, c, c->n_ctx, l, b, g, p), hd * 2);
                    memcpy(v + dst, cache_at(m->vc, c, c->n_ctx, l, b, g, p), hd * 2);
                }
    return 0;
}

/* One main layer on x[B][d] at position pos (writes that layer's K/V at pos, attends 0..pos),
 * out[B][d] = the residual stream after the layer.  n_past is not changed. */
int orc_layer_forward(orc_model* m, int layer, const double* x, int pos, double* out)
{
    const orc_config* c = &m->c;
    if (layer < 0 || layer >= c->n_layer || pos < 0 || pos >= c->n_ctx) { set_err("bad layer/pos"); return -1; }
    memcpy(out, x, sizeof(double) * (size_t)c->batch * c->d_model);
    for (int b = 0; b < c->batch; ++b)
        layer_forward(m, &m->L[layer], layer, b, out + (size_t)b * c->d_model, pos, m->kc, m->vc, c->n_ctx);
    return 0;
}

/* Whole-sequence causal forward written layer by layer with an explicit mask (keys j > i are
 * excluded), without the step's cache: the definition the prompt pass computes
 * ([J] §3.11: the prompt graph applies a causal mask; §3.12: a key column is masked when it
 * lies after the query's position).  Row 0 only; GPT2 and LLAMA. */
int orc_forward_sequence(const orc_model* m, const int32_t* toks, int n, double* logits, double* normed_hidden)
{
    const orc_config* c = &m->c;
    if (c->arch == ORC_TALKER_CP || n <= 0 || n > c->n_ctx) { set_err("unsupported"); return -1; }
    int d = c->d_model, H = c->n_head, Hk = c->n_kv_head, hd = c->head_dim, ff = c->d_ff, f = c->wfmt;
    int qd = H * hd, kd = Hk * hd, gpt2 = c->arch == ORC_GPT2, grp = H / Hk;
    double* X = (double*)malloc(sizeof(double) * (size_t)n * d);
    double* Q = (double*)malloc(sizeof(double) * (size_t)n * qd);
    double* Kd = (double*)malloc(sizeof(double) * (size_t)n * kd);
    double* Vd = (double*)malloc(sizeof(double) * (size_t)n * kd);
    double* nrm = (double*)malloc(sizeof(double) * (size_t)d);
    double* tmp = (double*)malloc(sizeof(double) * (size_t)(3 * d > ff ? 3 * d : ff) * 2);
    double* s = (double*)malloc(sizeof(double) * (size_t)n);
    double* a = (double*)malloc(sizeof(double) * (size_t)n);
    double* o = (double*)malloc(sizeof(double) * (size_t)qd);
    double* g = (double*)malloc(sizeof(double) * (size_t)ff);
    double* u = (double*)malloc(sizeof(double) * (size_t)ff);
    int bad = 0;
    for (int t = 0; t < n; ++t) bad |= embed(m, toks + t, t, X + (size_t)t * d);
    if (bad) n = 0; /* nothing computed; reported below */
    for (int l = 0; l < c->n_layer; ++l) {
        const orc_layer* L = &m->L[l];
        for (int t = 0; t < n; ++t) {
            double* x = X + (size_t)t * d;
            if (gpt2) {
                orc_layernorm(x, d, L->n1g, L->n1b, c->norm_eps, nrm);
                orc_gemv(f, L->wqkv, 3 * d, d, nrm, L->bqkv, tmp);
                memcpy(Q + (size_t)t * qd, tmp, sizeof(double) * d);
                memcpy(Kd + (size_t)t * kd, tmp + d, sizeof(double) * d);
                memcpy(Vd + (size_t)t * kd, tmp + 2 * d, sizeof(double) * d);
            } else {
                orc_rmsnorm(x, d, L->n1g, c->norm_eps, nrm);
                orc_gemv(f, L->wq, qd, d, nrm, NULL, Q + (size_t)t * qd);
                orc_gemv(f, L->wk, kd, d, nrm, NULL, Kd + (size_t)t * kd);
                orc_gemv(f, L->wv, kd, d, nrm, NULL, Vd + (size_t)t * kd);
                for (int h = 0; h < H; ++h) orc_rope_neox(Q + (size_t)t * qd + h * hd, hd, t, c->rope_theta);
                for (int h = 0; h < Hk; ++h) orc_rope_neox(Kd + (size_t)t * kd + h * hd, hd, t, c->rope_theta);
            }
            /* keys and values pass through their fp16 storage */
            for (int i = 0; i < kd; ++i) {
                Kd[(size_t)t * kd + i] = orc_half_to_double(orc_double_to_half(Kd[(size_t)t * kd + i]));
                Vd[(size_t)t * kd + i] = orc_half_to_double(orc_double_to_half(Vd[(size_t)t * kd + i]));
            }
        }
        for (int t = 0; t < n; ++t) {
            double* x = X + (size_t)t * d;
            for (int h = 0; h < H; ++h) {
                const double* qh = Q + (size_t)t * qd + h * hd;
                for (int j = 0; j < n; ++j) {
                    if (j > t) { s[j] = -INFINITY; continue; }      /* explicit causal mask */
                    const double* kj = Kd + (size_t)j * kd + (h / grp) * hd;
                    double dot = 0.0;
                    for (int i = 0; i < hd; ++i) dot += qh[i] * kj[i];
                    s[j] = dot / sqrt((double)hd);
                }
                orc_softmax(s, n, a);
                for (int i = 0; i < hd; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < n; ++j) acc += a[j] * Vd[(size_t)j * kd + (h / grp) * hd + i];
                    o[h * hd + i] = acc;
                }
            }
            orc_gemv(f, L->wo, d, qd, o, gpt2 ? L->bo : NULL, tmp);
            for (int i = 0; i < d; ++i) x[i] += tmp[i];
            if (gpt2) {
                orc_layernorm(x, d, L->n2g, L->n2b, c->norm_eps, nrm);
                orc_gemv(f, L->wfc, ff, d, nrm, L->bfc, g);
                for (int i = 0; i < ff; ++i) g[i] = orc_gelu_tanh(g[i]);
                orc_gemv(f, L->wdown, d, ff, g, L->bdown, tmp);
            } else {
                orc_rmsnorm(x, d, L->n2g, c->norm_eps, nrm);
                orc_gemv(f, L->wgate, ff, d, nrm, NULL, g);
                orc_gemv(f, L->wup, ff, d, nrm, NULL, u);
                for (int i = 0; i < ff; ++i) g[i] = orc_silu(g[i]) * u[i];
                orc_gemv(f, L->wdown, d, ff, g, NULL, tmp);
            }
            for (int i = 0; i < d; ++i) x[i] += tmp[i];
        }
    }
    for (int t = 0; t < n; ++t) {
        final_norm(m, X + (size_t)t * d, m->nfg, m->nfb, nrm);
        if (normed_hidden) memcpy(normed_hidden + (size_t)t * d, nrm, sizeof(double) * d);
        orc_gemv(f, m->head, c->vocab, d, nrm, NULL, logits + (size_t)t * c->vocab);
    }
    free(X); free(Q); free(Kd); free(Vd); free(nrm); free(tmp); free(s); free(a); free(o); free(g); free(u);
    if (bad) { set_err("token out of range"); return -1; }
    return 0;
}
