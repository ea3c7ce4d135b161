// kernels.h — host-side launchers of the libtsd kernels (internal).
#pragma once

#include "common.h"

namespace tsd {

// ---- GEMV ------------------------------------------------------------------------------------
// Prologue: how each workgroup builds its copy of the input vector x (into LDS).
// PRO_*_EMB: the input is the embedding gather of the first layer instead of src.
// PRO_ATTN: the input is the attention output, merged here from the per-chunk partials.
enum ProKind : int { PRO_LOAD = 0, PRO_LN = 1, PRO_RMS = 2, PRO_LN_EMB = 3, PRO_RMS_EMB = 4, PRO_ATTN = 5 };

// attention works on chunks of ATTN_CHUNK cached positions (one workgroup each)
constexpr int ATTN_CHUNK = 256;
__host__ __device__ inline int attn_max_split(int n_ctx) { return (n_ctx + ATTN_CHUNK - 1) / ATTN_CHUNK; }

struct ProArgs {
    const float* src;   // [NB][ld_src] input (ignored when n_emb > 0)
    int ld_src;
    const float* g;     // norm gain (LN / RMS)
    const float* beta;  // LayerNorm bias
    float eps;
    // embedding instead of src (one row): x0 = sum_c tab[c][tok[c]] (+ pos_tab[*pos]);
    // workgroup 0 stores x0 to x_out (the residual stream)
    int n_emb;
    const float* tab[16];
    int tab_rows[16];
    const int* tok;
    const float* pos_tab;
    const int* pos;      // position (embedding row, or the attention length: pos + 1 + pos_add keys)
    float* x_out;
    // attention partials [H][max_split][hd + 4] (o, m, l) for PRO_ATTN, one per chunk of
    // a_chunk positions
    const float* part;
    int a_hd, a_max_split, a_chunk, pos_add;
};

enum EpiKind : int {
    EPI_STORE = 0,     // y[b][n] = acc + bias
    EPI_RESID = 1,     // y[n] += acc + bias            (residual add into the stream)
    EPI_GELU = 2,      // y[n] = gelu_tanh(acc + bias)
    EPI_SWIGLU = 3,    // rows (2i, 2i+1) = (gate_i, up_i): y[i] = silu(gate) * up
    EPI_QKV = 4,       // rows [0,qr) -> q, [qr, qr+kr) -> K cache, rest -> V cache (+bias)
    EPI_QKV_ROPE = 5,  // as EPI_QKV, q/k rows stored in RoPE pairs (i, i+hd/2) and rotated
    EPI_HEAD_ARGMAX = 6  // logits + each workgroup's best (logit, index) key; a finalize kernel reduces
};

struct EpiArgs {
    float* y;
    int ldy;
    const float* bias;
    // QKV
    int qrows, krows, hd, n_ctx;
    float* q;
    __half* kc;
    __half* vc;
    const float2* rope;  // [n_ctx][hd/2] (cos, sin)
    const int* pos;      // device position (K/V slot, RoPE angle)
    // head / argmax: best key of workgroup i -> best[i]
    unsigned long long* best;
};

// Launch the fused GEMV y = epilogue(W . prologue(x)).  Returns hipSuccess or the launch error.
hipError_t launch_gemv(int fmt, int pro, int epi, const PackedMat& W, const ProArgs& pa, const EpiArgs& ea,
                       hipStream_t st);
// y = W x (+bias) with the weight loads marked non-temporal: for a matrix streamed once
hipError_t launch_gemv_stream(int fmt, const PackedMat& W, const ProArgs& pa, const EpiArgs& ea, hipStream_t st);
// the tile (rows per workgroup) the launcher uses for a shape; for byte/launch accounting
int gemv_rows_per_block(int fmt, int K, int epi);

hipError_t launch_pack(int fmt, const void* src, int N, int K, void* dst_base, int dst_N,
                       int dst_row0, int mode, int hd, hipStream_t st);
// row placement modes for launch_pack (and launch_pack_tiled)
enum PackMode : int { PACK_IDENTITY = 0, PACK_ROPE_PAIRS = 1, PACK_INTERLEAVE_EVEN = 2, PACK_INTERLEAVE_ODD = 3 };
// destination row of source row r:
//   IDENTITY: row0 + r
//   ROPE_PAIRS: within each head of hd rows, element i < hd/2 -> 2i, i >= hd/2 -> 2(i-hd/2)+1
//   INTERLEAVE_EVEN / _ODD: row0 + 2r (+1)
__host__ __device__ inline int place_row(int r, int mode, int hd, int row0)
{
    if (mode == PACK_ROPE_PAIRS) {
        const int h = r / hd, i = r - h * hd, half = hd / 2;
        return row0 + h * hd + (i < half ? 2 * i : 2 * (i - half) + 1);
    }
    if (mode == PACK_INTERLEAVE_EVEN) return row0 + 2 * r;
    if (mode == PACK_INTERLEAVE_ODD) return row0 + 2 * r + 1;
    return row0 + r;
}

// ---- attention -------------------------------------------------------------------------------
struct AttnArgs {
    const float* q;      // [B][ldq] with the H query heads at q + b*ldq
    int ldq;
    const __half* k;     // [B][Hkv][n_ctx][hd]
    const __half* v;
    float* out;          // [B][ldo] with head h at out + b*ldo + h*hd
    int ldo;
    float* part;         // [B][H][max_split][hd + 4]: unnormalised o, then m, l (log2 domain)
    int B, H, Hkv, hd, n_ctx;
    const int* pos;      // n_keys = *pos + 1 + pos_add when pos != null
    int pos_add;
    int n_keys;          // used when pos == null
    // when the cache fits one chunk (n_ctx <= ATTN_CHUNK) and act_hi is set, o is written straight
    // into the batched GEMM operand (row b, column h * hd + i, il_act layout) as fp16 hi and lo
    // (x - hi) instead of partials
    __half* act_hi;
    __half* act_lo;
};
size_t attn_part_bytes(int B, int H, int n_ctx, int hd);
hipError_t launch_attention(const AttnArgs& a, hipStream_t st);
// merges the partials into a.out (standalone operator only; the step merges in the O-proj)
hipError_t launch_attention_merge(const AttnArgs& a, int n_keys, hipStream_t st);

// ---- sampler finalize --------------------------------------------------------------------------
// greedy: reduce the head's per-workgroup keys [n], publish the id into tok, append it to the
// history at the current position and advance the position (one workgroup)
hipError_t launch_argmax_finalize(const unsigned long long* best, int n, int* tok, int* hist, int hist_stride, int* pos,
                                  hipStream_t st);

// ---- persistent decode step (step.hip) ---------------------------------------------------------
// One launch runs the whole batch-1 step; phases hand data over through exchange words
// (exchange.h).  Every layer's tensors sit at one fixed stride from the previous layer's in the
// workspace, so the kernel derives them with scalar adds instead of loading a table.
struct StepLayer {
    PackedMat qkv, o, fc, down;               // fc: FC (GPT-2) or interleaved gate/up (Llama)
    const float *n1g, *n1b, *n2g, *n2b;       // norm gains / LayerNorm biases (null for RMSNorm)
    const float *bqkv, *bo, *bfc, *bdown;     // linear biases (null without)
    __half *kc, *vc;                          // this layer's cache [Hkv][n_ctx][hd]
};
struct StepArgs {
    StepLayer L0;                             // layer 0; layer l is layer 0 moved by l strides
    long long lstride;                        // bytes between consecutive layers' weights and vectors
    long long kvstride;                       // elements between consecutive layers' caches
    int n_layer, H, Hk, n_ctx, vocab, max_split;
    float eps;
    const float* emb;                         // [vocab][d]
    const float* wpe;                         // [n_ctx][d] learned positions, or null
    const float *nfg, *nfb;                   // final norm
    PackedMat head;
    const float2* rope;                       // [n_ctx][hd/2] (cos, sin), Llama
    int *pos, *tok, *hist;                    // step state (read at launch start, advanced at its end)
    uint32_t* ctr;                            // launches completed: the epoch base
    uint32_t* abort_word;                     // sticky: a wait gave up
    float* logits;                            // [vocab]
    // exchange words: QKV out, attention partials [H][max_split][hd+2], attention-block output
    // (residual stream), MLP hidden, layer output (residual stream), per-workgroup argmax keys
    uint64_t *x_qkv, *x_part, *x_attn, *x_h, *x_out, *x_best;
    long long spin_limit;                     // ticks of the 100 MHz clock a wait may take
    // sampler: mode 0 greedy, 1 top-k (the head also publishes its logits as exchange words)
    int samp_mode, top_k;
    float temperature;
    unsigned long long seed;
    uint64_t* x_logit;                        // [vocab] exchange words of the logits (top-k)
};
// the step kernel for a shape, or null when the shape has no instantiation
const void* step_kernel_for(int fmt, int arch_llama, int d, int h, int hk, int hd, int ff, int vocab);
// d_args: the arguments in device memory (read by every phase)
hipError_t launch_step(const void* kernel, const StepArgs* d_args, int n_wg, hipStream_t st);

// ---- top-k sampler (sampler.hip, sampler.h) ----------------------------------------------------
// the id drawn from logits[0..n): k largest of logits / temperature, counter (pos, row, pass);
// pos is *posp when posp is set (then the id is also written to hist[pos * hist_stride] and *posp
// advanced), else pos_value.  k must be 1..min(n, 1024).
bool topk_supported(int n, int k);
hipError_t launch_topk(const float* logits, int n, int k, float temperature, unsigned long long seed, int row, int pass,
                       int* posp, int pos_value, int* out, int* hist, int hist_stride, hipStream_t st);

// ---- batched frame operators (frame.hip) -------------------------------------------------------
// Up to MM_ROWS rows of activations go through the matrix cores together.  The batched path keeps
// its data in layouts made for the MFMA operand fragments, so that one load instruction of a
// wave reads 1 KB of consecutive bytes:
//   * tiled weights (8-bit affine): for each 16-row tile t and group g of 64 along K, a 1 KB
//     block of 64 lanes x 16 bytes; lane (j, c) (j = lane / 16, c = lane % 16) holds row 16 t + c
//     at K offsets 64 g + kappa(j, e), e = 0..15, kappa(j, e) = 32 (e / 8) + 8 j + e % 8; then
//     one 32-bit (scale | bias << 16) word per (t, g, c);
//   * the fp32 rows x[b][k] (the residual stream) at il_x(b, k) = ((k / 4) 16 + b) 4 + k % 4;
//   * the fp16 hi/lo operand of a GEMM at il_act(b, k) = ((k / 8) 16 + b) 8 + k % 8.
// Every such buffer holds MM_ROWS rows; rows past the batch stay zero.
constexpr int MM_ROWS = 16;
constexpr int MM_MAX_SPLIT = 8;   // split-K slices of one GEMM, at most
constexpr int MM_MAX_K = 4096;    // longest reduction dimension

__host__ __device__ inline size_t il_x(int b, int k) { return ((size_t)(k >> 2) * MM_ROWS + b) * 4 + (k & 3); }
__host__ __device__ inline size_t il_act(int b, int k) { return ((size_t)(k >> 3) * MM_ROWS + b) * 8 + (k & 7); }

struct TiledMat {
    const uint8_t* q;     // [tiles][G][64 lanes][16]
    const uint32_t* sb;   // [tiles][G][16]
    int N, K;
};
inline size_t tiled_q_bytes(int N, int K) { return (size_t)((N + 15) / 16) * (K / 64) * 1024; }
inline size_t tiled_bytes(int N, int K) { return align256(tiled_q_bytes(N, K)) + (size_t)((N + 15) / 16) * (K / 64) * 64; }
inline TiledMat tiled_view(void* base, int N, int K)
{
    TiledMat m;
    m.q = (const uint8_t*)base;
    m.sb = (const uint32_t*)((uint8_t*)base + align256(tiled_q_bytes(N, K)));
    m.N = N;
    m.K = K;
    return m;
}
// canonical 8-bit affine matrix [N][K] -> rows place_row(r, ...) of a tiled matrix of dst_N rows
// (the destination must be zeroed first when some of its rows are not written)
hipError_t launch_pack_tiled(const void* src, int N, int K, void* dst_base, int dst_N, int dst_row0, int mode, int hd,
                             hipStream_t st);

// a GEMM operand as two fp16 numbers per element, hi = fp16(x) and lo = fp16(x - hi), il_act layout
struct Act16 {
    __half* hi;
    __half* lo;
};
constexpr int MM_MAX_SSQ = 256;   // partial row sums of squares a normed operand can come with

// The operand of a GEMM: ready fp16 hi/lo rows.  When it is a norm's input, a = hi/lo of x * g
// (x the residual rows, g the norm gain) and ssq holds n_ssq partial sums of x^2 per row
// ([n_ssq][MM_ROWS]); the GEMM then applies the RMSNorm's 1 / sqrt(sum / K + eps) to its results
// (summing the partials in a fixed order).
struct MmIn {
    Act16 a;
    const float* ssq;
    int n_ssq;
    float eps;
    int rows;            // rows b < rows are real (the others are zero)
};

enum Mm16Epi : int { MM_STORE = 0, MM_SWIGLU = 1, MM_QKV_ROPE = 2, MM_RESID = 3 };
struct Mm16Out {
    // STORE: y[split][b][n] at y + split * slice + b * ldy + n (row-major).
    // RESID: x[il_x(b, n)] += result (the residual stream); with next.hi set, also the next
    // norm's operand next[il_act(b, n)] = hi/lo of x * g_next[n] and, per 16-column tile t,
    // ssq_out[t][b] = sum over the tile of x^2.
    float* y;
    int ldy;
    long long slice;
    Act16 next;
    const float* g_next;
    float* ssq_out;
    // SWIGLU: rows (2m, 2m+1) = (gate_m, up_m); silu(gate) * up is written as the next GEMM's
    // operand act at il_act(b, m)
    Act16 act;
    int rows;            // activation rows b < rows are written
    // QKV_ROPE: rows [0, qrows) and [qrows, qrows + krows) in RoPE pairs (2i, 2i+1) = (i, i+hd/2)
    // of each head -> rotated q [b][qrows] (row-major) and K cache; the rest -> V cache; caches
    // [b][Hkv][n_ctx][hd] at slot pos (*posp, else pos_value)
    int qrows, krows, hd, Hkv, n_ctx;
    float* q;
    __half *kc, *vc;
    const float2* rope;
    const int* posp;
    int pos_value;
};

// A norm's input prepared one row per workgroup: the rows (rows b < B) come from
//   ROW_EMB:  sum over c < n_tab of tab[c][codes[b * ld_codes + c]] (ids clamped into rows[c]),
//   ROW_MAJOR: src[b][K] row-major,
//   ROW_NORMED: RMSNorm(src_il rows) * g_src (src in il_x layout),
// and are written to x (il_x, unless null), with the operand act = hi/lo of x * g (x alone when
// g is null) and ssq[0][b] = sum of x^2 (unless null).
enum RowSrc : int { ROW_EMB = 0, ROW_MAJOR = 1, ROW_NORMED = 2 };
struct RowPrep {
    int src;
    const float* tab[16];
    int tab_rows[16];
    const int* codes;
    int ld_codes, n_tab;
    const float* rows_src;   // ROW_MAJOR [B][K] / ROW_NORMED il_x
    const float* g_src;      // ROW_NORMED gain
    float eps;
    int K, B;
    float* x;
    Act16 act;
    const float* g;
    float* ssq;
};

struct EmbedTabs {
    const float* tab[16];
    int rows[16];
};

bool mm16_supported(int N, int K);   // any N, K % 64 == 0, K <= MM_MAX_K
hipError_t launch_mm16(int epi, const TiledMat& W, const MmIn& in, int splits, const Mm16Out& o, hipStream_t st);
hipError_t launch_row_prep(const RowPrep& p, hipStream_t st);
// attention partials (launch_attention layout, max_split slots per head) of rows b < B merged into
// the operand [B][H * hd]; n_keys = *posp + 1, else n_keys_value
hipError_t launch_merge16(const float* part, int B, int H, int hd, int max_split, const int* posp, int n_keys_value,
                          const Act16& a, hipStream_t st);
// il_x rows -> row-major [B][K]
hipError_t launch_il_to_rows(const float* src, int B, int K, float* dst, hipStream_t st);
// The code of every row b < B from logits[b * ld_l .. + n): greedy argmax (ties to the lowest
// index) when top_k == 0, else the top-k draw at counter (*posp, b, pass); written to
// code[b * ld_code].  Then, when prep.src >= 0, that row's next input is prepared as launch_row_prep
// does (ROW_EMB with the drawn code as the id of table 0, or ROW_NORMED).
struct PickArgs {
    const float* logits;
    int ld_l, n, B;
    int top_k;
    float temperature;
    unsigned long long seed;
    int pass;
    const int* posp;
    int* code;
    int ld_code;
    RowPrep prep;        // prep.src = -1: none
};
hipError_t launch_pick(const PickArgs& a, hipStream_t st);
// y[i] = sum over s < S of part[s * slice + i] for i < n
hipError_t launch_sum_slices(const float* part, int S, long long slice, float* y, long long n, hipStream_t st);
// hist[*pos][0..n) = codes[0..n) (n may be 0), then *pos += 1
hipError_t launch_frame_done(const int* codes, int n, int* hist, int* pos, hipStream_t st);

// ---- small state kernels ---------------------------------------------------------------------
// dst[r * cols + c] = src[r * src_stride + c]
hipError_t launch_gather_i32(int* dst, const int* src, int rows, int cols, long long src_stride, hipStream_t st);
hipError_t launch_copy_i32(int* dst, const int* src, int n, hipStream_t st);
hipError_t launch_fill_i32(int* dst, int value, int n, hipStream_t st);
hipError_t launch_fill_u32(unsigned int* dst, unsigned int value, int n, hipStream_t st);
hipError_t launch_fill_u64(unsigned long long* dst, unsigned long long value, int n, hipStream_t st);
hipError_t launch_fill_f32(float* dst, float value, size_t n, hipStream_t st);
hipError_t launch_copy_bytes(void* dst, const void* src, size_t n, hipStream_t st);

}  // namespace tsd
