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
// row placement modes for launch_pack
enum PackMode : int { PACK_IDENTITY = 0, PACK_ROPE_PAIRS = 1, PACK_INTERLEAVE_EVEN = 2, PACK_INTERLEAVE_ODD = 3 };

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
// Up to MM_ROWS rows of activations go through the matrix cores together.  Every GEMM operand
// buffer holds MM_ROWS rows; rows past the batch stay zero.
constexpr int MM_ROWS = 16;
constexpr int MM_MAX_SPLIT = 8;   // split-K slices of one GEMM, at most
constexpr int MM_MAX_K = 4096;    // longest reduction dimension

// a GEMM operand: x split into fp16 hi + lo (x - hi), and sum(hi + lo) over each group of 64
struct Act16 {
    __half* hi;        // [MM_ROWS][K]
    __half* lo;        // [MM_ROWS][K]
    float* gsum;       // [MM_ROWS][K / 64]
};

// prep: v = x[b] (+ sum over s < n_part of part[s][b]; then v is written back to x[b]);
// y = v, or RMSNorm(v) * g; the operand of y; optionally y itself to norm_out[b]
struct PrepArgs {
    float* x;
    int ldx;
    const float* part;   // [n_part][MM_ROWS][ldx]
    int n_part;
    const float* g;      // null: no norm
    float eps;
    int K, rows;
    Act16 a;
    float* norm_out;     // [rows][K] or null
};

enum Mm16Epi : int { MM_STORE = 0, MM_SWIGLU = 1, MM_QKV_ROPE = 2 };
struct Mm16Out {
    float* y;            // STORE: y[split][b][n] at y + split * slice + b * ldy + n; SWIGLU: y[b][n/2]
    int ldy;
    long long slice;
    int rows;            // activation rows b < rows are written
    // QKV_ROPE: rows [0, qrows) and [qrows, qrows + krows) in RoPE pairs (2i, 2i+1) = (i, i+hd/2)
    // of each head -> rotated q [b][qrows] and K cache; the rest -> V cache; caches
    // [b][Hkv][n_ctx][hd] at slot pos (*posp, else pos_value)
    int qrows, krows, hd, Hkv, n_ctx;
    float* q;
    __half *kc, *vc;
    const float2* rope;
    const int* posp;
    int pos_value;
};

struct EmbedTabs {
    const float* tab[16];
    int rows[16];
};

// W: AFF8 (the only format with a matrix-core path), any N, K % 64 == 0, K <= MM_MAX_K
bool mm16_supported(int fmt, int N, int K);
hipError_t launch_prep16(const PrepArgs& p, hipStream_t st);
hipError_t launch_mm16(int epi, const PackedMat& W, const Act16& a, int splits, const Mm16Out& o, hipStream_t st);
// attention partials (launch_attention layout, max_split slots per head) of rows b < B merged into
// the operand of [B][H * hd]; n_keys = *posp + 1, else n_keys_value
hipError_t launch_merge_prep16(const float* part, int B, int H, int hd, int max_split, const int* posp, int n_keys_value,
                               const Act16& a, hipStream_t st);
// x[b] = sum over c < n_tab of tab[c][codes[b * ld_codes + c]] for b < B (ids clamped into each table)
hipError_t launch_embed_sum16(const EmbedTabs& T, const int* codes, int ld_codes, int n_tab, int d, float* x, int B,
                              hipStream_t st);
// code[b * ld_code] = argmax of logits[b * ld_l + 0 .. n) for b < B (ties to the lowest index)
hipError_t launch_argmax_rows(const float* logits, int ld_l, int n, int* code, int ld_code, int B, hipStream_t st);
// y[i] = sum over s < S of part[s * slice + i] for i < n
hipError_t launch_sum_slices(const float* part, int S, long long slice, float* y, long long n, hipStream_t st);
// hist[*pos][0..n) = codes[0..n) (n may be 0), then *pos += 1
hipError_t launch_frame_done(const int* codes, int n, int* hist, int* pos, hipStream_t st);

// top-k draw for rows b < B: id of logits[b * ld_l ..] at counter (*posp, b, pass) -> out[b * ld_out]
hipError_t launch_topk_rows(const float* logits, int ld_l, int n, int k, float temperature, unsigned long long seed,
                            int pass, const int* posp, int* out, int ld_out, int B, hipStream_t st);

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
