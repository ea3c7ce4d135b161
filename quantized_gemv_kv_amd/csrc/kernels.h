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
// caches one workgroup can cover whole (then the attention can write the batched GEMM operand)
__host__ __device__ inline bool attn_direct_fits(int n_ctx) { return n_ctx <= 512; }

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
    // batch rows (blockIdx.y = row b): src and x_out move by b * rs_src, tok by b * rs_tok, part
    // by b * rs_part elements
    long long rs_src, rs_part;
    int rs_tok;
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
    // head: when *err is set (a rejected input, see launch_set_input) the logits are not written
    const uint32_t* err;
    // batch rows (blockIdx.y = row b): y moves by b * rs_y, q by b * rs_q, the caches by
    // b * rs_kv elements, best by b * (workgroups per row)
    long long rs_y, rs_q, rs_kv;
};

// Launch the fused GEMV y = epilogue(W . prologue(x)) for B batch rows (one grid row each, the
// row strides in pa / ea).  Returns hipSuccess or the launch error.
hipError_t launch_gemv(int fmt, int pro, int epi, const PackedMat& W, const ProArgs& pa, const EpiArgs& ea,
                       hipStream_t st, int B = 1);
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
    // when attn_direct_fits(n_ctx) and act_hi is set, o is written straight
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
// seq: when set, seq[*pos * hist_stride] = the token consumed at this position (*tok before it is
// overwritten by the id)
// B rows: row b's keys at best + b * n, its id to tok[b], hist[*pos * hist_stride + b] (and seq)
// err: when *err is set (a rejected input) nothing is written and the position stays
hipError_t launch_argmax_finalize(const unsigned long long* best, int n, int B, int* tok, int* hist, int* seq, int hist_stride, int* pos,
                                  const uint32_t* err, hipStream_t st);

// ---- persistent decode step (step.hip) ---------------------------------------------------------
// One launch runs the whole batch-1 step; phases hand data over through exchange words
// (exchange.h).  Every layer's tensors sit at one fixed stride from the previous layer's in the
// workspace, so the kernel derives them with scalar adds instead of loading a table.
struct StepLayer {
    PackedMat qkv, o, fc, down;               // fc: FC (GPT-2) or interleaved gate/up (Llama)
    const float *n1g, *n1b, *n2g, *n2b;       // norm gains / LayerNorm biases (null for RMSNorm)
    const float *bqkv, *bo, *bfc, *bdown;     // linear biases (null without)
    // LayerNorm-fed products (GPT-2): c = W g and d = W beta + bias per output row (null for RMSNorm)
    const float *cqkv, *dqkv, *cfc, *dfc;
    __half *kc, *vc;                          // this layer's cache [B][Hkv][n_ctx][hd]
};
// the sampler chain's parameters (sampler.h): temperature, k largest, nucleus, min-p, repetition
// penalty, and which of the two orders runs
constexpr int SAMP_ORDER_T3 = 0, SAMP_ORDER_MTL = 1;
struct SampChain {
    float temperature;   // > 0
    int k;               // 1 <= k <= min(vocabulary, 1024)
    float top_p;         // filters when 0 < top_p < 1
    float min_p;         // filters when 0 < min_p < 1 (SAMP_ORDER_MTL only)
    float penalty;       // applies when != 1
    int order;           // SAMP_ORDER_T3: temperature, top-k, top-p, penalty; SAMP_ORDER_MTL: penalty,
                         // temperature, min-p, top-p, top-k
};
// The residual-stream words (x_attn, x_out) of a batch row hold d words, then room for
// STEP_SHIFT_COPIES copies of word 0, STEP_SHIFT_STRIDE words apart (written by the batch-1
// GPT-2 step): the LayerNorm shift every thread of a consumer needs.  Each wave polls its own copy, on its own cache line, so that the waves of a
// compute unit never poll one line together (such polls merge, and a merged poll can return the
// word as it was when the first of them left).
constexpr int STEP_SHIFT_COPIES = 4, STEP_SHIFT_STRIDE = 16;
// An attention partial of the persistent step (o[0..hd), m, l) takes hd + STEP_PART_PAD words, a
// whole number of 128-byte lines, so that no line holds words of two partials (which the waves of
// the merging item poll separately).
constexpr int STEP_PART_PAD = 16;
// chunks per head the persistent step may split a context of n_ctx keys into (128 keys or more each)
__host__ __device__ inline int step_max_split(int n_ctx) { return (n_ctx + 127) / 128; }
struct StepArgs {
    StepLayer L0;                             // layer 0; layer l is layer 0 moved by l strides
    long long lstride;                        // bytes between consecutive layers' weights and vectors
    long long kvstride;                       // elements between consecutive layers' caches
    int n_layer, H, Hk, n_ctx, vocab, max_split;
    float eps;
    const float* emb;                         // [vocab][d]
    const float* wpe;                         // [n_ctx][d] learned positions, or null
    const float *nfg, *nfb;                   // final norm
    const float *hc, *hdv;                    // the head's W nfg and W nfb (LayerNorm), else null
    PackedMat head;
    const float2* rope;                       // [n_ctx][hd/2] (cos, sin), Llama
    int *pos, *tok, *hist;                    // step state (read at launch start, advanced at its end);
                                              // tok [B], hist [n_ctx][B]
    int* seq;                                 // [n_ctx][B] the token consumed at each position
    uint32_t* ctr;                            // launches completed: the epoch base
    uint32_t* abort_word;                     // sticky: a wait gave up
    const uint32_t* bad_input;                // sticky: an input id was rejected (the launch does nothing)
    float* logits;                            // [B][vocab]
    // exchange words: QKV out, attention partials [H][max_split][hd+STEP_PART_PAD], attention-block output
    // (residual stream), MLP hidden, layer output (residual stream), per-workgroup argmax keys;
    // batch row b's words of each buffer start b * its row stride (xs_*) after row 0's
    uint64_t *x_qkv, *x_part, *x_attn, *x_h, *x_out, *x_best;
    long long xs_qkv, xs_part, xs_d, xs_h, xs_best, xs_logit;   // row strides in words (xs_d: x_attn, x_out)
    uint64_t* x_ao;                           // [B][H * hd] the heads' attention outputs (one writer per head)
    long long xs_ao;
    long long kv_row;                         // elements between batch rows of a layer's cache
    int cfg;                                  // two rows guided: one draw from l0 + cfg_weight (l0 - l1)
    float cfg_weight;
    long long spin_limit;                     // ticks of the 100 MHz clock a wait may take
    // sampler: mode 0 the greedy argmax of the head's per-workgroup keys, 1 the chain's draw on
    // workgroup 0 (the head then also publishes its logits as exchange words)
    int samp_mode;
    SampChain chain;
    unsigned long long seed;
    uint64_t* x_logit;                        // [B][vocab] exchange words of the logits (draw; guided: row 0
                                              // holds the combined logits)
};
// the step kernel for a shape and batch (1 or 2), or null when the shape has no instantiation
const void* step_kernel_for(int fmt, int arch_llama, int d, int h, int hk, int hd, int ff, int vocab, int batch);
// d_args: the arguments in device memory (read by every phase)
hipError_t launch_step(const void* kernel, const StepArgs* d_args, int n_wg, hipStream_t st);

// ---- sampler chain (sampler.hip, sampler.h) --------------------------------------------------
// the id drawn from logits[0..n) by the chain ch with the uniform of counter (pos, row, pass); pos
// is *posp when posp is set (then the id is also written to hist[pos * hist_stride], the consumed
// token *cur to seq_out[pos * seq_stride], and *posp advanced), else pos_value.  The penalty's
// history is seq[p * seq_stride] for p < n_seq (n_seq < 0: p < pos), then *cur when cur is set.
// rows > 1: row r (counter row + r) draws from logits + r * ld_logits with history seq + r and
// consumed token cur[r], writing out[r], hist[.. + r], seq_out[.. + r].  cfg: rows must be 2 and
// one draw is made from the guided logits l0 + cfg_weight (l0 - l1) with row 0's counter and
// history; both rows get the id.
struct SampleArgs {
    const float* logits;
    int n;
    SampChain ch;
    unsigned long long seed;
    int row, pass;
    int* posp;
    int pos_value;
    int* out;
    int* hist;
    int hist_stride;
    const int* seq;
    long long seq_stride;
    int n_seq;
    const int* cur;
    int* seq_out;
    int rows;
    long long ld_logits;
    int cfg;
    float cfg_weight;
    const uint32_t* err;   // when *err is set (a rejected input) nothing is written and the position stays
};
bool sample_supported(int n, int k);
size_t sample_lds_bytes(int n);
hipError_t launch_sample(const SampleArgs& a, hipStream_t st);

// ---- the batched path's row-interleaved layouts (frame.h has the rest) ---------------------------
// fp32 rows x[b][k] at il_x(b, k); fp16 GEMM operands at il_act(b, k); MM_ROWS rows each
constexpr int MM_ROWS = 16;
__host__ __device__ inline size_t il_x(int b, int k) { return ((size_t)(k >> 2) * MM_ROWS + b) * 4 + (k & 3); }
__host__ __device__ inline size_t il_act(int b, int k) { return ((size_t)(k >> 3) * MM_ROWS + b) * 8 + (k & 7); }

// ---- input ids and the rejected-input word ----------------------------------------------------
// Ids enter the model through these kernels only.  An id is valid when 0 <= id < lim0 for column 0
// and 0 <= id < lim1 for the other columns (the Talker's code 0 and codes 1..C-1).
// launch_set_input: dst[r * cols + c] = src[r * src_stride + c] when every id is valid and *err is
// clear; otherwise nothing is copied and *err is set.  launch_check_ids: *err is set when any of the
// rows x n x cols ids at src ([rows][n][cols]) is invalid.  launch_set_pos: *pos = value unless
// *err is set.  Every kernel that writes the model's observable state (the position, the sampled
// ids, the history, the logits) checks *err and writes nothing when it is set, so a call given a
// bad id leaves the state as it was; tsd_synchronize reports and clears the word.
hipError_t launch_set_input(int* dst, const int* src, int rows, int cols, long long src_stride, int lim0, int lim1,
                            uint32_t* err, hipStream_t st);
hipError_t launch_check_ids(const int* src, int rows, int n, int cols, int lim0, int lim1, uint32_t* err, hipStream_t st);
hipError_t launch_set_pos(int* pos, int value, const uint32_t* err, hipStream_t st);

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
