// frame.h — host-side launchers of the batched Talker + code-predictor operators (internal).
#pragma once

#include "kernels.h"

namespace tsd {

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
constexpr int MM_MAX_SPLIT = 8;   // split-K slices of one GEMM, at most
constexpr int MM_MAX_K = 4096;    // longest reduction dimension


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
    const uint32_t* err;  // STORE: when *err is set (a rejected input) nothing is written
    // QKV_ROPE, fused with the attention (launch_qkv_attention): every value also goes out as an
    // exchange word xq[b * ldx + col] (q, then the fp16-rounded k, then v, columns as the rows of
    // W) tagged with epoch (*xctr) * FUSE_EPOCHS + xidx + 1; null xq: not published
    uint64_t* xq;
    int ldx;
    const uint32_t* xctr;
    int xidx;
};
constexpr int FUSE_EPOCHS = 128;   // fused launches per frame, at most (epochs FUSE_EPOCHS apart per frame)

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
    int draw;            // 0: the greedy argmax; 1: the chain's draw
    SampChain ch;
    unsigned long long seed;
    int pass;
    const int* posp;
    int* code;           // code[b * ld_code]: the row's code, overwritten by the pick
    int ld_code;
    // the penalty's history and the consumed-token record (null: none): seq[p * B + b] for
    // p < *posp, then the code this position consumed (code[b * ld_code] before the pick), which
    // is also written to seq[*posp * B + b]
    int* seq;
    RowPrep prep;        // prep.src = -1: none
    const uint32_t* err; // when *err is set (a rejected input) nothing is written
};
hipError_t launch_pick(const PickArgs& a, hipStream_t st);
// The QKV product of a layer (QKV_ROPE epilogue, publishing its values as exchange words, o.xq
// set) and the attention of that layer in one launch: after the product's workgroups, one
// workgroup per (head, row) preloads the cache rows of the positions before the new one, polls
// its query and the new key and value from the exchange (bounded by limit ticks of the 100 MHz
// clock; on time-out it raises *abort_word and leaves its output unwritten) and writes the
// output projection's operand as attention with act_hi set does (a.n_ctx <= 512).
hipError_t launch_qkv_attention(const TiledMat& W, const MmIn& in, const Mm16Out& o, const AttnArgs& a, long long limit,
                                uint32_t* abort_word, hipStream_t st);
bool qkv_attention_fits(const TiledMat& W, const AttnArgs& a);
// y[i] = sum over s < S of part[s * slice + i] for i < n
hipError_t launch_sum_slices(const float* part, int S, long long slice, float* y, long long n, hipStream_t st);
// hist[*pos][0..n) = codes[0..n) (n may be 0), with seq: seq[*pos * B + b] = codes[b * C] for
// b < B (the consumed code 0 of a frame no pick ran on); then *pos += 1.  Nothing when *err is set.
// *fctr (the fused launches' epoch counter, unless null) += 1 in every case.
hipError_t launch_frame_done(const int* codes, int n, int* hist, int* pos, int* seq, int B, int C, const uint32_t* err,
                             uint32_t* fctr, hipStream_t st);
hipError_t launch_bump_u32(uint32_t* p, hipStream_t st);   // *p += 1 (one thread)

}  // namespace tsd
