// prefill.h — the prompt pass of the GPT2/LLAMA decoders (internal; prefill.hip).
//
// A prompt of n positions is one causal forward over n rows ([J] §3.2: the prompt graph and the
// decode graph share one KV cache; §3.11: the prompt graph masks keys after each query's
// position).  With n rows every weight byte feeds n multiply-adds, so the linears are matrix
// products on the matrix cores; the activations of all rows sit in row-major buffers:
//   X  [rows][d]  fp32 residual stream
//   A  rows x K   fp16 hi / lo operand of the next product (hi = fp16(x), lo = fp16(x - hi)), in
//                 fragment order: per 16-row tile and 32-wide block of K, 1 KB in MFMA lane order
//                 (element (r, k) at (((r/16 * K/32 + k/32) * 4 + (k/8) % 4) * 16 + r % 16) * 8 + k % 8),
//                 in whole 32-row tiles
//   Q  [rows][H hd] fp32 queries after RoPE
// Row r is batch row b = r / n_pos, position pos0 + r % n_pos.
#pragma once

#include "frame.h"
#include "kernels.h"

namespace tsd {

constexpr int PF_TILE = 32;            // rows and columns of a product tile (one workgroup)
constexpr int PF_MAX_ROWS = 4096;      // rows one pass of the prompt holds (larger prompts are chunked)

enum PfEpi : int {
    PF_STORE = 0,    // y[r][n] = acc (+ bias[n])
    PF_QKV = 1,      // queries to Q, keys/values to the cache at the row's position (RoPE pairs when rope)
    PF_RESID = 2,    // x[r][n] += acc (+ bias[n])
    PF_GELU = 3,     // operand (hi/lo) [r][n] = gelu(acc + bias[n])
    PF_SWIGLU = 4,   // rows 2i/2i+1 = gate/up: operand [r][i] = silu(gate) * up
};

constexpr int PF_TILED8 = 100;   // weight source: the batched path's tiled 8-bit affine layout

struct PfGemmArgs {
    PackedMat W;                 // packed GEMV layout, N rows of K (W.N / W.K give the shape for either source)
    TiledMat T;                  // tiled 8-bit affine layout (launch_pf_gemm_tiled)
    int M;                       // operand rows
    const __half* ahi;           // operand, fragment order with W.K columns
    const __half* alo;
    const float* bias;           // [N] or null
    float* y;                    // PF_STORE / PF_RESID: [M][ldy] fp32
    int ldy;
    __half* ohi;                 // PF_GELU / PF_SWIGLU: next operand, fragment order with ldo columns
    __half* olo;
    int ldo;
    // PF_QKV
    float* q;                    // [M][ldq]
    int ldq;
    int qrows, krows, hd, rope;  // rope: q and k rows are in RoPE pairs (row 2i: element i, 2i+1: i + hd/2)
    const float2* rope_tab;      // [n_ctx][hd/2] (cos, sin)
    __half *kc, *vc;             // layer cache [B][Hkv][n_ctx][hd]
    long long kv_row;            // elements of one batch row's slab
    int n_ctx, n_pos, pos0;
};

struct PfRowArgs {
    int M, d, n_pos, pos0;
    // embedding rows: the sum over c < n_tab of tab[c][id_c], id_c = tok[(b * tok_stride + t0 + t)
    // * n_tab + c] clamped into [0, tab_rows[c]) (one table for GPT2/LLAMA, one per codebook for
    // the Talker)
    const int* tok;
    long long tok_stride;
    int t0, n_prompt;            // n_prompt: prompt length (for the history of the next id)
    int n_tab;
    const float* tab[16];
    int tab_rows[16];
    const float* wpe;            // [n_ctx][d] learned positions or null
    int* seq;                    // [n_ctx][B] consumed id (code 0)
    int* hist;                   // [n_ctx][B] next ids, or null
    int B;
    // norm
    const float* x;              // [M][d]
    float* x_out;
    const float* g;              // gain
    const float* bn;             // LayerNorm bias (null: RMSNorm)
    float eps;
    __half *ahi, *alo;           // operand, fragment order with d columns
};

struct PfAttnArgs {
    const float* q;              // [M][ldq] after RoPE
    int ldq;
    const __half *kc, *vc;       // layer cache [B][Hkv][n_ctx][hd]
    long long kv_row;
    int M, H, Hkv, hd, n_ctx, n_pos, pos0;
    __half *ohi, *olo;           // operand, fragment order with ldo columns (head h at column h hd)
    int ldo;
};

// supported when the reduction dimension is a multiple of 32 and the operand rows fit
bool pf_gemm_ok(int fmt, int K);
hipError_t launch_pf_gemm(int fmt, int epi, const PfGemmArgs& a, hipStream_t st);
// the same product with a.T (tiled 8-bit affine) as the weights; a.W.N / a.W.K carry the shape
hipError_t launch_pf_gemm_tiled(int epi, const PfGemmArgs& a, hipStream_t st);
// X rows from the embeddings (and the history words), then the first norm into the operand
hipError_t launch_pf_embed(const PfRowArgs& a, hipStream_t st);
hipError_t launch_pf_norm(const PfRowArgs& a, hipStream_t st);
// fp32 rows x [M][K] -> operand hi/lo in fragment order, rows up to the next multiple of 32
// zero-filled (standalone product)
hipError_t launch_pf_split(const float* x, int M, int K, __half* hi, __half* lo, hipStream_t st);
hipError_t launch_pf_attention(const PfAttnArgs& a, hipStream_t st);

}  // namespace tsd
