/*
 * tsd.h — C ABI of libtsd: the single-token, memory-bound decode step of a speech-token
 * transformer with block-quantized weights, on AMD Instinct MI355X (gfx950).
 *
 * Sources for what each call computes:
 *   [J] "Chatterbox -> ggml Port: Development Journal" (chatterbox.cpp PROGRESS.md)
 *   [F] "Every Frame Is a Memory Read: A Systems View of Speech Model Inference on Apple Silicon"
 *
 * General conventions
 *   - Every function returns tsd_status; 0 (TSD_OK) is success.  No C++ exception crosses the
 *     ABI.  On any error the model state is unchanged and tsd_last_error() describes it.
 *   - Token ids live in device memory, so they are checked on the device: an id outside its
 *     vocabulary (token or code 0: [0, vocab); TALKER_CP codes 1..C-1: [0, cp_vocab)) makes that
 *     call, and every model call after it, do nothing (no position, id, history or logit
 *     changes), and the next tsd_synchronize returns TSD_ERR_INVALID_ARGUMENT, resets n_past to
 *     what it was before the rejected call, and lets the model run again.  Until then tsd_n_past
 *     counts the skipped calls as if they had run.
 *   - Pointers named d_* are device pointers (HIP global memory) owned by the caller.  The
 *     library never allocates device memory for tensors: all model state lives in the
 *     caller's workspace.  (Creating the step graph lets the HIP runtime allocate its own
 *     small bookkeeping.)
 *   - `stream` is a hipStream_t passed as void*.  Calls only enqueue work on it; results in
 *     device memory are valid once the caller synchronises that stream.
 *   - A model is not thread-safe; use one model per stream.
 *
 * Weight formats ([J] appendix A3 "Quantize T3" and §3.23; [F] §3 "Predict first: the roofline"):
 *   TSD_W_Q4_0        rows of K/32 blocks, 18 bytes each: fp16 scale d (little endian), then 16
 *                     bytes; element j<16 is the low nibble of byte j, element j+16 its high
 *                     nibble; w = (q - 8) * d.
 *   TSD_W_Q8_0        rows of K/32 blocks, 34 bytes each: fp16 d, then 32 int8 q; w = d * q.
 *   TSD_W_AFFINE8_G64 planar: q[N][K] uint8, then s[N][K/64] fp16, then b[N][K/64] fp16;
 *                     w = s * q + b for each group of 64 along K.
 *   TSD_W_Q5_0        ([J] appendix A3's third legacy block) rows of K/32 blocks, 22 bytes each:
 *                     fp16 d, a little-endian 32-bit word whose bit j is element j's fifth bit,
 *                     then 16 nibble bytes ordered as in Q4_0; w = (q - 16) * d with
 *                     q = nibble | fifth bit << 4.
 *   TSD_W_AFFINE4_G64, TSD_W_AFFINE4_G32 ([F] §5.8's 4-bit variants, groups of 64 and 32)
 *                     planar: q[N][K/2] bytes, element 2i in the low nibble of byte i and 2i+1
 *                     in the high one, then s[N][K/G] fp16, then b[N][K/G] fp16; w = s * q + b.
 *   All matrices are W[N][K]: N output rows, each contiguous along the reduction axis K
 *   ([J] §3.2 issue 5).  K must be a multiple of the group: 32 (Q4_0, Q8_0, Q5_0, AFFINE4_G32)
 *   or 64 (AFFINE8_G64, AFFINE4_G64).  TALKER_CP takes TSD_W_AFFINE8_G64 only.
 */
#ifndef TSD_H
#define TSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TSD_OK = 0,
    TSD_ERR_INVALID_ARGUMENT = 1, /* null/undersized buffer, bad shape, token >= vocab */
    TSD_ERR_UNSUPPORTED = 2,      /* a valid configuration the library has no kernel for */
    TSD_ERR_OUT_OF_MEMORY = 3,    /* host allocation failed */
    TSD_ERR_CONTEXT_FULL = 4,     /* n_past + n > n_ctx */
    TSD_ERR_HIP = 5,              /* a HIP runtime call failed; message has hipGetErrorString */
    TSD_ERR_STATE = 6,            /* call not valid in the current state */
    TSD_ERR_TIMEOUT = 7           /* a bounded wait inside the persistent step gave up (see tsd_synchronize) */
} tsd_status;

typedef enum { TSD_ARCH_GPT2 = 0, TSD_ARCH_LLAMA = 1, TSD_ARCH_TALKER_CP = 2 } tsd_arch;
typedef enum {
    TSD_W_Q4_0 = 0,
    TSD_W_Q8_0 = 1,
    TSD_W_AFFINE8_G64 = 2,
    TSD_W_Q5_0 = 3,
    TSD_W_AFFINE4_G64 = 4,
    TSD_W_AFFINE4_G32 = 5
} tsd_wfmt;

/* How a step is launched.
 *   PERSISTENT (default): batch-1 GPT2/LLAMA steps run as ONE launch of one workgroup per
 *     compute unit that walks every layer, handing each phase's output to the next through
 *     epoch-tagged 64-bit words in the workspace (no kernel boundary between operators; [J]
 *     §3.14 and [F] §4 measure the per-kernel fixed cost this removes).  Shapes without a
 *     persistent kernel fall back to PER_OPERATOR.
 *   PER_OPERATOR: one launch per fused operator (QKV, attention, O-proj, FC, down, head,
 *     sampler), all captured in the step graph. */
typedef enum { TSD_LAUNCH_PERSISTENT = 0, TSD_LAUNCH_PER_OPERATOR = 1 } tsd_launch_mode;

/* Model shape.
 *   GPT2 : GPT-2-Medium-shaped T3 ([J] §3.2): learned positions, pre-LayerNorm, fused QKV with
 *          bias, GELU (tanh form) MLP with biases, untied head without bias.  Requires
 *          n_head * head_dim == d_model and n_kv_head == n_head.
 *   LLAMA: Llama-shaped T3 ([J] §3.19): RMSNorm, separate Q/K/V without bias, RoPE (NEOX
 *          half-split, theta rope_theta, no frequency scaling), SwiGLU MLP, head without bias.
 *   TALKER_CP: Talker + code predictor frame loop ([F] §1): LLAMA-shaped Talker of n_layer,
 *          then a LLAMA-shaped predictor of cp_n_layer (same widths) running n_codebooks-1
 *          sequential passes.  One step is one frame of n_codebooks codes.
 * batch: GPT2/LLAMA 1 or 2 (two rows read every weight once per step: two streams, or a
 * guided pair, see tsd_sampling.cfg; batch 2 runs PERSISTENT for the GPT-2-Medium Q4_0 and
 * Llama-520M Q8_0 shapes and the test shapes, else PER_OPERATOR); TALKER_CP 1..16.
 * norm_eps is used by every LayerNorm/RMSNorm. */
typedef struct {
    int32_t arch, wfmt;
    int32_t n_layer, d_model, n_head, n_kv_head, head_dim, d_ff, vocab, n_ctx, batch;
    float norm_eps, rope_theta;
    int32_t cp_n_layer, n_codebooks, cp_vocab; /* TALKER_CP only, else 0 */
    int32_t launch_mode;  /* tsd_launch_mode */
    int32_t n_workgroups; /* PERSISTENT: grid size, 0 = one per compute unit; more than can be
                             resident at once is TSD_ERR_UNSUPPORTED */
} tsd_config;

/* Sampler chain ([J] §3.2: the T3 port's order, temperature, top-k, top-p, repetition penalty;
 * [J] §3.19: the multilingual order, repetition penalty, temperature, min-p, top-p, top-k; [F]
 * §5.2 and §5.5: the random state and the penalty's history on the device).
 * mode 0: greedy argmax, ties to the lowest index; with rep_penalty on, the argmax of the
 *         penalized logits (processors, no warpers, as when not sampling).
 * mode 1: the chain in `order`, then a draw: u in [0,1) is the top 24 bits of the first word of
 *         Philox4x64-10 (Salmon et al. 2011) with key (seed, 0) and counter (position, row,
 *         pass, 0); the survivors are walked in descending order of their final values (ties by
 *         lower index) and the first whose cumulative mass exceeds u * total is returned.
 * The steps:
 *   temperature  logits / temperature (positive, finite);
 *   top_k        the k largest, ties by lower index; <= 0 or > vocab means the whole vocabulary;
 *   top_p        keep, in descending order, every entry whose preceding mass is below top_p
 *                (measured over what survives the steps before it); 0 or 1 is off;
 *   min_p        keep the entries whose probability is at least min_p times the largest; 0 is
 *                off; only in TSD_ORDER_MTL;
 *   rep_penalty  every id present in the row's history (counted once) gets logit / theta if the
 *                logit is >= 0, logit * theta if negative; 0 or 1 is off.  The history is the
 *                tokens the row consumed at positions 0..n_past (prompt included; for TALKER_CP
 *                code 0 of every frame); tsd_load_kv leaves the loaded positions without one.
 *                TALKER_CP: the Talker's code-0 head only, never the code predictor's heads.
 * Classifier-free guidance ([J] §3.19 "Sampling path", §3.21 phase 1: cond and uncond as two
 * rows of one batch-2 forward, combined at the logits): with cfg = 1 the model's two rows run
 * the same tokens after their own prompts; the logits that enter the chain (first, before the
 * penalty) are l_0 + cfg_weight * (l_0 - l_1); the draw uses row 0's counter and history, and
 * both rows get the id.  cfg_weight 0 is the conditioned row alone.
 * Draws with k > 1024 (or a vocabulary over 12288) are TSD_ERR_UNSUPPORTED. */
typedef enum { TSD_ORDER_T3 = 0, TSD_ORDER_MTL = 1 } tsd_sampler_order;
typedef struct {
    int32_t mode;
    int32_t top_k;
    float temperature;
    uint64_t seed;
    float top_p;
    float min_p;
    float rep_penalty;
    int32_t order;    /* tsd_sampler_order */
    int32_t cfg;      /* 1: classifier-free guidance over the two rows of a batch-2 GPT2/LLAMA model */
    float cfg_weight; /* w: the draw (or argmax) is over cond + w (cond - uncond), row 0 = cond */
} tsd_sampling;

typedef struct {
    const void* ptr; /* device pointer */
    size_t bytes;
} tsd_tensor;

typedef struct tsd_model tsd_model;

/* Bytes of device workspace a model of this shape needs (packed weights, KV cache,
 * activations, step state).  The caller allocates it (256-byte aligned). */
tsd_status tsd_workspace_bytes(const tsd_config* cfg, size_t* out_bytes);

/* Create a model.  `weights` is the canonical list (all device pointers, fp32 for tables,
 * norms and biases, the configured format for matrices):
 *   GPT2 : wte[V][d], wpe[n_ctx][d], per layer {ln1_g[d], ln1_b[d], qkv_w[3d][d], qkv_b[3d],
 *          o_w[d][d], o_b[d], ln2_g[d], ln2_b[d], fc_w[ff][d], fc_b[ff], down_w[d][ff],
 *          down_b[d]}, lnf_g[d], lnf_b[d], head_w[V][d]            (2 + 12 L + 3 tensors)
 *   LLAMA: emb[V][d], per layer {rms1_g[d], q_w[H hd][d], k_w[Hkv hd][d], v_w[Hkv hd][d],
 *          o_w[d][H hd], rms2_g[d], gate_w[ff][d], up_w[ff][d], down_w[d][ff]}, rmsf_g[d],
 *          head_w[V][d]                                                (1 + 9 L + 2 tensors)
 *   TALKER_CP: E_0[V][d], E_c[cp_vocab][d] for c = 1..C-1, Talker layers as LLAMA, rmsf_g,
 *          head_w[V][d], predictor layers as LLAMA, predictor rmsf_g, predictor heads
 *          c = 1..C-1 [cp_vocab][d]
 * The weights are repacked into the workspace on `stream`; the canonical buffers may be freed
 * once that stream has been synchronised.  The workspace must outlive the model.  The step
 * is captured once into a HIP graph here.  `sampling` may be NULL (greedy). */
tsd_status tsd_model_create(const tsd_config* cfg, const tsd_tensor* weights, int n_weights,
                            void* d_workspace, size_t workspace_bytes, void* stream,
                            const tsd_sampling* sampling, tsd_model** out);

/* Prefill ([J] §3.2: a prompt graph and a decode graph over one persistent KV cache; §3.11: the
 * prompt graph masks every key after its query's position).  Positions n_past .. n_past + n - 2
 * run as one causal prompt pass (matrix-core products over all their rows, chunks of up to 4096
 * rows of batch x positions; for TALKER_CP the Talker only, on the sums of each frame's code
 * embeddings), the last position as one decode step (head, sampler, history; for TALKER_CP the
 * whole frame).  d_tokens is [batch][n][tokens per position] (1, or n_codebooks for TALKER_CP);
 * d_next (may be NULL) receives [batch][tokens per step], the ids sampled after the last prompt
 * position.  The token history (tsd_get_tokens) at a GPT2/LLAMA prompt position before the last
 * holds the next prompt id (TALKER_CP prompt frames leave it alone).  The cached keys and values
 * agree with tsd_prefill_stepwise's to fp32 rounding (the sums run in another order), not bit
 * for bit.  TSD_ERR_CONTEXT_FULL if n_past + n > n_ctx.  Every id of the prompt is checked on the
 * device before the pass: one outside its vocabulary voids the call (see the conventions above;
 * tsd_synchronize reports TSD_ERR_INVALID_ARGUMENT).  n_past advances by n only once every launch
 * of the call has been enqueued. */
tsd_status tsd_prefill(tsd_model* m, const int32_t* d_tokens, int n, int32_t* d_next);
/* Prefill by the decode step at every prompt position (identical kernels, so the cache matches
 * what decoding the prompt one id at a time writes, bit for bit; TALKER_CP prompt frames run the
 * Talker only); arguments as tsd_prefill.  The GPT2/LLAMA history at a prompt position holds
 * the id the step sampled there. */
tsd_status tsd_prefill_stepwise(tsd_model* m, const int32_t* d_tokens, int n, int32_t* d_next);

/* One decode step (one frame for TALKER_CP) at position n_past: launches the persistent step
 * kernel (PERSISTENT: one launch, which a caller may capture into its own graph), or replays the
 * captured step graph (PER_OPERATOR, TALKER_CP).
 * d_in is [batch][tokens per position] or NULL for "the ids sampled by the previous step";
 * d_next may be NULL.  The sampled ids are also appended to the device token history
 * (tsd_get_tokens).  n_past increases by one. */
tsd_status tsd_step(tsd_model* m, const int32_t* d_in, int32_t* d_next);

/* The same step with the same kernels and arguments, enqueued launch by launch instead of as
 * the captured graph (for profilers and counter collectors that cannot follow graph launches).
 * Results are identical to tsd_step. */
tsd_status tsd_step_eager(tsd_model* m, const int32_t* d_in, int32_t* d_next);

/* Wait for the model's stream, then report what went wrong since the last call:
 *   a persistent step gave up on a bounded wait (each wait between its workgroups is limited to
 *     20 ms; it can only run out when other work holds compute units the grid needs, or on a
 *     fault).  That launch and every persistent launch after it returned without moving the
 *     position; nothing hangs and no memory outside the workspace is touched.  The model then
 *     switches to one launch per operator for good (tsd_model_info reports it) and restarts its
 *     exchange.  If every step since the last tsd_synchronize was a plain tsd_step(m, NULL, NULL)
 *     (ids from the device, none copied out), those steps run again at once and TSD_OK is returned
 *     (tsd_last_error says what happened); otherwise n_past is set back to the first lost
 *     position and TSD_ERR_TIMEOUT is returned, and the caller submits the positions from there
 *     again.  A TALKER_CP frame whose fused attention gave up on its wait reports TSD_ERR_TIMEOUT
 *     with the frames since unspecified until tsd_reset.
 *   TSD_ERR_INVALID_ARGUMENT if a call since the last tsd_synchronize passed a token id outside its
 *     vocabulary.  That call and the model calls after it did nothing; n_past is set back to the
 *     device's position and the rejection is cleared, so the model can be used again. */
tsd_status tsd_synchronize(tsd_model* m);

/* For tests of the time-out path only: the limit of every bounded wait of the persistent step,
 * in ticks of the 100 MHz constant clock (ticks <= 0: the normal 20 ms).  With a tiny limit the
 * first wait of the next step gives up at once and every workgroup leaves the kernel normally.
 * TSD_ERR_UNSUPPORTED when the model does not run the persistent step. */
tsd_status tsd_debug_set_wait_limit(tsd_model* m, int64_t ticks);

tsd_status tsd_reset(tsd_model* m);                     /* n_past = 0, history, timeout and rejection cleared */
/* The launch configuration in effect: *launch_mode is PERSISTENT only when the shape has a
 * persistent kernel (else PER_OPERATOR), *n_workgroups its grid (0 for PER_OPERATOR).
 * Either pointer may be NULL. */
tsd_status tsd_model_info(const tsd_model* m, int32_t* launch_mode, int32_t* n_workgroups);
tsd_status tsd_truncate(tsd_model* m, int n_past);      /* keep the first n_past positions */
tsd_status tsd_n_past(const tsd_model* m, int* out);
tsd_status tsd_model_destroy(tsd_model* m);
/* Message of the last error on m (NULL: of the last failed tsd_model_create or standalone
 * call on this thread). */
const char* tsd_last_error(const tsd_model* m);

/* Logits of the last step: [batch][vocab] fp32; for TALKER_CP [batch][n_codebooks][vmax]
 * with vmax = max(vocab, cp_vocab) (entries past a head's vocabulary are 0). */
tsd_status tsd_get_logits(tsd_model* m, float* d_out);
/* Ids sampled at positions [first, first + n): [n][batch][tokens per step] int32. */
tsd_status tsd_get_tokens(tsd_model* m, int first, int n, int32_t* d_out);

/* Replace the (Talker) KV cache by d_k/d_v given as [n_layer][batch][n_kv_head][n_pos]
 * [head_dim] fp16 and set n_past = n_pos (used to start from a given context). */
tsd_status tsd_load_kv(tsd_model* m, const uint16_t* d_k, const uint16_t* d_v, int n_pos);

/* Copy the (Talker) KV cache of positions 0..n_pos-1 (n_pos <= n_past) out to d_k/d_v, laid out
 * as tsd_load_kv takes it: [n_layer][batch][n_kv_head][n_pos][head_dim] fp16 (device).
 * n_pos = 0 copies nothing (d_k/d_v may then be null); n_pos > n_past is TSD_ERR_INVALID_ARGUMENT. */
tsd_status tsd_get_kv(tsd_model* m, uint16_t* d_k, uint16_t* d_v, int n_pos);

/* One main decoder layer on hidden states d_x [batch][d_model] at position pos: writes that
 * layer's K/V at pos, attends to positions 0..pos, writes the residual stream after the
 * layer to d_out [batch][d_model].  n_past is not changed.  Uses the same kernels as the
 * step. */
tsd_status tsd_layer_forward(tsd_model* m, int layer, const float* d_x, int pos, float* d_out);

/* Measurement: runs n_steps real decode steps (advancing n_past like tsd_step, sampled ids fed
 * forward) by enqueueing the step's kernels, with the step's launch configuration and
 * arguments, directly on the model's stream with every launch of one kernel kind bracketed by
 * HIP event records; synchronises after each step and returns the mean duration of that kernel
 * in *avg_us and its launches per step.  Each bracket's own cost is calibrated by an empty
 * bracket recorded just before it and subtracted.  Kinds: 0 norm + fused
 * QKV GEMV, 1 attention, 2 attention merge + output projection, 3 norm + FC / gate-up,
 * 4 down projection, 5 final norm + head + sampler (kinds 0-5: PER_OPERATOR launches),
 * 6 the whole persistent step (PERSISTENT).  A kind the model does not launch is
 * TSD_ERR_UNSUPPORTED. */
tsd_status tsd_time_kernel(tsd_model* m, int kind, int n_steps, float* avg_us, int* launches_per_step);

/* ---- standalone operators (same kernels as the step) ------------------------------------- */

/* The step's top-k draw on d_logits[0..n) (fp32, device): the id is written to d_out[0] (device).
 * k = top_k, or n when top_k <= 0 or > n; the uniform is drawn at counter (pos, row, pass, 0)
 * with key (seed, 0) as in tsd_sampling.  TSD_ERR_UNSUPPORTED for k > 1024 or n > 12288;
 * TSD_ERR_INVALID_ARGUMENT for null buffers, n <= 0, negative counters or a temperature that is
 * not positive and finite. */
tsd_status tsd_sample_topk(const float* d_logits, int n, int top_k, float temperature, uint64_t seed, int row,
                           int pos, int pass, int32_t* d_out, void* stream);

/* The step's sampler chain (tsd_sampling, any mode and order) on d_logits[0..n) (fp32, device)
 * with the history d_hist[0..n_hist) (int32 token ids, device; ids outside [0, n) are ignored;
 * may be NULL when n_hist is 0): the id is written to d_out[0] (device).  The uniform is drawn
 * at counter (pos, row, pass, 0) with key (s->seed, 0).  TSD_ERR_INVALID_ARGUMENT for null
 * buffers, n <= 0, negative counters or n_hist, and parameters outside the ranges of
 * tsd_sampling; TSD_ERR_UNSUPPORTED for k > 1024 or n > 12288. */
tsd_status tsd_sample(const float* d_logits, int n, const tsd_sampling* s, const int32_t* d_hist, int n_hist,
                      int row, int pos, int pass, int32_t* d_out, void* stream);

/* Debug mat-vec on the canonical blocks, no repacking ([J] appendix A3 and §3.23 for the legacy
 * blocks, [F] §3 and §5.8 for the affine groups): d_y[b][n] = sum_k W[n][k] d_x[b][k] for b < B,
 * with every weight decoded from d_w's bytes exactly as its format defines it and the products
 * summed in fp32 in K order, one thread per output.  d_w is the canonical blob of an N x K matrix
 * in format wfmt (w_bytes must equal its canonical size); d_x [B][K] and d_y [B][N] fp32
 * row-major (device, caller-owned; d_y is overwritten).  Slow by design: a reference for checking
 * weights or the packed kernels, never used by the step.  TSD_ERR_INVALID_ARGUMENT for null
 * buffers, an unknown format, N, K or B not positive, K not a multiple of the format's group, or a
 * w_bytes mismatch. */
tsd_status tsd_debug_gemv(int wfmt, const void* d_w, size_t w_bytes, const float* d_x, float* d_y, int N, int K, int B,
                          void* stream);

/* Bytes of the kernel layout of one W[N][K] matrix (tsd_gemv_pack's output). */
tsd_status tsd_gemv_packed_bytes(int wfmt, int N, int K, size_t* out_bytes);
/* Repack a canonical matrix d_w into the kernel layout d_packed (device to device). */
tsd_status tsd_gemv_pack(int wfmt, const void* d_w, size_t w_bytes, int N, int K, void* d_packed,
                         size_t packed_bytes, void* stream);
/* Fused block-dequant GEMV on the packed layout: d_y[b][n] = sum_k W[n][k] d_x[b][k]
 * (+ d_bias[n] if not NULL) for b < B (1 <= B <= 4), fp32 accumulation
 * ([J] §3.15 mat-vec with the bias added in the same kernel).  The matrix is read with
 * non-temporal loads (it is streamed once per call). */
tsd_status tsd_gemv(int wfmt, const void* d_packed, int N, int K, int B, const float* d_x,
                    const float* d_bias, float* d_y, void* stream);

/* Prompt-pass product on the matrix cores from the GEMV layout (tsd_gemv_pack's output, 256-byte
 * aligned): d_y[m][n] = sum_k W[n][k] d_x[m][k] (+ d_bias[n] if not NULL) for m < M, d_x [M][K]
 * and d_y [M][N] fp32 row-major (device, caller-owned; d_y is overwritten).  Each block of 32
 * weights enters as exact fp16 integers (its codes minus their zero point) and each x as two
 * fp16 numbers (hi, x - hi); products accumulate in fp32 per block and the block's scale (and
 * affine bias times the block's sum of x) is applied in fp32 ([J] §3.2 prompt graph: the same
 * weights as the step's mat-vecs, all prompt rows at once).  Any format; K a multiple of the
 * format's group (and of 32).  d_scratch (256-byte aligned, tsd_gemm_scratch_bytes) holds the
 * operand rows. */
tsd_status tsd_gemm_scratch_bytes(int M, int K, size_t* out_bytes);
tsd_status tsd_gemm(int wfmt, const void* d_packed, int N, int K, int M, const float* d_x, const float* d_bias,
                    float* d_y, void* d_scratch, size_t scratch_bytes, void* stream);

/* Batched GEMM on the matrix cores for the 8-bit affine format ([F] §8: batched rollouts turn
 * the memory-bound mat-vec into a skinny product; §3: affine groups of 64):
 * d_y[b][n] = sum_k W[n][k] d_x[b][k] for b < B (1 <= B <= 16), d_x [B][K] and d_y [B][N] fp32
 * row-major (device, caller-owned, d_y is overwritten).  W is first repacked by
 * tsd_gemm_rows_pack from the canonical TSD_W_AFFINE8_G64 matrix into the batched path's own
 * layout (16-row tiles of 1 KB blocks, one per group of 64, in the order the matrix cores read
 * them; tsd_gemm_rows_packed_bytes, 256-byte aligned).  Each x is split into two fp16 numbers
 * (hi, x - hi) and each weight enters exactly (q - 128 in fp16); products accumulate in fp32,
 * the group's scale and bias are applied in fp32.  K must be a multiple of 64 and at most 4096.
 * `splits` (1..8, at most K/64) cuts K into slices run by separate workgroups and summed
 * afterwards.  d_scratch (256-byte aligned, tsd_gemm_rows_scratch_bytes) holds the operand rows
 * and the slices. */
tsd_status tsd_gemm_rows_packed_bytes(int N, int K, size_t* out_bytes);
tsd_status tsd_gemm_rows_pack(const void* d_w, size_t w_bytes, int N, int K, void* d_packed,
                              size_t packed_bytes, void* stream);
tsd_status tsd_gemm_rows_scratch_bytes(int N, int K, int splits, size_t* out_bytes);
tsd_status tsd_gemm_rows(const void* d_packed, int N, int K, int B, const float* d_x, float* d_y,
                         int splits, void* d_scratch, size_t scratch_bytes, void* stream);

/* Split-KV flash-decode attention of one query per head over an fp16 cache
 * ([J] §3.13: cache laid out head-dim fastest, then position, then head; no mask for a single
 * new token): d_q [B][H][hd] fp32, d_k/d_v [B][Hkv][n_ctx][hd] fp16, attends keys
 * 0..n_keys-1, d_out [B][H][hd] = softmax(q K^T / sqrt(hd)) V.  Query head h reads KV head
 * h / (H / Hkv).  hd must be 64 or 128.  d_scratch holds the split partials
 * (tsd_attention_scratch_bytes). */
tsd_status tsd_attention_scratch_bytes(int B, int H, int n_ctx, int hd, size_t* out_bytes);
tsd_status tsd_attention(const float* d_q, const uint16_t* d_k, const uint16_t* d_v, int B, int H,
                         int Hkv, int hd, int n_keys, int n_ctx, float* d_out, void* d_scratch,
                         size_t scratch_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, serving loops or
 * harnesses that forbid hipMalloc): tsd_attention with the split partials in a fixed array inside
 * the library (TSD_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends) instead of
 * d_scratch.  Arguments, layouts and results are those of tsd_attention (the same kernels).  It
 * allocates nothing.  TSD_ERR_INVALID_ARGUMENT when the shape's partials
 * (tsd_attention_scratch_bytes) exceed TSD_NOALLOC_SCRATCH_BYTES, and for what tsd_attention
 * rejects.  Every call on one GPU shares that GPU's array: calls that overlap on one GPU (other
 * streams or threads) race and must be serialised by the caller.  The stream must belong to the
 * current device. */
#define TSD_NOALLOC_SCRATCH_BYTES (4u << 20)
tsd_status tsd_attention_noalloc(const float* d_q, const uint16_t* d_k, const uint16_t* d_v, int B, int H, int Hkv,
                                 int hd, int n_keys, int n_ctx, float* d_out, void* stream);

#ifdef __cplusplus
}
#endif
#endif
