/*
 * tsd_oracle.h — plain, slow, single-threaded CPU definition of the quantized speech-token
 * decode step.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
 * baseline leg load this library; the product path (libtsd) never does, and the two share no
 * code, header, table or helper.
 *
 * Everything is computed in fp64 from the stored quantized bytes.  The only rounding the method
 * itself prescribes is the fp16 storage of the key/value cache, which this file performs with
 * its own IEEE-754 round-to-nearest-even encoder.
 *
 * Sources (the pages this follows):
 *   [J]  "Chatterbox -> ggml Port: Development Journal" (chatterbox.cpp PROGRESS.md)
 *   [F]  "Every Frame Is a Memory Read: A Systems View of Speech Model Inference on Apple Silicon"
 *
 * Parity status of each function is given next to its definition in tsd_oracle.c.
 */
#ifndef TSD_ORACLE_H
#define TSD_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* weight formats (values are this library's own; the Python side maps names) */
enum { ORC_Q4_0 = 0, ORC_Q8_0 = 1, ORC_AFF8 = 2, ORC_Q5_0 = 3, ORC_AFF4_G64 = 4, ORC_AFF4_G32 = 5 };
/* architectures */
enum { ORC_GPT2 = 0, ORC_LLAMA = 1, ORC_TALKER_CP = 2 };

typedef struct {
    int arch, wfmt;
    int n_layer, d_model, n_head, n_kv_head, head_dim, d_ff, vocab, n_ctx, batch;
    double norm_eps, rope_theta;
    int cp_n_layer, n_codebooks, cp_vocab; /* TALKER_CP only */
    int sample_mode;                       /* 0 greedy, 1 draw */
    int top_k;
    double temperature;
    uint64_t seed;
    double top_p, min_p, rep_penalty;      /* off: 0 (or >= 1), 0, 0 (or 1) */
    int sample_order;                      /* ORC_ORDER_T3 or ORC_ORDER_MTL */
    int cfg;                               /* 1: rows 0 (cond) and 1 (uncond) guided together */
    double cfg_weight;
} orc_config;

/* sampler chain orders ([J] §3.2 and §3.19) */
enum { ORC_ORDER_T3 = 0, ORC_ORDER_MTL = 1 };

typedef struct {
    int mode;                              /* 0 greedy (penalty, then argmax), 1 draw */
    int top_k;                             /* <= 0 or > n: the whole vocabulary */
    double temperature, top_p, min_p, rep_penalty;
    int order;
} orc_sampling;

typedef struct orc_model orc_model;

/* ---- scalars ---- */
double   orc_half_to_double(uint16_t h);
uint16_t orc_double_to_half(double x);              /* IEEE binary16, round to nearest even */
void     orc_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]);
double   orc_uniform24(uint64_t seed, uint32_t row, uint32_t pos, uint32_t pass);

/* ---- formats ---- */
size_t orc_matrix_bytes(int fmt, int N, int K);      /* 0 if K is not a multiple of the block */
int    orc_dequant_row(int fmt, const uint8_t* blob, int N, int K, int n, double* w_out);

/* ---- operators (fp64) ---- */
int  orc_gemv(int fmt, const uint8_t* blob, int N, int K, const double* x, const double* bias,
              double* y);
int  orc_gemv_f32(int fmt, const uint8_t* blob, int N, int K, int B, const float* x,
                  const float* bias, double* y); /* x [B][K] fp32, y [B][N] */
void orc_layernorm(const double* x, int n, const double* g, const double* b, double eps, double* y);
void orc_rmsnorm(const double* x, int n, const double* g, double eps, double* y);
double orc_gelu_tanh(double x);
double orc_silu(double x);
void orc_rope_neox(double* v, int hd, int pos, double theta);
void orc_softmax(const double* s, int n, double* a);
void orc_attend(const double* q, const uint16_t* kc, const uint16_t* vc, int n_keys, int hd,
                double* o); /* kc/vc: [n_keys][hd] fp16 rows */
int  orc_argmax(const double* v, int n);
int  orc_sample_topk(const double* logits, int n, int k, double temperature, double u);
/* the sampler chain over logits[n] with the history's token ids (out-of-range ids ignored);
 * margins: NULL or 6 doubles (see tsd_oracle.c) */
int  orc_sample_chain(const double* logits, int n, const orc_sampling* s, const int32_t* hist,
                      int n_hist, double u, double* margins);

/* ---- models ---- */
int  orc_n_weights(const orc_config* c);
orc_model* orc_model_create(const orc_config* c, const void* const* w, const size_t* sizes, int n);
const char* orc_last_error(void);
void orc_model_destroy(orc_model* m);
void orc_reset(orc_model* m);
int  orc_n_past(const orc_model* m);
int  orc_truncate(orc_model* m, int n_past);
/* tokens per position: 1 (GPT2/LLAMA) or n_codebooks (TALKER_CP) */
int  orc_step(orc_model* m, const int32_t* tok_in, int32_t* tok_out);
int  orc_prefill(orc_model* m, const int32_t* toks, int n, int32_t* tok_out);
/* logits of the last step: [batch][vocab] (head 0) — for TALKER_CP [batch][n_codebooks][vocab_j] */
int  orc_get_logits(const orc_model* m, double* out, size_t n_out);
int  orc_load_kv(orc_model* m, const uint16_t* k, const uint16_t* v, int n_pos);
int  orc_get_kv(const orc_model* m, uint16_t* k, uint16_t* v, int n_pos);
int  orc_layer_forward(orc_model* m, int layer, const double* x, int pos, double* out);
/* full-sequence causal forward from scratch, no cache reuse: logits [n][vocab] and optionally
 * the final-normed hidden states [n][d] (GPT2/LLAMA) */
int  orc_forward_sequence(const orc_model* m, const int32_t* toks, int n, double* logits,
                          double* normed_hidden);

#ifdef __cplusplus
}
#endif
#endif
