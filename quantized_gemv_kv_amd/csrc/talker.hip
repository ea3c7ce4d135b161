// talker.hip — the Talker + code-predictor frame (TALKER_CP) behind the C ABI.
//
// What one frame computes ("Every Frame Is a Memory Read", §1 and §3): for each batch row, the
// Talker input is the sum of the previous frame's n_codebooks code embeddings (E_0 for code 0,
// E_c for code c); the Talker (LLAMA-shaped: RMSNorm, RoPE, grouped-query attention, SwiGLU)
// advances its cache by one position, its final RMSNorm and head give code 0; then the code
// predictor (LLAMA-shaped, same widths, its own cache restarted every frame) runs its position
// 0 on the Talker's final-normed hidden state and position j on E_{j-1}(c_{j-1}), and its own
// final RMSNorm and head j give code j, for j = 1 .. n_codebooks - 1.
//
// How: every linear is the batched matrix-core GEMM of frame.hip over all rows at once; one
// launch per operator, recorded into the step graph (a frame of the 28 + 5 x 16 layers is about
// a thousand launches, replayed with one graph launch).  Per layer:
//   QKV GEMM (RMSNorm of the fp32 residual rows in its prologue; RoPE and the fp16 K/V append
//   in its epilogue) -> split-KV attention (a one-chunk cache, the predictor's, writes the next
//   operand itself; the Talker's two chunks are merged by a small kernel) -> O-proj GEMM adding
//   into the residual -> gate/up GEMM (RMSNorm prologue, SwiGLU epilogue writing the next
//   operand) -> down GEMM adding into the residual: five or six launches per layer.
// The O and down projections have few 16-row tiles and a long K: sixteen waves of one
// workgroup share the K range, so every result has a single writer and adds deterministically.
#include <algorithm>
#include <string>

#include "model.h"

namespace tsd {
namespace {

#define TRY(expr)                            \
    do {                                     \
        hipError_t e_ = (expr);              \
        if (e_ != hipSuccess) return e_;     \
    } while (0)

// embedding rows gathered by the first predictor layer (its input is E_{j-1}(c_{j-1}))
struct Gather {
    const float* tab;
    int rows;
    const int* codes;
};

// One LLAMA-shaped layer on the residual stream x[rows][d] whose cache (kc, vc: [rows][Hkv]
// [n_ctx][hd]) gets slot pos = *posp (Talker) or pos_value (predictor).  With gather, the
// layer's input rows are embedding rows, which the QKV GEMM also stores to x.
hipError_t layer16(tsd_model* m, const TLayerW& w, float* x, __half* kc, __half* vc, int n_ctx, const int* posp,
                   int pos_value, hipStream_t st, Probe* pr, const Gather* gather = nullptr)
{
    const tsd_config& c = m->c;
    const int d = c.d_model, H = c.n_head, Hk = c.n_kv_head, hd = c.head_dim, ff = c.d_ff, B = c.batch;
    // norm + fused QKV, RoPE and the K/V append
    MmIn iq{};
    iq.x = x;
    iq.g = w.n1g;
    iq.norm = 1;
    iq.eps = c.norm_eps;
    iq.rows = B;
    if (gather) {
        iq.x = nullptr;
        iq.tab = gather->tab;
        iq.tab_rows = gather->rows;
        iq.codes = gather->codes;
        iq.ld_codes = c.n_codebooks;
        iq.x_out = x;
    }
    Mm16Out oq{};
    oq.rows = B;
    oq.qrows = H * hd;
    oq.krows = Hk * hd;
    oq.hd = hd;
    oq.Hkv = Hk;
    oq.n_ctx = n_ctx;
    oq.q = m->qkv;
    oq.kc = kc;
    oq.vc = vc;
    oq.rope = m->rope;
    oq.posp = posp;
    oq.pos_value = pos_value;
    {
        Bracket br(pr, KIND_QKV, st);
        TRY(launch_mm16(MM_QKV_ROPE, MP_X, w.qkv, iq, 1, oq, st));
    }
    // attention; a cache of one chunk writes the output projection's operand directly
    const bool direct = attn_max_split(n_ctx) == 1;
    AttnArgs aa{};
    aa.q = m->qkv;
    aa.ldq = H * hd;
    aa.k = kc;
    aa.v = vc;
    aa.ldo = H * hd;
    aa.part = m->part;
    aa.B = B;
    aa.H = H;
    aa.Hkv = Hk;
    aa.hd = hd;
    aa.n_ctx = n_ctx;
    aa.pos = posp;
    aa.n_keys = pos_value + 1;
    aa.act_hi = direct ? m->act.hi : nullptr;
    aa.act_lo = direct ? m->act.lo : nullptr;
    {
        Bracket br(pr, KIND_ATTN, st);
        TRY(launch_attention(aa, st));
    }
    if (!direct) TRY(launch_merge16(m->part, B, H, hd, attn_max_split(n_ctx), posp, pos_value + 1, m->act, st));
    // output projection + residual
    MmIn ia{};
    ia.a = m->act;
    ia.rows = B;
    Mm16Out orr{};
    orr.y = x;
    orr.rows = B;
    {
        Bracket br(pr, KIND_OPROJ, st);
        TRY(launch_mm16(MM_RESID, MP_ACT, w.o, ia, 1, orr, st));
    }
    // norm + gate/up + SwiGLU, written as the down projection's operand
    MmIn ig{};
    ig.x = x;
    ig.g = w.n2g;
    ig.norm = 1;
    ig.eps = c.norm_eps;
    ig.rows = B;
    Mm16Out of{};
    of.act = m->act;
    of.rows = B;
    {
        Bracket br(pr, KIND_FC, st);
        TRY(launch_mm16(MM_SWIGLU, MP_X, w.fc, ig, 1, of, st));
    }
    // down projection + residual
    {
        Bracket br(pr, KIND_DOWN, st);
        TRY(launch_mm16(MM_RESID, MP_ACT, w.down, ia, 1, orr, st));
    }
    (void)ff;
    return hipSuccess;
}

// final RMSNorm + head j into logits[b][j][..], and code j of every row into tok[b][j];
// norm_out receives the normed hidden state (or null)
hipError_t head16(tsd_model* m, hipStream_t st, Probe* pr, float* x, const float* g, const TiledMat& W, int j, int vocab,
                  float* norm_out)
{
    const tsd_config& c = m->c;
    const int C = c.n_codebooks, B = c.batch;
    MmIn ih{};
    ih.x = x;
    ih.g = g;
    ih.norm = 1;
    ih.eps = c.norm_eps;
    ih.rows = B;
    ih.norm_out = norm_out;
    Mm16Out oh{};
    oh.y = m->logits + (size_t)j * m->vmax;
    oh.ldy = C * m->vmax;
    oh.rows = B;
    {
        Bracket br(pr, KIND_HEAD, st);
        TRY(launch_mm16(MM_STORE, MP_X, W, ih, 1, oh, st));
    }
    const float* lg = m->logits + (size_t)j * m->vmax;
    if (m->samp.mode == 1) {
        const int k = (m->samp.top_k <= 0 || m->samp.top_k > vocab) ? vocab : m->samp.top_k;
        return launch_topk_rows(lg, C * m->vmax, vocab, k, m->samp.temperature, m->samp.seed, j, m->pos, m->tok + j, C, B,
                                st);
    }
    return launch_argmax_rows(lg, C * m->vmax, vocab, m->tok + j, C, B, st);
}

}  // namespace

tsd_status talker_validate(const tsd_config* c, std::string& msg)
{
    if (c->wfmt != TSD_W_AFFINE8_G64) {
        msg = "TALKER_CP runs its batch through the matrix-core GEMM, built for 8-bit affine weights only";
        return TSD_ERR_UNSUPPORTED;
    }
    if (c->batch < 1 || c->batch > MM_ROWS) {
        msg = "TALKER_CP batch must be 1.." + std::to_string(MM_ROWS);
        return TSD_ERR_UNSUPPORTED;
    }
    if (c->n_codebooks < 2 || c->n_codebooks > 16 || c->cp_n_layer <= 0 || c->cp_vocab <= 0) {
        msg = "TALKER_CP needs 2..16 codebooks, cp_n_layer >= 1 and cp_vocab >= 1";
        return TSD_ERR_INVALID_ARGUMENT;
    }
    if (c->head_dim != 64 && c->head_dim != 128) {
        msg = "head_dim must be 64 or 128";
        return TSD_ERR_UNSUPPORTED;
    }
    const int qd = c->n_head * c->head_dim;
    for (int K : {c->d_model, c->d_ff, qd})
        if (K > MM_MAX_K) {
            msg = "reduction dimension " + std::to_string(K) + " exceeds " + std::to_string(MM_MAX_K);
            return TSD_ERR_UNSUPPORTED;
        }
    return TSD_OK;
}

void talker_canonical_sizes(const tsd_config* c, size_t (*matrix_bytes)(int, int, int), std::vector<size_t>& sz)
{
    const int d = c->d_model, ff = c->d_ff, f = c->wfmt, qd = c->n_head * c->head_dim, kd = c->n_kv_head * c->head_dim;
    auto F32 = [&](size_t n) { sz.push_back(n * 4); };
    auto MAT = [&](int N, int K) { sz.push_back(matrix_bytes(f, N, K)); };
    auto layers = [&](int n) {
        for (int l = 0; l < n; ++l) {
            F32(d); MAT(qd, d); MAT(kd, d); MAT(kd, d); MAT(d, qd);
            F32(d); MAT(ff, d); MAT(ff, d); MAT(d, ff);
        }
    };
    F32((size_t)c->vocab * d);
    for (int k = 1; k < c->n_codebooks; ++k) F32((size_t)c->cp_vocab * d);
    layers(c->n_layer);
    F32(d);
    MAT(c->vocab, d);
    layers(c->cp_n_layer);
    F32(d);
    for (int k = 1; k < c->n_codebooks; ++k) MAT(c->cp_vocab, d);
}

size_t talker_plan(tsd_model* m, const tsd_config* c, uint8_t* base)
{
    Planner P(base);
    const int d = c->d_model, H = c->n_head, Hk = c->n_kv_head, hd = c->head_dim, ff = c->d_ff, B = c->batch;
    const int C = c->n_codebooks, V = c->vocab, Vc = c->cp_vocab;
    const int qd = H * hd, kd = Hk * hd, vmax = std::max(V, Vc), kmax = std::max(d, std::max(qd, ff));
    const int rope_rows = std::max(c->n_ctx, C);
    int* pos = (int*)P.take(4 * sizeof(int));
    int* tok = (int*)P.take(sizeof(int) * B * C);
    int* hist = (int*)P.take(sizeof(int) * (size_t)c->n_ctx * B * C);
    uint32_t* ctl = (uint32_t*)P.take(sizeof(uint32_t) * 64);
    float* x = (float*)P.take(sizeof(float) * MM_ROWS * d);
    float* xc = (float*)P.take(sizeof(float) * MM_ROWS * d);
    __half* hi = (__half*)P.take(2 * (size_t)MM_ROWS * kmax);
    __half* lo = (__half*)P.take(2 * (size_t)MM_ROWS * kmax);
    float* q = (float*)P.take(sizeof(float) * MM_ROWS * qd);
    float* h = (float*)P.take(sizeof(float) * MM_ROWS * (size_t)ff);
    float* logits = (float*)P.take(sizeof(float) * (size_t)B * C * vmax);
    float* part = (float*)P.take(attn_part_bytes(B, H, c->n_ctx, hd));
    float2* rope = (float2*)P.take(sizeof(float2) * (size_t)rope_rows * (hd / 2));
    float* emb[16] = {};
    emb[0] = (float*)P.take(sizeof(float) * (size_t)V * d);
    for (int k = 1; k < C; ++k) emb[k] = (float*)P.take(sizeof(float) * (size_t)Vc * d);
    auto layers = [&](int n) {
        std::vector<TLayerW> Ls(n);
        for (TLayerW& w : Ls) {
            w.qkv = take_tiled(P, qd + 2 * kd, d);
            w.o = take_tiled(P, d, qd);
            w.fc = take_tiled(P, 2 * ff, d);
            w.down = take_tiled(P, d, ff);
            w.n1g = (float*)P.take(4 * d);
            w.n2g = (float*)P.take(4 * d);
        }
        return Ls;
    };
    std::vector<TLayerW> Lt = layers(c->n_layer);
    float* nfg = (float*)P.take(4 * d);
    TiledMat head = take_tiled(P, V, d);
    std::vector<TLayerW> Lc = layers(c->cp_n_layer);
    float* cp_nfg = (float*)P.take(4 * d);
    TiledMat cp_head[16] = {};
    for (int k = 1; k < C; ++k) cp_head[k] = take_tiled(P, Vc, d);
    const size_t kv_layer = (size_t)B * Hk * c->n_ctx * hd;
    const size_t ckv_layer = (size_t)B * Hk * C * hd;
    __half* kc = (__half*)P.take(2 * kv_layer * c->n_layer);
    __half* vc = (__half*)P.take(2 * kv_layer * c->n_layer);
    __half* ckc = (__half*)P.take(2 * ckv_layer * c->cp_n_layer);
    __half* cvc = (__half*)P.take(2 * ckv_layer * c->cp_n_layer);
    if (m && base) {
        m->pos = pos; m->dbg_pos = pos + 1; m->tok = tok; m->hist = hist; m->ctl = ctl;
        m->x = x; m->xc = xc; m->qkv = q; m->h = h; m->logits = logits; m->part = part;
        m->act.hi = hi; m->act.lo = lo;
        m->rope = rope; m->rope_rows = rope_rows;
        for (int k = 0; k < C; ++k) {
            m->emb[k] = emb[k];
            m->emb_rows[k] = k == 0 ? V : Vc;
        }
        m->Lt = Lt; m->nfg = nfg; m->t_head = head;
        m->Lc = Lc; m->cp_nfg = cp_nfg;
        for (int k = 0; k < 16; ++k) m->cp_head[k] = cp_head[k];
        m->kc = kc; m->vc = vc; m->kv_layer_elems = kv_layer;
        m->ckc = ckc; m->cvc = cvc; m->ckv_layer_elems = ckv_layer;
        m->tpp = C; m->vmax = vmax; m->qkv_rows = qd + 2 * kd;
    }
    return align256(P.off);
}

tsd_status talker_pack(tsd_model* m, const tsd_tensor* w)
{
    const tsd_config& c = m->c;
    const int d = c.d_model, H = c.n_head, Hk = c.n_kv_head, hd = c.head_dim, ff = c.d_ff, C = c.n_codebooks;
    hipStream_t st = m->st;
    int i = 0;
    auto cp = [&](const void* dst, int idx) {
        return hipMemcpyAsync((void*)dst, w[idx].ptr, w[idx].bytes, hipMemcpyDeviceToDevice, st);
    };
    auto pk = [&](const TiledMat& dst, int idx, int N, int K, int row0, int mode) {
        return launch_pack_tiled(w[idx].ptr, N, K, (void*)dst.q, dst.N, row0, mode, hd, st);
    };
    for (int k = 0; k < C; ++k) HIP_TRY(m, cp(m->emb[k], i++), "copy embedding");
    auto layers = [&](std::vector<TLayerW>& Ls) -> tsd_status {
        for (TLayerW& L : Ls) {
            HIP_TRY(m, cp(L.n1g, i++), "copy");
            HIP_TRY(m, pk(L.qkv, i++, H * hd, d, 0, PACK_ROPE_PAIRS), "pack q");
            HIP_TRY(m, pk(L.qkv, i++, Hk * hd, d, H * hd, PACK_ROPE_PAIRS), "pack k");
            HIP_TRY(m, pk(L.qkv, i++, Hk * hd, d, (H + Hk) * hd, PACK_IDENTITY), "pack v");
            HIP_TRY(m, pk(L.o, i++, d, H * hd, 0, PACK_IDENTITY), "pack o");
            HIP_TRY(m, cp(L.n2g, i++), "copy");
            HIP_TRY(m, pk(L.fc, i++, ff, d, 0, PACK_INTERLEAVE_EVEN), "pack gate");
            HIP_TRY(m, pk(L.fc, i++, ff, d, 0, PACK_INTERLEAVE_ODD), "pack up");
            HIP_TRY(m, pk(L.down, i++, d, ff, 0, PACK_IDENTITY), "pack down");
        }
        return TSD_OK;
    };
    tsd_status s = layers(m->Lt);
    if (s != TSD_OK) return s;
    HIP_TRY(m, cp(m->nfg, i++), "copy");
    HIP_TRY(m, pk(m->t_head, i++, c.vocab, d, 0, PACK_IDENTITY), "pack head");
    s = layers(m->Lc);
    if (s != TSD_OK) return s;
    HIP_TRY(m, cp(m->cp_nfg, i++), "copy");
    for (int k = 1; k < C; ++k) HIP_TRY(m, pk(m->cp_head[k], i++, c.cp_vocab, d, 0, PACK_IDENTITY), "pack predictor head");
    // operand rows past the batch are read by the GEMM and must stay finite: zero everything once
    const int kmax = std::max(d, std::max(H * hd, ff));
    HIP_TRY(m, launch_fill_u32((unsigned*)m->act.hi, 0u, MM_ROWS * kmax / 2, st), "init");
    HIP_TRY(m, launch_fill_u32((unsigned*)m->act.lo, 0u, MM_ROWS * kmax / 2, st), "init");
    HIP_TRY(m, launch_fill_f32(m->x, 0.f, (size_t)MM_ROWS * d, st), "init");
    HIP_TRY(m, launch_fill_f32(m->xc, 0.f, (size_t)MM_ROWS * d, st), "init");
    return TSD_OK;
}

hipError_t talker_enqueue(tsd_model* m, hipStream_t st, bool with_cp, Probe* pr)
{
    const tsd_config& c = m->c;
    const int d = c.d_model, B = c.batch, C = c.n_codebooks;
    EmbedTabs T{};
    for (int k = 0; k < C; ++k) {
        T.tab[k] = m->emb[k];
        T.rows[k] = m->emb_rows[k];
    }
    TRY(launch_embed_sum16(T, m->tok, C, C, d, m->x, B, st));
    for (int l = 0; l < c.n_layer; ++l)
        TRY(layer16(m, m->Lt[l], m->x, m->kc + m->kv_layer_elems * l, m->vc + m->kv_layer_elems * l, c.n_ctx, m->pos, 0,
                    st, pr));
    if (!with_cp) return launch_frame_done(m->tok, 0, m->hist, m->pos, st);   // advance the position only
    // code 0; the Talker's final-normed hidden state is the predictor's position 0
    TRY(head16(m, st, pr, m->x, m->nfg, m->t_head, 0, c.vocab, m->xc));
    for (int cpos = 0; cpos < C; ++cpos) {
        Gather g{};
        if (cpos > 0) g = Gather{m->emb[cpos - 1], m->emb_rows[cpos - 1], m->tok + (cpos - 1)};
        for (int l = 0; l < c.cp_n_layer; ++l)
            TRY(layer16(m, m->Lc[l], m->xc, m->ckc + m->ckv_layer_elems * l, m->cvc + m->ckv_layer_elems * l, C,
                        nullptr, cpos, st, pr, (cpos > 0 && l == 0) ? &g : nullptr));
        if (cpos > 0) TRY(head16(m, st, pr, m->xc, m->cp_nfg, m->cp_head[cpos], cpos, c.cp_vocab, nullptr));
    }
    return launch_frame_done(m->tok, B * C, m->hist, m->pos, st);
}

hipError_t talker_layer(tsd_model* m, int l, hipStream_t st, const int* pos)
{
    const tsd_config& c = m->c;
    return layer16(m, m->Lt[l], m->x, m->kc + m->kv_layer_elems * l, m->vc + m->kv_layer_elems * l, c.n_ctx, pos, 0, st,
                   nullptr);
}

void talker_kind_launches(const tsd_model* m, int* out)
{
    const tsd_config& c = m->c;
    const int per_layer = c.n_layer + c.n_codebooks * c.cp_n_layer;
    for (int k : {KIND_QKV, KIND_ATTN, KIND_OPROJ, KIND_FC, KIND_DOWN}) out[k] = per_layer;
    out[KIND_HEAD] = c.n_codebooks;
    out[KIND_STEP] = 0;
}

}  // namespace tsd
