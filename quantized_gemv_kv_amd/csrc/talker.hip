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
//   QKV GEMM (the first norm applied to its results; RoPE and the fp16 K/V append in its
//   epilogue) -> attention (a cache of up to 512 positions is covered by one workgroup per head
//   and row, which writes the next operand itself; longer Talker caches are split and merged by
//   a small kernel) -> O-proj GEMM adding into the
//   residual and writing the second norm's input -> gate/up GEMM (norm applied, SwiGLU
//   epilogue writing the next operand) -> down GEMM adding into the residual and writing the
//   next layer's norm input: five launches per layer (six with a merge).
// The O and down projections have few 16-row tiles and a long K: up to sixteen waves of one
// workgroup share the K range, so every result has a single writer and adds deterministically.
// The sampler of each head also prepares the predictor's next input row.
#include <algorithm>
#include <string>

#include "model.h"
#include "prefill.h"

namespace tsd {
namespace {

#define TRY(expr)                            \
    do {                                     \
        hipError_t e_ = (expr);              \
        if (e_ != hipSuccess) return e_;     \
    } while (0)

// One LLAMA-shaped layer on the residual stream x (il_x rows) whose cache (kc, vc: [rows][Hkv]
// [n_ctx][hd]) gets slot pos = *posp (Talker) or pos_value (predictor).  On entry act2 holds
// hi/lo of x * n1g with n_ssq partial row sums of x^2 in ssq; on exit the same for the next norm,
// whose gain is g_after.
hipError_t layer16(tsd_model* m, const TLayerW& w, float* x, int n_ssq, const float* g_after, __half* kc, __half* vc,
                   int n_ctx, const int* posp, int pos_value, hipStream_t st, Probe* pr, int fuse_idx)
{
    const tsd_config& c = m->c;
    const int d = c.d_model, H = c.n_head, Hk = c.n_kv_head, hd = c.head_dim, B = c.batch;
    const int tiles_d = (d + 15) / 16;
    // norm + fused QKV, RoPE and the K/V append
    MmIn iq{};
    iq.a = m->act2;
    iq.ssq = m->ssq;
    iq.n_ssq = n_ssq;
    iq.eps = c.norm_eps;
    iq.rows = B;
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
    // attention; a cache of one chunk writes the output projection's operand directly
    const bool direct = attn_direct_fits(n_ctx);
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
    if (fuse_idx >= 0 && m->frame_fused && qkv_attention_fits(w.qkv, aa)) {
        // the product and the attention in one launch (the query and the new key and value cross
        // through exchange words tagged for this launch)
        oq.xq = m->xbuf;
        oq.ldx = w.qkv.N;
        oq.xctr = m->ctl + CTL_EPOCH;
        oq.xidx = fuse_idx;
        Bracket br(pr, KIND_QKV, st);
        TRY(launch_qkv_attention(w.qkv, iq, oq, aa, STEP_SPIN_LIMIT, m->ctl + CTL_ABORT, st));
    } else {
        {
            Bracket br(pr, KIND_QKV, st);
            TRY(launch_mm16(MM_QKV_ROPE, w.qkv, iq, 1, oq, st));
        }
        {
            Bracket br(pr, KIND_ATTN, st);
            TRY(launch_attention(aa, st));
        }
        if (!direct) TRY(launch_merge16(m->part, B, H, hd, attn_max_split(n_ctx), posp, pos_value + 1, m->act, st));
    }
    // output projection into the residual, which also prepares the second norm's input
    MmIn ia{};
    ia.a = m->act;
    ia.rows = B;
    Mm16Out orr{};
    orr.y = x;
    orr.rows = B;
    orr.next = m->act2;
    orr.g_next = w.n2g;
    orr.ssq_out = m->ssq;
    {
        Bracket br(pr, KIND_OPROJ, st);
        TRY(launch_mm16(MM_RESID, w.o, ia, 1, orr, st));
    }
    // norm + gate/up + SwiGLU, written as the down projection's operand
    MmIn ig{};
    ig.a = m->act2;
    ig.ssq = m->ssq;
    ig.n_ssq = tiles_d;
    ig.eps = c.norm_eps;
    ig.rows = B;
    Mm16Out of{};
    of.act = m->act;
    of.rows = B;
    {
        Bracket br(pr, KIND_FC, st);
        TRY(launch_mm16(MM_SWIGLU, w.fc, ig, 1, of, st));
    }
    // down projection into the residual, preparing the next norm's input
    orr.g_next = g_after;
    {
        Bracket br(pr, KIND_DOWN, st);
        TRY(launch_mm16(MM_RESID, w.down, ia, 1, orr, st));
    }
    return hipSuccess;
}

// final RMSNorm (act2 and ssq as left by the last layer) + head j into logits[b][j][..]
hipError_t head16(tsd_model* m, hipStream_t st, Probe* pr, const TiledMat& W, int j)
{
    const tsd_config& c = m->c;
    MmIn ih{};
    ih.a = m->act2;
    ih.ssq = m->ssq;
    ih.n_ssq = (c.d_model + 15) / 16;
    ih.eps = c.norm_eps;
    ih.rows = c.batch;
    Mm16Out oh{};
    oh.y = m->logits + (size_t)j * m->vmax;
    oh.ldy = c.n_codebooks * m->vmax;
    oh.rows = c.batch;
    oh.err = m->ctl + CTL_BAD_INPUT;
    Bracket br(pr, KIND_HEAD, st);
    return launch_mm16(MM_STORE, W, ih, 1, oh, st);
}

// code j of every row from head j's logits into tok[b][j], then the row's next input
hipError_t pick16(tsd_model* m, hipStream_t st, int j, int vocab, const RowPrep* prep)
{
    const tsd_config& c = m->c;
    PickArgs a{};
    a.logits = m->logits + (size_t)j * m->vmax;
    a.ld_l = c.n_codebooks * m->vmax;
    a.n = vocab;
    a.B = c.batch;
    a.draw = j == 0 ? m->draw : m->cp_draw;
    a.ch = j == 0 ? m->chain : m->cp_chain;
    a.seq = j == 0 ? m->seq : nullptr;   // the penalty and the consumed-token record: code 0 only
    a.seed = m->samp.seed;
    a.pass = j;
    a.posp = m->pos;
    a.code = m->tok + j;
    a.ld_code = c.n_codebooks;
    a.prep.src = -1;
    if (prep) a.prep = *prep;
    a.err = m->ctl + CTL_BAD_INPUT;
    return launch_pick(a, st);
}

// the predictor's input rows (xc, act2, ssq): an embedding row (id from codes, or the picked code)
RowPrep cp_input_emb(tsd_model* m, int table, const int* codes)
{
    const tsd_config& c = m->c;
    RowPrep p{};
    p.src = ROW_EMB;
    p.tab[0] = m->emb[table];
    p.tab_rows[0] = m->emb_rows[table];
    p.codes = codes;
    p.ld_codes = c.n_codebooks;
    p.n_tab = 1;
    p.K = c.d_model;
    p.B = c.batch;
    p.x = m->xc;
    p.act = m->act2;
    p.g = m->Lc[0].n1g;
    p.ssq = m->ssq;
    return p;
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
    int* seq = (int*)P.take(sizeof(int) * (size_t)c->n_ctx * B);
    uint32_t* ctl = (uint32_t*)P.take(sizeof(uint32_t) * 64);
    float* x = (float*)P.take(sizeof(float) * MM_ROWS * d);
    float* xc = (float*)P.take(sizeof(float) * MM_ROWS * d);
    __half* hi = (__half*)P.take(2 * (size_t)MM_ROWS * kmax);
    __half* lo = (__half*)P.take(2 * (size_t)MM_ROWS * kmax);
    __half* hi2 = (__half*)P.take(2 * (size_t)MM_ROWS * kmax);
    __half* lo2 = (__half*)P.take(2 * (size_t)MM_ROWS * kmax);
    float* ssq = (float*)P.take(sizeof(float) * MM_MAX_SSQ * MM_ROWS);
    float* q = (float*)P.take(sizeof(float) * MM_ROWS * qd);
    float* h = (float*)P.take(sizeof(float) * MM_ROWS * (size_t)ff);
    float* logits = (float*)P.take(sizeof(float) * (size_t)B * C * vmax);
    float* part = (float*)P.take(attn_part_bytes(B, H, c->n_ctx, hd));
    float2* rope = (float2*)P.take(sizeof(float2) * (size_t)rope_rows * (hd / 2));
    // exchange words of the fused QKV + attention launches (one row of q, k, v per batch row)
    const size_t xwords = (size_t)MM_ROWS * (qd + 2 * kd);
    uint64_t* xq = (uint64_t*)P.take(sizeof(uint64_t) * xwords);
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
    // prompt pass rows (row-major, batch rows x positions)
    const int pf_rows = (int)std::min<long long>(PF_MAX_ROWS, ((long long)B * c->n_ctx + PF_TILE - 1) / PF_TILE * PF_TILE);
    const int amax = std::max(d, qd);
    float* pf_x = (float*)P.take(sizeof(float) * (size_t)pf_rows * d);
    float* pf_q = (float*)P.take(sizeof(float) * (size_t)pf_rows * qd);
    __half* pf_ahi = (__half*)P.take(2 * (size_t)pf_rows * amax);
    __half* pf_alo = (__half*)P.take(2 * (size_t)pf_rows * amax);
    __half* pf_hhi = (__half*)P.take(2 * (size_t)pf_rows * ff);
    __half* pf_hlo = (__half*)P.take(2 * (size_t)pf_rows * ff);
    const size_t kv_layer = (size_t)B * Hk * c->n_ctx * hd;
    const size_t ckv_layer = (size_t)B * Hk * C * hd;
    __half* kc = (__half*)P.take(2 * kv_layer * c->n_layer);
    __half* vc = (__half*)P.take(2 * kv_layer * c->n_layer);
    __half* ckc = (__half*)P.take(2 * ckv_layer * c->cp_n_layer);
    __half* cvc = (__half*)P.take(2 * ckv_layer * c->cp_n_layer);
    if (m && base) {
        m->pos = pos; m->dbg_pos = pos + 1; m->tok = tok; m->hist = hist; m->seq = seq; m->ctl = ctl;
        m->x = x; m->xc = xc; m->qkv = q; m->h = h; m->logits = logits; m->part = part;
        m->act.hi = hi; m->act.lo = lo; m->act2.hi = hi2; m->act2.lo = lo2; m->ssq = ssq;
        m->rope = rope; m->rope_rows = rope_rows;
        m->xbuf = xq; m->xbuf_words = xwords;
        // every fused launch of a frame needs its own epoch
        m->frame_fused = c->n_layer + c->n_codebooks * c->cp_n_layer <= FUSE_EPOCHS - 1;
        m->max_launches = 0xFFFFFFFFull / FUSE_EPOCHS - 2;
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
        m->pf_rows = pf_rows;
        m->pf_x = pf_x; m->pf_q = pf_q; m->pf_ahi = pf_ahi; m->pf_alo = pf_alo; m->pf_hhi = pf_hhi; m->pf_hlo = pf_hlo;
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
    for (__half* a : {m->act.hi, m->act.lo, m->act2.hi, m->act2.lo})
        HIP_TRY(m, launch_fill_u32((unsigned*)a, 0u, MM_ROWS * kmax / 2, st), "init");
    HIP_TRY(m, launch_fill_f32(m->ssq, 0.f, (size_t)MM_MAX_SSQ * MM_ROWS, st), "init");
    HIP_TRY(m, launch_fill_f32(m->x, 0.f, (size_t)MM_ROWS * d, st), "init");
    HIP_TRY(m, launch_fill_f32(m->xc, 0.f, (size_t)MM_ROWS * d, st), "init");
    return TSD_OK;
}

hipError_t talker_enqueue(tsd_model* m, hipStream_t st, bool with_cp, Probe* pr)
{
    const tsd_config& c = m->c;
    const int d = c.d_model, B = c.batch, C = c.n_codebooks, L = c.n_layer, Lc = c.cp_n_layer;
    const int tiles_d = (d + 15) / 16;
    // the Talker's input: the sum of the frame's code embeddings
    RowPrep e{};
    e.src = ROW_EMB;
    for (int k = 0; k < C; ++k) {
        e.tab[k] = m->emb[k];
        e.tab_rows[k] = m->emb_rows[k];
    }
    e.codes = m->tok;
    e.ld_codes = C;
    e.n_tab = C;
    e.K = d;
    e.B = B;
    e.x = m->x;
    e.act = m->act2;
    e.g = m->Lt[0].n1g;
    e.ssq = m->ssq;
    TRY(launch_row_prep(e, st));
    int n_ssq = 1;
    for (int l = 0; l < L; ++l) {
        TRY(layer16(m, m->Lt[l], m->x, n_ssq, l + 1 < L ? m->Lt[l + 1].n1g : m->nfg, m->kc + m->kv_layer_elems * l,
                    m->vc + m->kv_layer_elems * l, c.n_ctx, m->pos, 0, st, pr, l));
        n_ssq = tiles_d;
    }
    if (!with_cp)   // advance the position and record the consumed code 0 only
        return launch_frame_done(m->tok, 0, m->hist, m->pos, m->seq, c.batch, c.n_codebooks, m->ctl + CTL_BAD_INPUT,
                                 m->ctl + CTL_EPOCH, st);
    // code 0; the Talker's final-normed hidden state is the predictor's position 0
    TRY(head16(m, st, pr, m->t_head, 0));
    RowPrep h{};
    h.src = ROW_NORMED;
    h.rows_src = m->x;
    h.g_src = m->nfg;
    h.eps = c.norm_eps;
    h.K = d;
    h.B = B;
    h.x = m->xc;
    h.act = m->act2;
    h.g = m->Lc[0].n1g;
    h.ssq = m->ssq;
    TRY(pick16(m, st, 0, c.vocab, &h));
    for (int cpos = 0; cpos < C; ++cpos) {
        if (cpos == 1) {   // position 1 consumes E_0(c_0)
            const RowPrep p = cp_input_emb(m, 0, m->tok);
            TRY(launch_row_prep(p, st));
        }
        n_ssq = 1;
        for (int l = 0; l < Lc; ++l) {
            TRY(layer16(m, m->Lc[l], m->xc, n_ssq, l + 1 < Lc ? m->Lc[l + 1].n1g : m->cp_nfg,
                        m->ckc + m->ckv_layer_elems * l, m->cvc + m->ckv_layer_elems * l, C, nullptr, cpos, st, pr,
                        L + cpos * Lc + l));
            n_ssq = tiles_d;
        }
        if (cpos == 0) continue;
        TRY(head16(m, st, pr, m->cp_head[cpos], cpos));
        // code cpos, and position cpos + 1's input E_cpos(c_cpos)
        const RowPrep p = cp_input_emb(m, cpos, nullptr);
        TRY(pick16(m, st, cpos, c.cp_vocab, cpos + 1 < C ? &p : nullptr));
    }
    return launch_frame_done(m->tok, B * C, m->hist, m->pos, nullptr, B, C, m->ctl + CTL_BAD_INPUT, m->ctl + CTL_EPOCH, st);
}

hipError_t talker_layer(tsd_model* m, int l, hipStream_t st, const float* d_x, const int* pos)
{
    const tsd_config& c = m->c;
    RowPrep p{};
    p.src = ROW_MAJOR;
    p.rows_src = d_x;
    p.K = c.d_model;
    p.B = c.batch;
    p.x = m->x;
    p.act = m->act2;
    p.g = m->Lt[l].n1g;
    p.ssq = m->ssq;
    TRY(launch_row_prep(p, st));
    TRY(layer16(m, m->Lt[l], m->x, 1, m->Lt[l].n1g, m->kc + m->kv_layer_elems * l, m->vc + m->kv_layer_elems * l,
                c.n_ctx, pos, 0, st, nullptr, 0));
    return launch_bump_u32(m->ctl + CTL_EPOCH, st);   // the next launch tags its words anew
}

void talker_kind_launches(const tsd_model* m, int* out)
{
    const tsd_config& c = m->c;
    const int per_layer = c.n_layer + c.n_codebooks * c.cp_n_layer;
    for (int k : {KIND_QKV, KIND_ATTN, KIND_OPROJ, KIND_FC, KIND_DOWN}) out[k] = per_layer;
    if (m->frame_fused) out[KIND_ATTN] = 0;   // the attention runs inside the QKV launches
    out[KIND_HEAD] = c.n_codebooks;
    out[KIND_STEP] = 0;
}

}  // namespace tsd
