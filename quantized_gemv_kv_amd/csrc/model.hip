// model.hip — the decode-step executor behind the C ABI (include/tsd.h).
//
// At creation: validate the shape, plan the caller's workspace, repack every canonical weight
// into the kernel layout (fusing Q/K/V rows, pairing RoPE rows, interleaving gate/up rows),
// then record the whole step — every layer's kernels, the head and the sampler — into one HIP
// graph.  A step is then a single graph launch: the position, the input token and the sampled
// id live in device memory and are advanced by the graph itself, so one instantiated graph
// replays every step with no host work beyond the launch ("Chatterbox -> ggml Port:
// Development Journal", §3.8 graph reuse and §3.22 no per-step allocator work; "Every Frame Is
// a Memory Read", §5.2: the random state and the sampled ids stay inside the compiled graph).
#include <math.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "model.h"
#include "prefill.h"

using namespace tsd;

namespace tsd {

thread_local std::string g_err;

tsd_status fail(tsd_model* m, tsd_status s, const std::string& msg)
{
    if (m) m->err = msg;
    else g_err = msg;
    return s;
}

tsd_status hip_fail(tsd_model* m, hipError_t e, const char* what)
{
    return fail(m, TSD_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

int group_of(int f) { return f == TSD_W_AFFINE8_G64 || f == TSD_W_AFFINE4_G64 ? 64 : 32; }

size_t canonical_matrix_bytes(int f, int N, int K)
{
    if (f == TSD_W_Q4_0) return (size_t)N * (K / 32) * 18;
    if (f == TSD_W_Q8_0) return (size_t)N * (K / 32) * 34;
    if (f == TSD_W_Q5_0) return (size_t)N * (K / 32) * 22;
    if (f == TSD_W_AFFINE4_G64 || f == TSD_W_AFFINE4_G32) return (size_t)N * K / 2 + (size_t)N * (K / group_of(f)) * 4;
    return (size_t)N * K + (size_t)N * (K / 64) * 4;
}

}  // namespace tsd

namespace {

constexpr int MAX_STEP_WG = 1024;          // workgroups of the persistent step, at most

bool known_format(int f) { return f >= 0 && f < FMT_COUNT; }

tsd_status validate(const tsd_config* c, std::string& msg)
{
    if (!c) { msg = "null config"; return TSD_ERR_INVALID_ARGUMENT; }
    if (c->arch < 0 || c->arch > 2 || !known_format(c->wfmt)) { msg = "unknown arch or weight format"; return TSD_ERR_INVALID_ARGUMENT; }
    if (c->n_layer <= 0 || c->d_model <= 0 || c->n_head <= 0 || c->n_kv_head <= 0 || c->head_dim <= 0 || c->d_ff <= 0 ||
        c->vocab <= 0 || c->n_ctx <= 0 || c->batch <= 0 || c->n_head % c->n_kv_head) {
        msg = "dimensions must be positive and n_head a multiple of n_kv_head";
        return TSD_ERR_INVALID_ARGUMENT;
    }
    if (c->arch == TSD_ARCH_GPT2 && (c->n_head * c->head_dim != c->d_model || c->n_kv_head != c->n_head)) {
        msg = "GPT2 needs n_head*head_dim == d_model and n_kv_head == n_head";
        return TSD_ERR_INVALID_ARGUMENT;
    }
    const int g = group_of(c->wfmt);
    const int qd = c->n_head * c->head_dim;
    if (c->d_model % g || c->d_ff % g || qd % g) {
        msg = "every reduction dimension (d_model, d_ff, n_head*head_dim) must be a multiple of the quant block (" +
              std::to_string(g) + ")";
        return TSD_ERR_INVALID_ARGUMENT;
    }
    if (c->arch == TSD_ARCH_TALKER_CP) return talker_validate(c, msg);
    if (c->batch != 1 && c->batch != 2) { msg = "GPT2/LLAMA decode supports batch 1 or 2"; return TSD_ERR_UNSUPPORTED; }
    if (c->head_dim != 64 && c->head_dim != 128) { msg = "head_dim must be 64 or 128"; return TSD_ERR_UNSUPPORTED; }
    for (int K : {c->d_model, c->d_ff, qd})
        if (K > 4096 || !gemv_shape_ok(c->wfmt, K)) {
            msg = "reduction dimension " + std::to_string(K) + " has no GEMV lane mapping";
            return TSD_ERR_UNSUPPORTED;
        }
    return TSD_OK;
}

int n_weights_of(const tsd_config* c)
{
    if (c->arch == TSD_ARCH_GPT2) return 2 + 12 * c->n_layer + 3;
    if (c->arch == TSD_ARCH_LLAMA) return 1 + 9 * c->n_layer + 2;
    return c->n_codebooks + 9 * c->n_layer + 2 + 9 * c->cp_n_layer + 1 + (c->n_codebooks - 1);
}

// expected canonical sizes in order; kinds: 0 fp32 tensor, 1 matrix
void canonical_sizes(const tsd_config* c, std::vector<size_t>& sz)
{
    if (c->arch == TSD_ARCH_TALKER_CP) return talker_canonical_sizes(c, canonical_matrix_bytes, sz);
    const int d = c->d_model, ff = c->d_ff, f = c->wfmt, qd = c->n_head * c->head_dim, kd = c->n_kv_head * c->head_dim;
    auto F32 = [&](size_t n) { sz.push_back(n * 4); };
    auto MAT = [&](int N, int K) { sz.push_back(canonical_matrix_bytes(f, N, K)); };
    if (c->arch == TSD_ARCH_GPT2) {
        F32((size_t)c->vocab * d);
        F32((size_t)c->n_ctx * d);
        for (int l = 0; l < c->n_layer; ++l) {
            F32(d); F32(d); MAT(3 * d, d); F32(3 * d); MAT(d, d); F32(d);
            F32(d); F32(d); MAT(ff, d); F32(ff); MAT(d, ff); F32(d);
        }
        F32(d); F32(d); MAT(c->vocab, d);
    } else {
        F32((size_t)c->vocab * d);
        for (int l = 0; l < c->n_layer; ++l) {
            F32(d); MAT(qd, d); MAT(kd, d); MAT(kd, d); MAT(d, qd);
            F32(d); MAT(ff, d); MAT(ff, d); MAT(d, ff);
        }
        F32(d); MAT(c->vocab, d);
    }
}

// walk the workspace; with base == nullptr it only sizes it
size_t plan(tsd_model* m, const tsd_config* c, uint8_t* base)
{
    if (c->arch == TSD_ARCH_TALKER_CP) return talker_plan(m, c, base);
    Planner P(base);
    const int d = c->d_model, H = c->n_head, Hk = c->n_kv_head, hd = c->head_dim, ff = c->d_ff, B = c->batch, f = c->wfmt;
    const int tpp = 1, vmax = c->vocab;
    const int qkv_rows = (H + 2 * Hk) * hd;
    // step state
    int* pos = (int*)P.take(4 * sizeof(int));
    int* tok = (int*)P.take(sizeof(int) * B * tpp);
    const int head_blocks = (c->vocab + gemv_rows_per_block(f, d, EPI_HEAD_ARGMAX) - 1) / gemv_rows_per_block(f, d, EPI_HEAD_ARGMAX);
    unsigned long long* best = (unsigned long long*)P.take(sizeof(unsigned long long) * B * tpp * head_blocks);
    int* hist = (int*)P.take(sizeof(int) * (size_t)c->n_ctx * B * tpp);
    int* seq = (int*)P.take(sizeof(int) * (size_t)c->n_ctx * B);
    // activations
    float* x = (float*)P.take(sizeof(float) * B * d);
    float* qkv = (float*)P.take(sizeof(float) * B * qkv_rows);
    float* attn = (float*)P.take(sizeof(float) * B * H * hd);
    float* h = (float*)P.take(sizeof(float) * B * (size_t)ff);
    float* logits = (float*)P.take(sizeof(float) * (size_t)B * tpp * vmax);
    float* part = (float*)P.take(attn_part_bytes(B, H, c->n_ctx, hd));
    float2* rope = (float2*)P.take(sizeof(float2) * (size_t)c->n_ctx * (hd / 2));
    // embeddings
    float* emb0 = (float*)P.take(sizeof(float) * (size_t)c->vocab * d);
    float* wpe = c->arch == TSD_ARCH_GPT2 ? (float*)P.take(sizeof(float) * (size_t)c->n_ctx * d) : nullptr;
    // layers
    std::vector<LayerW> Ls(c->n_layer);
    for (int l = 0; l < c->n_layer; ++l) {
        LayerW& w = Ls[l];
        if (c->arch == TSD_ARCH_GPT2) {
            w.qkv = take_mat(P, f, 3 * d, d);
            w.o = take_mat(P, f, d, d);
            w.fc = take_mat(P, f, ff, d);
            w.down = take_mat(P, f, d, ff);
            w.n1g = (float*)P.take(4 * d); w.n1b = (float*)P.take(4 * d);
            w.n2g = (float*)P.take(4 * d); w.n2b = (float*)P.take(4 * d);
            w.bqkv = (float*)P.take(4 * 3 * d); w.bo = (float*)P.take(4 * d);
            w.bfc = (float*)P.take(4 * (size_t)ff); w.bdown = (float*)P.take(4 * d);
            w.cqkv = (float*)P.take(4 * 3 * d); w.dqkv = (float*)P.take(4 * 3 * d);
            w.cfc = (float*)P.take(4 * (size_t)ff); w.dfc = (float*)P.take(4 * (size_t)ff);
        } else {
            w.qkv = take_mat(P, f, qkv_rows, d);
            w.o = take_mat(P, f, d, H * hd);
            w.fc = take_mat(P, f, 2 * ff, d);
            w.down = take_mat(P, f, d, ff);
            w.n1g = (float*)P.take(4 * d);
            w.n2g = (float*)P.take(4 * d);
        }
    }
    float* nfg = (float*)P.take(4 * d);
    float* nfb = c->arch == TSD_ARCH_GPT2 ? (float*)P.take(4 * d) : nullptr;
    PackedMat head = take_mat(P, f, c->vocab, d);
    float* hc = c->arch == TSD_ARCH_GPT2 ? (float*)P.take(4 * (size_t)c->vocab) : nullptr;
    float* hdv = c->arch == TSD_ARCH_GPT2 ? (float*)P.take(4 * (size_t)c->vocab) : nullptr;
    const size_t kv_layer = (size_t)B * Hk * c->n_ctx * hd;
    __half* kc = (__half*)P.take(2 * kv_layer * c->n_layer);
    __half* vc = (__half*)P.take(2 * kv_layer * c->n_layer);
    // persistent step: layer table, control words, exchange words
    uint32_t* ctl = (uint32_t*)P.take(sizeof(uint32_t) * 64);
    StepArgs* d_sa = (StepArgs*)P.take(sizeof(StepArgs));
    const size_t n_part = (size_t)H * step_max_split(c->n_ctx) * (hd + STEP_PART_PAD);
    // one batch row's words of each buffer (rounded up as below); a buffer holds B rows
    const size_t dsh = (size_t)d + STEP_SHIFT_COPIES * STEP_SHIFT_STRIDE;   // residual words + the shift's copies
    const size_t xw[8] = {(size_t)qkv_rows, n_part, dsh, (size_t)ff, dsh, 2 * (size_t)MAX_STEP_WG, (size_t)vmax, (size_t)H * hd};
    size_t xrs[8], xtot = 0;
    // Placement (measured, same-box A/B): every buffer in a region of its own that starts at a
    // 64 KB boundary of the device address space, 4 KB times its index further on, with each
    // batch row of a buffer at a 4 KB boundary plus 256 bytes.  Against rows packed at 256-byte
    // steps from wherever the weights end, the 64 KB start and the 4 KB rows took C3 293.8 ->
    // 289.6 us per step and C4 420.1 -> 415.7 us; the regions keep a buffer's place independent
    // of the other buffers' sizes.
    // The polls of a phase go to the memory-side cache, whose slice follows the address, so
    // where the polled lines sit decides how they queue.
    constexpr size_t XREG = 8192;   // 64 KB in words
    static const size_t XSKEW[8] = {0, 512, 1024, 1536, 2048, 2560, 3072, 3584};
    size_t xoff[8];
    for (int i = 0; i < 8; ++i) {
        xrs[i] = ((xw[i] + 511) & ~(size_t)511) + 32;
        xoff[i] = xtot + XSKEW[i];
        xtot = (xoff[i] + xrs[i] * B + XREG - 1) / XREG * XREG;
    }
    P.align_abs(65536);
    uint64_t* xbuf = (uint64_t*)P.take(sizeof(uint64_t) * xtot);
    // prompt pass rows
    const int pf_rows = (int)std::min<long long>(PF_MAX_ROWS, ((long long)B * c->n_ctx + PF_TILE - 1) / PF_TILE * PF_TILE);
    const int qd = H * hd, amax = std::max(d, qd);
    float* pf_x = (float*)P.take(sizeof(float) * (size_t)pf_rows * d);
    float* pf_q = (float*)P.take(sizeof(float) * (size_t)pf_rows * qd);
    __half* pf_ahi = (__half*)P.take(2 * (size_t)pf_rows * amax);
    __half* pf_alo = (__half*)P.take(2 * (size_t)pf_rows * amax);
    __half* pf_hhi = (__half*)P.take(2 * (size_t)pf_rows * ff);
    __half* pf_hlo = (__half*)P.take(2 * (size_t)pf_rows * ff);
    if (m && base) {
        m->pf_rows = pf_rows;
        m->pf_x = pf_x; m->pf_q = pf_q; m->pf_ahi = pf_ahi; m->pf_alo = pf_alo; m->pf_hhi = pf_hhi; m->pf_hlo = pf_hlo;
        m->pos = pos; m->dbg_pos = pos + 1; m->tok = tok; m->best = best;
        m->hist = hist; m->seq = seq; m->x = x; m->qkv = qkv; m->attn = attn; m->h = h; m->logits = logits; m->part = part;
        m->rope = rope; m->rope_rows = c->n_ctx; m->emb[0] = emb0; m->emb_rows[0] = c->vocab; m->wpe = wpe; m->L = Ls; m->nfg = nfg; m->nfb = nfb;
        m->hc = hc; m->hdv = hdv;
        m->head = head; m->kc = kc; m->vc = vc; m->kv_layer_elems = kv_layer; m->tpp = tpp; m->vmax = vmax;
        m->qkv_rows = qkv_rows;
        m->ctl = ctl;
        m->d_sa = d_sa;
        m->xbuf = xbuf;
        m->xbuf_words = xtot;
        uint64_t* xp[8];
        for (int i = 0; i < 8; ++i) xp[i] = xbuf + xoff[i];
        StepArgs& a = m->sa;
        a.x_qkv = xp[0]; a.x_part = xp[1]; a.x_attn = xp[2]; a.x_h = xp[3]; a.x_out = xp[4]; a.x_best = xp[5];
        a.x_logit = xp[6];
        a.xs_qkv = (long long)xrs[0]; a.xs_part = (long long)xrs[1]; a.xs_d = (long long)xrs[2]; a.xs_h = (long long)xrs[3];
        a.xs_best = (long long)xrs[5]; a.xs_logit = (long long)xrs[6];
        a.x_ao = xp[7]; a.xs_ao = (long long)xrs[7];
    }
    return align256(P.off);
}

// ---- the step's kernels --------------------------------------------------------------------

hipError_t enqueue_layer(tsd_model* m, int l, hipStream_t st, const int* pos, bool embed, Probe* pr = nullptr)
{
    const tsd_config& c = m->c;
    const int d = c.d_model, H = c.n_head, Hk = c.n_kv_head, hd = c.head_dim, B = c.batch;
    const LayerW& w = m->L[l];
    const bool gpt2 = c.arch == TSD_ARCH_GPT2;
    __half* kc = m->kc + m->kv_layer_elems * l;
    __half* vc = m->vc + m->kv_layer_elems * l;
    const long long kv_row = (long long)Hk * c.n_ctx * hd;   // one batch row's slab of a layer's cache
    hipError_t e;

    // norm + fused QKV (+bias | +RoPE) + K/V append
    ProArgs pa{};
    pa.src = m->x;
    pa.g = w.n1g;
    pa.beta = w.n1b;
    pa.eps = c.norm_eps;
    if (embed) {
        pa.n_emb = 1;
        pa.tab[0] = m->emb[0];
        pa.tab_rows[0] = m->emb_rows[0];
        pa.tok = m->tok;
        pa.pos_tab = m->wpe;
        pa.pos = pos;
        pa.x_out = m->x;
    }
    EpiArgs ea{};
    ea.bias = w.bqkv;
    ea.qrows = H * hd;
    ea.krows = Hk * hd;
    ea.hd = hd;
    ea.n_ctx = c.n_ctx;
    ea.q = m->qkv;
    ea.kc = kc;
    ea.vc = vc;
    ea.rope = m->rope;
    ea.pos = pos;
    pa.rs_src = d;
    pa.rs_tok = m->tpp;
    ea.rs_q = m->qkv_rows;
    ea.rs_kv = kv_row;
    const int pro = embed ? (gpt2 ? PRO_LN_EMB : PRO_RMS_EMB) : (gpt2 ? PRO_LN : PRO_RMS);
    {
        Bracket br(pr, KIND_QKV, st);
        e = launch_gemv(c.wfmt, pro, gpt2 ? EPI_QKV : EPI_QKV_ROPE, w.qkv, pa, ea, st, B);
    }
    if (e != hipSuccess) return e;

    // split-KV flash-decode over positions 0..pos
    AttnArgs aa{};
    aa.q = m->qkv;
    aa.ldq = m->qkv_rows;
    aa.k = kc;
    aa.v = vc;
    aa.out = m->attn;
    aa.ldo = H * hd;
    aa.part = m->part;
    aa.B = B;
    aa.H = H;
    aa.Hkv = Hk;
    aa.hd = hd;
    aa.n_ctx = c.n_ctx;
    aa.pos = pos;
    {
        Bracket br(pr, KIND_ATTN, st);
        e = launch_attention(aa, st);
    }
    if (e != hipSuccess) return e;

    // merge of the attention partials + output projection + bias + residual
    ProArgs po{};
    po.part = m->part;
    po.a_hd = hd;
    po.a_chunk = ATTN_CHUNK;
    po.a_max_split = (c.n_ctx + po.a_chunk - 1) / po.a_chunk;
    po.pos = pos;
    po.rs_part = (long long)H * po.a_max_split * (hd + 4);
    EpiArgs eo{};
    eo.y = m->x;
    eo.bias = w.bo;
    eo.rs_y = d;
    {
        Bracket br(pr, KIND_OPROJ, st);
        e = launch_gemv(c.wfmt, PRO_ATTN, EPI_RESID, w.o, po, eo, st, B);
    }
    if (e != hipSuccess) return e;

    // norm + FC (+bias, GELU) or gate/up (SwiGLU)
    ProArgs pf{};
    pf.src = m->x;
    pf.g = w.n2g;
    pf.beta = w.n2b;
    pf.eps = c.norm_eps;
    pf.rs_src = d;
    EpiArgs ef{};
    ef.y = m->h;
    ef.bias = w.bfc;
    ef.rs_y = c.d_ff;
    {
        Bracket br(pr, KIND_FC, st);
        e = launch_gemv(c.wfmt, gpt2 ? PRO_LN : PRO_RMS, gpt2 ? EPI_GELU : EPI_SWIGLU, w.fc, pf, ef, st, B);
    }
    if (e != hipSuccess) return e;

    // down projection + bias + residual
    ProArgs pd{};
    pd.src = m->h;
    pd.rs_src = c.d_ff;
    EpiArgs ed{};
    ed.y = m->x;
    ed.bias = w.bdown;
    ed.rs_y = d;
    Bracket br(pr, KIND_DOWN, st);
    return launch_gemv(c.wfmt, PRO_LOAD, EPI_RESID, w.down, pd, ed, st, B);
}

hipError_t enqueue_step(tsd_model* m, hipStream_t st, Probe* pr = nullptr)
{
    const tsd_config& c = m->c;
    if (c.arch == TSD_ARCH_TALKER_CP) return talker_enqueue(m, st, true, pr);
    if (m->step_fn) {
        Bracket br(pr, KIND_STEP, st);
        return launch_step(m->step_fn, m->d_sa, m->n_wg, st);
    }
    for (int l = 0; l < c.n_layer; ++l) {
        hipError_t e = enqueue_layer(m, l, st, m->pos, l == 0, pr);
        if (e != hipSuccess) return e;
    }
    ProArgs ph{};
    ph.src = m->x;
    ph.g = m->nfg;
    ph.beta = m->nfb;
    ph.eps = c.norm_eps;
    ph.rs_src = c.d_model;
    EpiArgs eh{};
    eh.y = m->logits;
    eh.ldy = c.vocab;
    eh.best = m->best;
    eh.err = m->ctl + CTL_BAD_INPUT;
    eh.rs_y = c.vocab;
    Bracket br(pr, KIND_HEAD, st);
    hipError_t e = launch_gemv(c.wfmt, c.arch == TSD_ARCH_GPT2 ? PRO_LN : PRO_RMS, EPI_HEAD_ARGMAX, m->head, ph, eh, st,
                               c.batch);
    if (e != hipSuccess) return e;
    if (m->draw) {
        SampleArgs s{};
        s.rows = c.batch;
        s.ld_logits = c.vocab;
        s.cfg = m->samp.cfg;
        s.cfg_weight = m->samp.cfg_weight;
        s.logits = m->logits;
        s.n = c.vocab;
        s.ch = m->chain;
        s.seed = m->samp.seed;
        s.posp = m->pos;
        s.out = m->tok;
        s.hist = m->hist;
        s.hist_stride = c.batch * m->tpp;
        s.seq = m->seq;
        s.seq_stride = c.batch;
        s.n_seq = -1;
        s.cur = m->tok;
        s.seq_out = m->seq;
        s.err = m->ctl + CTL_BAD_INPUT;
        return launch_sample(s, st);
    }
    const int nblk = (c.vocab + gemv_rows_per_block(c.wfmt, c.d_model, EPI_HEAD_ARGMAX) - 1) /
                     gemv_rows_per_block(c.wfmt, c.d_model, EPI_HEAD_ARGMAX);
    return launch_argmax_finalize(m->best, nblk, c.batch, m->tok, m->hist, m->seq, c.batch * m->tpp, m->pos,
                                  m->ctl + CTL_BAD_INPUT, st);
}

tsd_status pack_weights(tsd_model* m, const tsd_tensor* w)
{
    const tsd_config& c = m->c;
    if (c.arch == TSD_ARCH_TALKER_CP) return talker_pack(m, w);
    const int d = c.d_model, H = c.n_head, Hk = c.n_kv_head, hd = c.head_dim, ff = c.d_ff, f = c.wfmt;
    hipStream_t st = m->st;
    int i = 0;
    auto cp = [&](void* dst, int idx) { return hipMemcpyAsync(dst, w[idx].ptr, w[idx].bytes, hipMemcpyDeviceToDevice, st); };
    auto pk = [&](const PackedMat& dst, int idx, int N, int K, int row0, int mode) {
        return launch_pack(f, w[idx].ptr, N, K, (void*)dst.q, dst.N, row0, mode, hd, st);
    };
    HIP_TRY(m, cp((void*)m->emb[0], i++), "copy embedding");
    if (c.arch == TSD_ARCH_GPT2) HIP_TRY(m, cp((void*)m->wpe, i++), "copy positions");
    for (int l = 0; l < c.n_layer; ++l) {
        LayerW& L = m->L[l];
        if (c.arch == TSD_ARCH_GPT2) {
            HIP_TRY(m, cp(L.n1g, i++), "copy"); HIP_TRY(m, cp(L.n1b, i++), "copy");
            HIP_TRY(m, pk(L.qkv, i++, 3 * d, d, 0, PACK_IDENTITY), "pack qkv");
            HIP_TRY(m, cp(L.bqkv, i++), "copy");
            HIP_TRY(m, pk(L.o, i++, d, d, 0, PACK_IDENTITY), "pack o");
            HIP_TRY(m, cp(L.bo, i++), "copy");
            HIP_TRY(m, cp(L.n2g, i++), "copy"); HIP_TRY(m, cp(L.n2b, i++), "copy");
            HIP_TRY(m, pk(L.fc, i++, ff, d, 0, PACK_IDENTITY), "pack fc");
            HIP_TRY(m, cp(L.bfc, i++), "copy");
            HIP_TRY(m, pk(L.down, i++, d, ff, 0, PACK_IDENTITY), "pack down");
            HIP_TRY(m, cp(L.bdown, i++), "copy");
        } else {
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
    }
    HIP_TRY(m, cp(m->nfg, i++), "copy");
    if (c.arch == TSD_ARCH_GPT2) HIP_TRY(m, cp(m->nfb, i++), "copy");
    HIP_TRY(m, pk(m->head, i++, c.vocab, d, 0, PACK_IDENTITY), "pack head");
    if (c.arch == TSD_ARCH_GPT2) {
        // c = W g, d = W beta + bias for every LayerNorm-fed product (the persistent step's
        // deferred normalisation: LN(x) . W = r (W g (x - x0) - (mean - x0) c) + d)
        auto mv = [&](const PackedMat& W, const float* x, const float* bias, float* y) {
            ProArgs pa{};
            pa.src = x;
            EpiArgs ea{};
            ea.y = y;
            ea.bias = bias;
            return launch_gemv(f, PRO_LOAD, EPI_STORE, W, pa, ea, st);
        };
        for (int l = 0; l < c.n_layer; ++l) {
            const LayerW& L = m->L[l];
            HIP_TRY(m, mv(L.qkv, L.n1g, nullptr, L.cqkv), "layer-norm constants");
            HIP_TRY(m, mv(L.qkv, L.n1b, L.bqkv, L.dqkv), "layer-norm constants");
            HIP_TRY(m, mv(L.fc, L.n2g, nullptr, L.cfc), "layer-norm constants");
            HIP_TRY(m, mv(L.fc, L.n2b, L.bfc, L.dfc), "layer-norm constants");
        }
        HIP_TRY(m, mv(m->head, m->nfg, nullptr, m->hc), "layer-norm constants");
        HIP_TRY(m, mv(m->head, m->nfb, nullptr, m->hdv), "layer-norm constants");
    }
    return TSD_OK;
}

// zero every exchange word and the control words: epochs restart at 1, nothing stale can match
hipError_t reset_exchange(tsd_model* m)
{
    hipError_t e = launch_fill_u64((unsigned long long*)m->xbuf, 0ull, (int)m->xbuf_words, m->st);
    if (e == hipSuccess) e = launch_fill_u32(m->ctl + CTL_EPOCH, 0u, 2, m->st);   // epoch base and time-out word
    m->launches = 0;
    return e;
}

// choose the persistent step kernel and its grid; leaves step_fn null for one launch per operator
tsd_status setup_step(tsd_model* m)
{
    const tsd_config& c = m->c;
    if (c.launch_mode == TSD_LAUNCH_PER_OPERATOR) return TSD_OK;
    if (c.launch_mode != TSD_LAUNCH_PERSISTENT) return fail(m, TSD_ERR_INVALID_ARGUMENT, "unknown launch_mode");
    if (c.arch == TSD_ARCH_TALKER_CP) return TSD_OK;   // the frame runs one launch per operator
    m->step_fn = step_kernel_for(c.wfmt, c.arch == TSD_ARCH_LLAMA, c.d_model, c.n_head, c.n_kv_head, c.head_dim, c.d_ff,
                                 c.vocab, c.batch);
    if (!m->step_fn) return TSD_OK;   // this shape runs one launch per operator
    int dev = 0, n_cu = 0, per_cu = 0;
    HIP_TRY(m, hipGetDevice(&dev), "device");
    HIP_TRY(m, hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev), "CU count");
    HIP_TRY(m, hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, m->step_fn, 256, 0), "occupancy");
    // every workgroup must be resident at once (they wait on each other): at most what fits
    const int fit = n_cu * per_cu;
    int g = c.n_workgroups > 0 ? c.n_workgroups : n_cu;
    if (g > fit || g > MAX_STEP_WG)
        return fail(m, TSD_ERR_UNSUPPORTED, "n_workgroups " + std::to_string(g) + " exceeds the " +
                    std::to_string(fit < MAX_STEP_WG ? fit : MAX_STEP_WG) + " that can be resident at once");
    // every layer at one stride from the previous (the planner lays layers out identically)
    auto lay = [&](int l) {
        const LayerW& w = m->L[l];
        StepLayer t;
        t.qkv = w.qkv; t.o = w.o; t.fc = w.fc; t.down = w.down;
        t.n1g = w.n1g; t.n1b = w.n1b; t.n2g = w.n2g; t.n2b = w.n2b;
        t.bqkv = w.bqkv; t.bo = w.bo; t.bfc = w.bfc; t.bdown = w.bdown;
        t.cqkv = w.cqkv; t.dqkv = w.dqkv; t.cfc = w.cfc; t.dfc = w.dfc;
        t.kc = m->kc + m->kv_layer_elems * l;
        t.vc = m->vc + m->kv_layer_elems * l;
        return t;
    };
    const StepLayer L0 = lay(0);
    const long long stride = c.n_layer > 1 ? (const char*)m->L[1].qkv.q - (const char*)m->L[0].qkv.q : 0;
    auto same = [&](const void* p0, const void* pl, int l) {
        return p0 ? (const char*)pl == (const char*)p0 + stride * l : pl == nullptr;
    };
    for (int l = 1; l < c.n_layer; ++l) {
        const StepLayer t = lay(l);
        const void* a0[] = {L0.qkv.q, L0.qkv.s, L0.qkv.b, L0.o.q, L0.o.s, L0.o.b, L0.fc.q, L0.fc.s, L0.fc.b, L0.down.q,
                            L0.down.s, L0.down.b, L0.n1g, L0.n1b, L0.n2g, L0.n2b, L0.bqkv, L0.bo, L0.bfc, L0.bdown,
                            L0.cqkv, L0.dqkv, L0.cfc, L0.dfc};
        const void* al[] = {t.qkv.q, t.qkv.s, t.qkv.b, t.o.q, t.o.s, t.o.b, t.fc.q, t.fc.s, t.fc.b, t.down.q,
                            t.down.s, t.down.b, t.n1g, t.n1b, t.n2g, t.n2b, t.bqkv, t.bo, t.bfc, t.bdown,
                            t.cqkv, t.dqkv, t.cfc, t.dfc};
        for (size_t i = 0; i < sizeof(a0) / sizeof(a0[0]); ++i)
            if (!same(a0[i], al[i], l)) return fail(m, TSD_ERR_STATE, "layer tensors are not at a uniform stride");
    }
    m->n_wg = g;
    StepArgs& a = m->sa;
    a.L0 = L0;
    a.lstride = stride;
    a.kvstride = (long long)m->kv_layer_elems;
    a.n_layer = c.n_layer; a.H = c.n_head; a.Hk = c.n_kv_head; a.n_ctx = c.n_ctx; a.vocab = c.vocab;
    a.max_split = step_max_split(c.n_ctx);
    a.eps = c.norm_eps;
    a.emb = m->emb[0]; a.wpe = m->wpe; a.nfg = m->nfg; a.nfb = m->nfb; a.hc = m->hc; a.hdv = m->hdv; a.head = m->head; a.rope = m->rope;
    a.pos = m->pos; a.tok = m->tok; a.hist = m->hist; a.seq = m->seq; a.ctr = m->ctl + CTL_EPOCH; a.abort_word = m->ctl + CTL_ABORT;
    a.bad_input = m->ctl + CTL_BAD_INPUT;
    a.logits = m->logits;
    a.spin_limit = STEP_SPIN_LIMIT;
    a.samp_mode = m->draw;
    a.chain = m->chain;
    a.seed = m->samp.seed;
    a.kv_row = (long long)c.n_kv_head * c.n_ctx * c.head_dim;
    a.cfg = c.batch == 2 && m->samp.cfg ? 1 : 0;
    a.cfg_weight = m->samp.cfg_weight;
    const uint64_t nph = 5ull * c.n_layer + 1ull;
    m->max_launches = (0xFFFFFFF0ull - nph) / nph;
    return TSD_OK;
}

// before each persistent launch: restart the epochs before they would wrap
hipError_t before_launch(tsd_model* m)
{
    if (!m->step_fn && !m->frame_fused) return hipSuccess;
    if (m->launches >= m->max_launches) {
        hipError_t e = reset_exchange(m);
        if (e != hipSuccess) return e;
    }
    m->launches += 1;
    return hipSuccess;
}

tsd_status init_state(tsd_model* m)
{
    const tsd_config& c = m->c;
    hipStream_t st = m->st;
    HIP_TRY(m, launch_fill_i32(m->pos, 0, 4, st), "init");
    HIP_TRY(m, launch_fill_i32(m->tok, 0, c.batch * m->tpp, st), "init");
    HIP_TRY(m, launch_fill_i32(m->hist, 0, c.n_ctx * c.batch * m->tpp, st), "init");
    HIP_TRY(m, launch_fill_i32(m->seq, -1, c.n_ctx * c.batch, st), "init");
    HIP_TRY(m, launch_fill_f32(m->logits, 0.f, (size_t)c.batch * m->tpp * m->vmax, st), "init");
    // the prompt pass's operands: rows past a prompt's last row are read (never stored), keep them finite
    const size_t amax = (size_t)std::max(c.d_model, c.n_head * c.head_dim);
    for (__half* a : {m->pf_ahi, m->pf_alo})
        HIP_TRY(m, launch_fill_u32((unsigned*)a, 0u, (int)(m->pf_rows * amax / 2), st), "init");
    for (__half* a : {m->pf_hhi, m->pf_hlo})
        HIP_TRY(m, launch_fill_u32((unsigned*)a, 0u, (int)((size_t)m->pf_rows * c.d_ff / 2), st), "init");
    // RoPE table in fp64 on the host: angle = pos * theta^(-2i/hd)
    const int half = c.head_dim / 2;
    std::vector<float2> tab((size_t)m->rope_rows * half);
    for (int p = 0; p < m->rope_rows; ++p)
        for (int i = 0; i < half; ++i) {
            const double a = (double)p * pow((double)c.rope_theta, -2.0 * i / c.head_dim);
            tab[(size_t)p * half + i] = make_float2((float)cos(a), (float)sin(a));
        }
    HIP_TRY(m, hipMemcpyAsync(m->rope, tab.data(), tab.size() * sizeof(float2), hipMemcpyHostToDevice, st), "rope table");
    if (m->step_fn) {
        HIP_TRY(m, hipMemcpyAsync(m->d_sa, &m->sa, sizeof(StepArgs), hipMemcpyHostToDevice, st), "step arguments");
        HIP_TRY(m, hipStreamSynchronize(st), "step arguments");
    }
    HIP_TRY(m, launch_fill_u32(m->ctl, 0u, CTL_WORDS, st), "control words");
    HIP_TRY(m, reset_exchange(m), "exchange init");
    HIP_TRY(m, hipStreamSynchronize(st), "create sync");
    return TSD_OK;
}

// launches of each kind in one step (timing probes size their events from it)
void count_launches(tsd_model* m)
{
    const tsd_config& c = m->c;
    for (int k = 0; k < TSD_KERNEL_KINDS; ++k) m->kind_launches[k] = 0;
    if (c.arch == TSD_ARCH_TALKER_CP) return talker_kind_launches(m, m->kind_launches);
    if (m->step_fn) {
        m->kind_launches[KIND_STEP] = 1;
        return;
    }
    for (int k : {KIND_QKV, KIND_ATTN, KIND_OPROJ, KIND_FC, KIND_DOWN}) m->kind_launches[k] = c.n_layer;
    m->kind_launches[KIND_HEAD] = 1;
}

// ---- the prompt pass -------------------------------------------------------------------------
// Prompt positions t0 .. t0 + np - 1 of every batch row (ids d_tokens[b][n_prompt][tokens per
// position]) at cache positions pos0 .. pos0 + np - 1: the embedding rows (the sum of
// the frame's code embeddings for the Talker), then per layer norm, QKV product (queries, RoPE,
// K/V into the cache), causal attention, output projection into the residual stream, norm,
// FC / gate-up product and down projection.  No head: the last prompt position goes through the
// decode step (the whole frame for TALKER_CP).
hipError_t pf_enqueue(tsd_model* m, const int32_t* d_tokens, int n_prompt, int t0, int np, int pos0, hipStream_t st)
{
    const tsd_config& c = m->c;
    const int d = c.d_model, H = c.n_head, Hk = c.n_kv_head, hd = c.head_dim, ff = c.d_ff, B = c.batch, f = c.wfmt;
    const bool gpt2 = c.arch == TSD_ARCH_GPT2, talker = c.arch == TSD_ARCH_TALKER_CP;
    const int M = B * np, qd = H * hd;
    PfRowArgs ra{};
    ra.M = M; ra.d = d; ra.n_pos = np; ra.pos0 = pos0;
    ra.tok = d_tokens; ra.tok_stride = n_prompt; ra.t0 = t0; ra.n_prompt = n_prompt;
    ra.n_tab = m->tpp;
    for (int k = 0; k < m->tpp; ++k) {
        ra.tab[k] = m->emb[k];
        ra.tab_rows[k] = m->emb_rows[k];
    }
    ra.wpe = m->wpe; ra.seq = m->seq; ra.B = B;
    ra.hist = talker ? nullptr : m->hist;   // the Talker's prompt frames leave their history alone, as its frames do
    ra.x = m->pf_x; ra.x_out = m->pf_x; ra.eps = c.norm_eps;
    ra.ahi = m->pf_ahi; ra.alo = m->pf_alo;
    PfGemmArgs ga{};
    ga.M = M;
    ga.n_ctx = c.n_ctx; ga.n_pos = np; ga.pos0 = pos0;
    ga.kv_row = (long long)Hk * c.n_ctx * hd;
    PfAttnArgs aa{};
    aa.q = m->pf_q; aa.ldq = qd; aa.kv_row = ga.kv_row;
    aa.M = M; aa.H = H; aa.Hkv = Hk; aa.hd = hd; aa.n_ctx = c.n_ctx; aa.n_pos = np; aa.pos0 = pos0;
    aa.ohi = m->pf_ahi; aa.olo = m->pf_alo; aa.ldo = qd;
    // one product: the packed matrix (GPT2/LLAMA) or the tiled one (Talker)
    auto gemm = [&](PfGemmArgs g, int epi, const PackedMat* P, const TiledMat* T) {
        if (T) {
            g.T = *T;
            g.W.N = T->N;
            g.W.K = T->K;
            return launch_pf_gemm_tiled(epi, g, st);
        }
        g.W = *P;
        return launch_pf_gemm(f, epi, g, st);
    };
    hipError_t e = hipSuccess;
    for (int l = 0; l < c.n_layer && e == hipSuccess; ++l) {
        const LayerW* w = talker ? nullptr : &m->L[l];
        const TLayerW* tw = talker ? &m->Lt[l] : nullptr;
        __half* kc = m->kc + m->kv_layer_elems * l;
        __half* vc = m->vc + m->kv_layer_elems * l;
        ra.g = talker ? tw->n1g : w->n1g;
        ra.bn = talker ? nullptr : w->n1b;
        e = l == 0 ? launch_pf_embed(ra, st) : launch_pf_norm(ra, st);
        // Q/K/V: queries (after RoPE) to pf_q, keys and values into the cache
        PfGemmArgs q = ga;
        q.ahi = m->pf_ahi; q.alo = m->pf_alo; q.bias = talker ? nullptr : w->bqkv;
        q.q = m->pf_q; q.ldq = qd; q.qrows = qd; q.krows = Hk * hd; q.hd = hd; q.rope = gpt2 ? 0 : 1;
        q.rope_tab = m->rope; q.kc = kc; q.vc = vc;
        if (e == hipSuccess) e = gemm(q, PF_QKV, talker ? nullptr : &w->qkv, talker ? &tw->qkv : nullptr);
        aa.kc = kc; aa.vc = vc;
        if (e == hipSuccess) e = launch_pf_attention(aa, st);
        PfGemmArgs o = ga;
        o.ahi = m->pf_ahi; o.alo = m->pf_alo; o.bias = talker ? nullptr : w->bo; o.y = m->pf_x; o.ldy = d;
        if (e == hipSuccess) e = gemm(o, PF_RESID, talker ? nullptr : &w->o, talker ? &tw->o : nullptr);
        ra.g = talker ? tw->n2g : w->n2g;
        ra.bn = talker ? nullptr : w->n2b;
        if (e == hipSuccess) e = launch_pf_norm(ra, st);
        PfGemmArgs u = ga;
        u.ahi = m->pf_ahi; u.alo = m->pf_alo; u.bias = talker ? nullptr : w->bfc;
        u.ohi = m->pf_hhi; u.olo = m->pf_hlo; u.ldo = ff;
        if (e == hipSuccess) e = gemm(u, gpt2 ? PF_GELU : PF_SWIGLU, talker ? nullptr : &w->fc, talker ? &tw->fc : nullptr);
        PfGemmArgs dn = ga;
        dn.ahi = m->pf_hhi; dn.alo = m->pf_hlo; dn.bias = talker ? nullptr : w->bdown; dn.y = m->pf_x; dn.ldy = d;
        if (e == hipSuccess) e = gemm(dn, PF_RESID, talker ? nullptr : &w->down, talker ? &tw->down : nullptr);
    }
    return e;
}

// the step graph; talker_only: the TALKER_CP frame without head and predictor (prefill positions)
tsd_status capture(tsd_model* m, bool talker_only, hipGraph_t* out_g, hipGraphExec_t* out_x)
{
    hipStream_t cs;
    HIP_TRY(m, hipStreamCreateWithFlags(&cs, hipStreamNonBlocking), "capture stream");
    hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) { (void)hipStreamDestroy(cs); return hip_fail(m, e, "begin capture"); }
    hipError_t le = talker_only ? talker_enqueue(m, cs, false) : enqueue_step(m, cs);
    hipGraph_t g = nullptr;
    e = hipStreamEndCapture(cs, &g);
    (void)hipStreamDestroy(cs);
    if (le != hipSuccess) { if (g) (void)hipGraphDestroy(g); return hip_fail(m, le, "step launch during capture"); }
    if (e != hipSuccess) return hip_fail(m, e, "end capture");
    hipGraphExec_t x = nullptr;
    e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
    if (e != hipSuccess) { (void)hipGraphDestroy(g); return hip_fail(m, e, "instantiate"); }
    *out_g = g;
    *out_x = x;
    return TSD_OK;
}

}  // namespace

// ---- C ABI --------------------------------------------------------------------------------

extern "C" {

tsd_status tsd_workspace_bytes(const tsd_config* cfg, size_t* out)
{
    std::string msg;
    tsd_status s = validate(cfg, msg);
    if (s != TSD_OK) return fail(nullptr, s, msg);
    if (!out) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "null output");
    *out = plan(nullptr, cfg, nullptr);
    return TSD_OK;
}

// the sampling parameters' ranges: mode 0 or 1; a positive finite temperature (mode 1); top_p in
// [0, 1] (0 and 1 off); min_p in [0, 1), only in the multilingual order; rep_penalty 0 (off) or
// positive and finite; order T3 or MTL
tsd_status check_sampling(const tsd_sampling* s, std::string& msg)
{
    if (s->mode != 0 && s->mode != 1) return msg = "sampling mode must be 0 (greedy) or 1 (draw)", TSD_ERR_INVALID_ARGUMENT;
    if (s->mode == 1 && (!(s->temperature > 0.f) || !std::isfinite(s->temperature)))
        return msg = "temperature must be positive and finite", TSD_ERR_INVALID_ARGUMENT;
    if (!(s->top_p >= 0.f && s->top_p <= 1.f)) return msg = "top_p must lie in [0, 1]", TSD_ERR_INVALID_ARGUMENT;
    if (!(s->min_p >= 0.f && s->min_p < 1.f)) return msg = "min_p must lie in [0, 1)", TSD_ERR_INVALID_ARGUMENT;
    if (!(s->rep_penalty >= 0.f) || !std::isfinite(s->rep_penalty))
        return msg = "rep_penalty must be 0 (off) or positive and finite", TSD_ERR_INVALID_ARGUMENT;
    if (s->order != TSD_ORDER_T3 && s->order != TSD_ORDER_MTL) return msg = "unknown sampler order", TSD_ERR_INVALID_ARGUMENT;
    if (s->min_p > 0.f && s->order != TSD_ORDER_MTL)
        return msg = "min_p is a step of the multilingual order (TSD_ORDER_MTL)", TSD_ERR_INVALID_ARGUMENT;
    if (s->cfg != 0 && s->cfg != 1) return msg = "cfg must be 0 or 1", TSD_ERR_INVALID_ARGUMENT;
    if (!std::isfinite(s->cfg_weight)) return msg = "cfg_weight must be finite", TSD_ERR_INVALID_ARGUMENT;
    return TSD_OK;
}

// the chain the kernels run for a head of n ids (with_penalty: the head the penalty covers);
// greedy with a penalty is the draw of the single largest penalized logit
bool chain_of(const tsd_sampling* s, int n, bool with_penalty, SampChain* ch, int* draw)
{
    const bool pen = with_penalty && s->rep_penalty > 0.f && s->rep_penalty != 1.f;
    *ch = SampChain{1.f, 1, 0.f, 0.f, 1.f, SAMP_ORDER_MTL};
    *draw = 0;
    if (s->mode == 0) {
        if (!pen && !s->cfg) return true;   // greedy over guided logits is the draw's k = 1
        if (!pen) {
            *draw = 1;
            return sample_supported(n, 1);
        }
        ch->penalty = s->rep_penalty;
        *draw = 1;
        return sample_supported(n, 1);
    }
    ch->temperature = s->temperature;
    ch->k = (s->top_k <= 0 || s->top_k > n) ? n : s->top_k;
    ch->top_p = s->top_p;
    ch->min_p = s->min_p;
    ch->penalty = pen ? s->rep_penalty : 1.f;
    ch->order = s->order == TSD_ORDER_MTL ? SAMP_ORDER_MTL : SAMP_ORDER_T3;
    *draw = 1;
    return sample_supported(n, ch->k);
}

tsd_status tsd_model_create(const tsd_config* cfg, const tsd_tensor* weights, int n_weights, void* d_ws,
                            size_t ws_bytes, void* stream, const tsd_sampling* sampling, tsd_model** out)
{
    std::string msg;
    tsd_status s = validate(cfg, msg);
    if (s != TSD_OK) return fail(nullptr, s, msg);
    if (!out || !weights || !d_ws) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "null argument");
    *out = nullptr;
    if ((uintptr_t)d_ws % 256) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    const size_t need = plan(nullptr, cfg, nullptr);
    if (ws_bytes < need)
        return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "workspace too small: need " + std::to_string(need) + " bytes");
    if (n_weights != n_weights_of(cfg))
        return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "expected " + std::to_string(n_weights_of(cfg)) + " weights");
    std::vector<size_t> sz;
    canonical_sizes(cfg, sz);
    for (int i = 0; i < n_weights; ++i)
        if (!weights[i].ptr || weights[i].bytes != sz[i])
            return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "weight " + std::to_string(i) + ": " +
                        std::to_string(weights[i].bytes) + " bytes, expected " + std::to_string(sz[i]));
    tsd_sampling sv{};
    if (sampling) sv = *sampling;
    std::string smsg;
    s = check_sampling(&sv, smsg);
    if (s != TSD_OK) return fail(nullptr, s, smsg);
    if (sv.cfg && (cfg->arch == TSD_ARCH_TALKER_CP || cfg->batch != 2))
        return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "classifier-free guidance needs a GPT2/LLAMA model of batch 2 "
                                                       "(row 0 conditioned, row 1 unconditioned)");
    SampChain ch{}, cch{};
    int draw = 0, cdraw = 0;
    if (!chain_of(&sv, cfg->vocab, true, &ch, &draw))
        return fail(nullptr, TSD_ERR_UNSUPPORTED, "draws support k <= 1024 and vocabularies up to 12288");
    if (cfg->arch == TSD_ARCH_TALKER_CP && !chain_of(&sv, cfg->cp_vocab, false, &cch, &cdraw))
        return fail(nullptr, TSD_ERR_UNSUPPORTED, "draws support k <= 1024 and vocabularies up to 12288");
    tsd_model* m = new (std::nothrow) tsd_model();
    if (!m) return fail(nullptr, TSD_ERR_OUT_OF_MEMORY, "host allocation");
    m->c = *cfg;
    m->samp = sv;
    m->chain = ch;
    m->cp_chain = cch;
    m->draw = draw;
    m->cp_draw = cdraw;
    m->top_k = ch.k;
    m->st = (hipStream_t)stream;
    m->ws = (uint8_t*)d_ws;
    m->ws_bytes = ws_bytes;
    plan(m, cfg, (uint8_t*)d_ws);
    tsd_status r = setup_step(m);
    if (r == TSD_OK) r = pack_weights(m, weights);
    if (r == TSD_OK) r = init_state(m);
    if (r == TSD_OK) r = capture(m, false, &m->graph, &m->exec);
    if (r == TSD_OK && cfg->arch == TSD_ARCH_TALKER_CP) r = capture(m, true, &m->graph_talker, &m->exec_talker);
    if (r == TSD_OK) count_launches(m);
    if (r != TSD_OK) {
        g_err = m->err;
        tsd_model_destroy(m);
        return r;
    }
    *out = m;
    return TSD_OK;
}

tsd_status tsd_model_destroy(tsd_model* m)
{
    if (!m) return TSD_OK;
    if (m->exec) (void)hipGraphExecDestroy(m->exec);
    if (m->graph) (void)hipGraphDestroy(m->graph);
    if (m->exec_talker) (void)hipGraphExecDestroy(m->exec_talker);
    if (m->graph_talker) (void)hipGraphDestroy(m->graph_talker);
    for (int k = 0; k < TSD_KERNEL_KINDS; ++k)
        for (hipEvent_t ev : m->probe_ev[k]) (void)hipEventDestroy(ev);
    delete m;
    return TSD_OK;
}

const char* tsd_last_error(const tsd_model* m) { return m ? m->err.c_str() : g_err.c_str(); }

namespace {
// One step on the model's stream.  A persistent step is a single kernel: it is launched directly,
// which leaves ~2 us between back-to-back steps where replaying it as a one-node graph left ~7 us
// (it can still be captured into a caller's graph); the other modes replay their step graph.
hipError_t launch_one_step(tsd_model* m, hipGraphExec_t x)
{
    if (m->step_fn && x == m->exec) return launch_step(m->step_fn, m->d_sa, m->n_wg, m->st);
    return hipGraphLaunch(x, m->st);
}

// the ids of one position (rows of tok_per_pos ids, src_stride apart) into the step's input slots,
// checked on the device: a rejected set leaves the slots alone and raises the bad-input word
hipError_t set_input(tsd_model* m, const int32_t* src, long long src_stride)
{
    const bool talker = m->c.arch == TSD_ARCH_TALKER_CP;
    return launch_set_input(m->tok, src, m->c.batch, m->tpp, src_stride, m->c.vocab, talker ? m->c.cp_vocab : m->c.vocab,
                            m->ctl + CTL_BAD_INPUT, m->st);
}
}  // namespace

tsd_status tsd_step(tsd_model* m, const int32_t* d_in, int32_t* d_next)
{
    if (!m) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "null model");
    if (m->n_past >= m->c.n_ctx) return fail(m, TSD_ERR_CONTEXT_FULL, "context full");
    const int nt = m->c.batch * m->tpp;
    if (d_in || d_next) m->io_since_sync = true;
    if (d_in) HIP_TRY(m, set_input(m, d_in, m->tpp), "set input");
    HIP_TRY(m, before_launch(m), "exchange restart");
    HIP_TRY(m, launch_one_step(m, m->exec), "step launch");
    if (d_next) HIP_TRY(m, launch_copy_i32(d_next, m->tok, nt, m->st), "copy ids");
    m->n_past += 1;
    return TSD_OK;
}

tsd_status tsd_step_eager(tsd_model* m, const int32_t* d_in, int32_t* d_next)
{
    if (!m) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "null model");
    if (m->n_past >= m->c.n_ctx) return fail(m, TSD_ERR_CONTEXT_FULL, "context full");
    const int nt = m->c.batch * m->tpp;
    if (d_in || d_next) m->io_since_sync = true;
    if (d_in) HIP_TRY(m, set_input(m, d_in, m->tpp), "set input");
    HIP_TRY(m, before_launch(m), "exchange restart");
    HIP_TRY(m, enqueue_step(m, m->st), "eager step");
    if (d_next) HIP_TRY(m, launch_copy_i32(d_next, m->tok, nt, m->st), "copy ids");
    m->n_past += 1;
    return TSD_OK;
}

tsd_status tsd_prefill(tsd_model* m, const int32_t* d_tokens, int n, int32_t* d_next)
{
    if (!m) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "null model");
    if (!d_tokens || n <= 0) return fail(m, TSD_ERR_INVALID_ARGUMENT, "empty prompt");
    if (m->n_past + n > m->c.n_ctx) return fail(m, TSD_ERR_CONTEXT_FULL, "prompt does not fit the context");
    m->io_since_sync = true;
    const int nt = m->c.batch * m->tpp;
    const bool talker = m->c.arch == TSD_ARCH_TALKER_CP;
    // every id of the prompt is checked first; a bad one makes every launch below leave the state
    // alone (the prompt pass only writes cache rows and records at positions from n_past on,
    // which no step reads before they are written again)
    HIP_TRY(m, launch_check_ids(d_tokens, m->c.batch, n, m->tpp, m->c.vocab, talker ? m->c.cp_vocab : m->c.vocab,
                                m->ctl + CTL_BAD_INPUT, m->st),
            "check ids");
    const int n_past0 = m->n_past;
    // every position but the last through the prompt pass, in chunks of pf_rows rows; the model's
    // position count changes only once everything is enqueued
    const int chunk = m->pf_rows / m->c.batch;
    int p = n_past0;
    for (int t0 = 0; t0 < n - 1; t0 += chunk) {
        const int np = std::min(chunk, n - 1 - t0);
        HIP_TRY(m, pf_enqueue(m, d_tokens, n, t0, np, p, m->st), "prompt pass");
        p += np;
    }
    hipError_t e = hipSuccess;
    if (n > 1) e = launch_set_pos(m->pos, p, m->ctl + CTL_BAD_INPUT, m->st);
    // the last position: one decode step (head, sampler, history; the whole frame for TALKER_CP)
    if (e == hipSuccess) e = set_input(m, d_tokens + (size_t)(n - 1) * m->tpp, (long long)n * m->tpp);
    if (e == hipSuccess) e = before_launch(m);
    if (e == hipSuccess) e = launch_one_step(m, m->exec);
    if (e != hipSuccess) {
        if (n > 1) (void)launch_fill_i32(m->pos, n_past0, 1, m->st);   // the position as it was
        return hip_fail(m, e, "prefill");
    }
    m->n_past = p + 1;
    if (d_next) HIP_TRY(m, launch_copy_i32(d_next, m->tok, nt, m->st), "copy ids");
    return TSD_OK;
}

tsd_status tsd_prefill_stepwise(tsd_model* m, const int32_t* d_tokens, int n, int32_t* d_next)
{
    if (!m) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "null model");
    if (!d_tokens || n <= 0) return fail(m, TSD_ERR_INVALID_ARGUMENT, "empty prompt");
    if (m->n_past + n > m->c.n_ctx) return fail(m, TSD_ERR_CONTEXT_FULL, "prompt does not fit the context");
    m->io_since_sync = true;
    const int nt = m->c.batch * m->tpp;
    const bool talker = m->c.arch == TSD_ARCH_TALKER_CP;
    HIP_TRY(m, launch_check_ids(d_tokens, m->c.batch, n, m->tpp, m->c.vocab, talker ? m->c.cp_vocab : m->c.vocab,
                                m->ctl + CTL_BAD_INPUT, m->st),
            "check ids");
    for (int t = 0; t < n; ++t) {
        // tokens are [batch][n][tokens per position]: position t of every row
        HIP_TRY(m, set_input(m, d_tokens + (size_t)t * m->tpp, (long long)n * m->tpp), "set input");
        HIP_TRY(m, before_launch(m), "exchange restart");
        // TALKER_CP prompt frames before the last need neither head nor predictor
        hipGraphExec_t x = (m->exec_talker && t + 1 < n) ? m->exec_talker : m->exec;
        HIP_TRY(m, launch_one_step(m, x), "step launch");
        m->n_past += 1;
    }
    if (d_next) HIP_TRY(m, launch_copy_i32(d_next, m->tok, nt, m->st), "copy ids");
    return TSD_OK;
}

namespace {
// A wait inside a persistent step timed out (another kernel held compute units the grid needed,
// or a fault in the exchange): that launch and every persistent launch after it returned without
// moving the position.  The model falls back to one launch per operator for good (no waits
// between workgroups), the exchange restarts, and the lost positions, which read their input from
// the device, run again; those whose ids came from or went to caller buffers are left for the
// caller to submit again (TSD_ERR_TIMEOUT, with n_past at the first lost position).
tsd_status recover_persistent(tsd_model* m)
{
    int pos = 0;
    HIP_TRY(m, hipMemcpy(&pos, m->pos, sizeof(pos), hipMemcpyDeviceToHost), "read position");
    const int lost = m->n_past - pos;
    const void* fn = m->step_fn;
    m->step_fn = nullptr;
    hipGraph_t g = nullptr;
    hipGraphExec_t x = nullptr;
    tsd_status s = capture(m, false, &g, &x);
    if (s != TSD_OK) {
        m->step_fn = fn;
        return s;
    }
    if (m->exec) (void)hipGraphExecDestroy(m->exec);
    if (m->graph) (void)hipGraphDestroy(m->graph);
    m->graph = g;
    m->exec = x;
    count_launches(m);
    HIP_TRY(m, reset_exchange(m), "exchange restart");
    m->n_past = pos;
    if (m->io_since_sync) {
        m->io_since_sync = false;
        HIP_TRY(m, hipStreamSynchronize(m->st), "stream sync");
        return fail(m, TSD_ERR_TIMEOUT, "a wait inside the persistent step timed out; the model now runs one launch "
                                        "per operator, and the positions from n_past on must be submitted again");
    }
    for (int i = 0; i < lost; ++i) {
        HIP_TRY(m, launch_one_step(m, m->exec), "step launch");
        m->n_past += 1;
    }
    HIP_TRY(m, hipStreamSynchronize(m->st), "stream sync");
    m->err = "a wait inside the persistent step timed out; the " + std::to_string(lost) +
             " steps since ran again with one launch per operator, which the model keeps using";
    return TSD_OK;
}
}  // namespace

tsd_status tsd_synchronize(tsd_model* m)
{
    if (!m) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "null model");
    HIP_TRY(m, hipStreamSynchronize(m->st), "stream sync");
    uint32_t ctl[CTL_BAD_INPUT + 1] = {};
    HIP_TRY(m, hipMemcpy(ctl, m->ctl, sizeof(ctl), hipMemcpyDeviceToHost), "read control words");
    if (m->step_fn && ctl[CTL_ABORT]) return recover_persistent(m);
    if (m->frame_fused && ctl[CTL_ABORT])
        return fail(m, TSD_ERR_TIMEOUT, "a wait inside a frame launch timed out; the frames since are void "
                                        "(tsd_reset clears the state)");
    if (ctl[CTL_BAD_INPUT]) {
        // the calls since the rejected input did nothing: the position count is the device's
        int pos = 0;
        HIP_TRY(m, hipMemcpy(&pos, m->pos, sizeof(pos), hipMemcpyDeviceToHost), "read position");
        m->n_past = pos;
        HIP_TRY(m, launch_fill_u32(m->ctl + CTL_BAD_INPUT, 0u, 1, m->st), "clear bad-input word");
        HIP_TRY(m, hipStreamSynchronize(m->st), "stream sync");
        m->io_since_sync = false;
        return fail(m, TSD_ERR_INVALID_ARGUMENT, "a token id outside its vocabulary was passed in; that call and "
                                                 "every model call after it until now did nothing (the model state "
                                                 "is as it was before that call)");
    }
    m->io_since_sync = false;
    return TSD_OK;
}

tsd_status tsd_model_info(const tsd_model* m, int32_t* launch_mode, int32_t* n_workgroups)
{
    if (!m) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "null model");
    if (launch_mode) *launch_mode = m->step_fn ? TSD_LAUNCH_PERSISTENT : TSD_LAUNCH_PER_OPERATOR;
    if (n_workgroups) *n_workgroups = m->step_fn ? m->n_wg : 0;
    return TSD_OK;
}

tsd_status tsd_debug_set_wait_limit(tsd_model* m, int64_t ticks)
{
    if (!m) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "null model");
    if (!m->step_fn) return fail(m, TSD_ERR_UNSUPPORTED, "the model does not run the persistent step");
    m->sa.spin_limit = ticks > 0 ? (long long)ticks : STEP_SPIN_LIMIT;
    HIP_TRY(m, hipMemcpyAsync(m->d_sa, &m->sa, sizeof(StepArgs), hipMemcpyHostToDevice, m->st), "step arguments");
    HIP_TRY(m, hipStreamSynchronize(m->st), "step arguments");
    return TSD_OK;
}

tsd_status tsd_reset(tsd_model* m)
{
    if (!m) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "null model");
    HIP_TRY(m, launch_fill_i32(m->pos, 0, 1, m->st), "reset");
    HIP_TRY(m, launch_fill_i32(m->hist, 0, m->c.n_ctx * m->c.batch * m->tpp, m->st), "reset");
    HIP_TRY(m, launch_fill_i32(m->seq, -1, m->c.n_ctx * m->c.batch, m->st), "reset");
    HIP_TRY(m, launch_fill_u32(m->ctl + CTL_BAD_INPUT, 0u, 1, m->st), "reset");
    if (m->step_fn || m->frame_fused) HIP_TRY(m, reset_exchange(m), "reset");
    m->n_past = 0;
    return TSD_OK;
}

tsd_status tsd_truncate(tsd_model* m, int n_past)
{
    if (!m) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "null model");
    if (n_past < 0 || n_past > m->n_past) return fail(m, TSD_ERR_INVALID_ARGUMENT, "truncate beyond n_past");
    HIP_TRY(m, launch_fill_i32(m->pos, n_past, 1, m->st), "truncate");
    m->n_past = n_past;
    return TSD_OK;
}

tsd_status tsd_n_past(const tsd_model* m, int* out)
{
    if (!m || !out) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "null argument");
    *out = m->n_past;
    return TSD_OK;
}

tsd_status tsd_get_logits(tsd_model* m, float* d_out)
{
    if (!m || !d_out) return fail(m, TSD_ERR_INVALID_ARGUMENT, "null argument");
    const size_t n = (size_t)m->c.batch * m->tpp * m->vmax;
    HIP_TRY(m, hipMemcpyAsync(d_out, m->logits, n * sizeof(float), hipMemcpyDeviceToDevice, m->st), "copy logits");
    return TSD_OK;
}

tsd_status tsd_get_tokens(tsd_model* m, int first, int n, int32_t* d_out)
{
    if (!m || !d_out) return fail(m, TSD_ERR_INVALID_ARGUMENT, "null argument");
    if (first < 0 || n < 0 || first + n > m->c.n_ctx) return fail(m, TSD_ERR_INVALID_ARGUMENT, "range outside the context");
    const size_t nt = (size_t)m->c.batch * m->tpp;
    HIP_TRY(m, hipMemcpyAsync(d_out, m->hist + first * nt, n * nt * sizeof(int), hipMemcpyDeviceToDevice, m->st), "copy tokens");
    return TSD_OK;
}

tsd_status tsd_load_kv(tsd_model* m, const uint16_t* d_k, const uint16_t* d_v, int n_pos)
{
    if (!m || !d_k || !d_v) return fail(m, TSD_ERR_INVALID_ARGUMENT, "null argument");
    const tsd_config& c = m->c;
    if (n_pos < 0 || n_pos > c.n_ctx) return fail(m, TSD_ERR_CONTEXT_FULL, "n_pos outside the context");
    if (n_pos > 0) {
        const size_t w = (size_t)n_pos * c.head_dim * 2, dp = (size_t)c.n_ctx * c.head_dim * 2;
        const size_t rows = (size_t)c.n_layer * c.batch * c.n_kv_head;
        HIP_TRY(m, hipMemcpy2DAsync(m->kc, dp, d_k, w, w, rows, hipMemcpyDeviceToDevice, m->st), "load k");
        HIP_TRY(m, hipMemcpy2DAsync(m->vc, dp, d_v, w, w, rows, hipMemcpyDeviceToDevice, m->st), "load v");
    }
    HIP_TRY(m, launch_fill_i32(m->pos, n_pos, 1, m->st), "set position");
    HIP_TRY(m, launch_fill_i32(m->seq, -1, m->c.n_ctx * m->c.batch, m->st), "load kv");   // tokens unknown
    m->n_past = n_pos;
    return TSD_OK;
}

tsd_status tsd_get_kv(tsd_model* m, uint16_t* d_k, uint16_t* d_v, int n_pos)
{
    if (!m) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "null model");
    const tsd_config& c = m->c;
    if (n_pos < 0 || n_pos > m->n_past) return fail(m, TSD_ERR_INVALID_ARGUMENT, "n_pos outside 0..n_past");
    if (n_pos > 0) {
        if (!d_k || !d_v) return fail(m, TSD_ERR_INVALID_ARGUMENT, "null argument");
        const size_t w = (size_t)n_pos * c.head_dim * 2, sp = (size_t)c.n_ctx * c.head_dim * 2;
        const size_t rows = (size_t)c.n_layer * c.batch * c.n_kv_head;
        HIP_TRY(m, hipMemcpy2DAsync(d_k, w, m->kc, sp, w, rows, hipMemcpyDeviceToDevice, m->st), "get k");
        HIP_TRY(m, hipMemcpy2DAsync(d_v, w, m->vc, sp, w, rows, hipMemcpyDeviceToDevice, m->st), "get v");
    }
    return TSD_OK;
}

tsd_status tsd_layer_forward(tsd_model* m, int layer, const float* d_x, int pos, float* d_out)
{
    if (!m || !d_x || !d_out) return fail(m, TSD_ERR_INVALID_ARGUMENT, "null argument");
    const tsd_config& c = m->c;
    if (layer < 0 || layer >= c.n_layer) return fail(m, TSD_ERR_INVALID_ARGUMENT, "layer out of range");
    if (pos < 0 || pos >= c.n_ctx) return fail(m, TSD_ERR_CONTEXT_FULL, "position outside the context");
    HIP_TRY(m, launch_fill_i32(m->dbg_pos, pos, 1, m->st), "set position");
    if (c.arch == TSD_ARCH_TALKER_CP) {   // the batched frame keeps its rows interleaved
        HIP_TRY(m, before_launch(m), "exchange restart");
        HIP_TRY(m, talker_layer(m, layer, m->st, d_x, m->dbg_pos), "layer");
        HIP_TRY(m, launch_il_to_rows(m->x, c.batch, c.d_model, d_out, m->st), "copy out");
        return TSD_OK;
    }
    const size_t xb = (size_t)c.batch * c.d_model * sizeof(float);
    HIP_TRY(m, hipMemcpyAsync(m->x, d_x, xb, hipMemcpyDeviceToDevice, m->st), "copy x");
    HIP_TRY(m, enqueue_layer(m, layer, m->st, m->dbg_pos, false), "layer");
    HIP_TRY(m, hipMemcpyAsync(d_out, m->x, xb, hipMemcpyDeviceToDevice, m->st), "copy out");
    return TSD_OK;
}

tsd_status tsd_time_kernel(tsd_model* m, int kind, int n_steps, float* avg_us, int* launches_per_step)
{
    if (!m || !avg_us) return fail(m, TSD_ERR_INVALID_ARGUMENT, "null argument");
    if (kind < 0 || kind >= TSD_KERNEL_KINDS || n_steps <= 0) return fail(m, TSD_ERR_INVALID_ARGUMENT, "bad kind or step count");
    if (m->n_past + n_steps > m->c.n_ctx) return fail(m, TSD_ERR_CONTEXT_FULL, "probe steps do not fit the context");
    if ((kind == KIND_STEP) != (m->step_fn != nullptr))
        return fail(m, TSD_ERR_UNSUPPORTED, "this model does not launch a kernel of that kind");
    const int pairs_max = m->kind_launches[kind];
    if (pairs_max == 0) return fail(m, TSD_ERR_UNSUPPORTED, "this step has no kernel of that kind");
    if (m->probe_ev[kind].empty()) {
        m->probe_ev[kind].resize(4 * pairs_max);
        for (auto& ev : m->probe_ev[kind]) HIP_TRY(m, hipEventCreate(&ev), "probe event");
    }
    // the step's kernels with their step arguments, enqueued directly on the model's stream
    // (graph-recorded events carry no timestamps), events around every launch of `kind`
    double total_ms = 0.0;
    int pairs = 0;
    for (int s = 0; s < n_steps; ++s) {
        Probe pr;
        pr.kind = kind;
        pr.ev = m->probe_ev[kind].data();
        HIP_TRY(m, before_launch(m), "exchange restart");
        HIP_TRY(m, enqueue_step(m, m->st, &pr), "probe step");
        HIP_TRY(m, hipStreamSynchronize(m->st), "probe sync");
        m->n_past += 1;
        pairs = pr.next / 4;
        if (pairs == 0) return fail(m, TSD_ERR_UNSUPPORTED, "this step has no kernel of that kind");
        for (int i = 0; i < pairs; ++i) {
            float e = 0.f, k = 0.f;
            const hipEvent_t* ev = &m->probe_ev[kind][4 * i];
            HIP_TRY(m, hipEventElapsedTime(&e, ev[0], ev[1]), "probe elapsed");
            HIP_TRY(m, hipEventElapsedTime(&k, ev[2], ev[3]), "probe elapsed");
            total_ms += k - e;
        }
    }
    *avg_us = (float)(total_ms * 1e3 / ((double)n_steps * pairs));
    if (launches_per_step) *launches_per_step = pairs;
    return TSD_OK;
}

// ---- standalone operators -------------------------------------------------------------------

tsd_status tsd_gemm_scratch_bytes(int M, int K, size_t* out)
{
    if (!out || M <= 0 || K <= 0 || K % 32) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "bad shape");
    *out = 2 * align256((size_t)((M + 31) / 32 * 32) * K * 2);   // the operand rows (whole 32-row tiles), fp16 hi then lo
    return TSD_OK;
}

tsd_status tsd_gemm(int wfmt, const void* d_packed, int N, int K, int M, const float* d_x, const float* d_bias,
                    float* d_y, void* d_scratch, size_t scratch_bytes, void* stream)
{
    size_t need = 0;
    if (!known_format(wfmt) || N <= 0 || M <= 0 || K <= 0 || K % group_of(wfmt) || !pf_gemm_ok(wfmt, K))
        return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "bad format or shape");
    tsd_status s = tsd_gemm_scratch_bytes(M, K, &need);
    if (s != TSD_OK) return s;
    if (!d_packed || !d_x || !d_y || !d_scratch) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "null buffer");
    if ((uintptr_t)d_scratch % 256 || (uintptr_t)d_packed % 256)
        return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "packed matrix and scratch must be 256-byte aligned");
    if (scratch_bytes < need) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "scratch too small");
    hipStream_t st = (hipStream_t)stream;
    __half* hi = (__half*)d_scratch;
    __half* lo = (__half*)((uint8_t*)d_scratch + need / 2);
    hipError_t e = launch_pf_split(d_x, M, K, hi, lo, st);
    PfGemmArgs a{};
    a.W = packed_view(wfmt, (void*)d_packed, N, K);
    a.M = M;
    a.ahi = hi;
    a.alo = lo;
    a.bias = d_bias;
    a.y = d_y;
    a.ldy = N;
    if (e == hipSuccess) e = launch_pf_gemm(wfmt, PF_STORE, a, st);
    return e == hipSuccess ? TSD_OK : hip_fail(nullptr, e, "gemm");
}

tsd_status tsd_gemv_packed_bytes(int wfmt, int N, int K, size_t* out)
{
    if (!out || !known_format(wfmt) || N <= 0 || K <= 0 || K % group_of(wfmt))
        return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "bad format or shape");
    *out = packed_layout(wfmt, N, K).total;
    return TSD_OK;
}

tsd_status tsd_gemv_pack(int wfmt, const void* d_w, size_t w_bytes, int N, int K, void* d_packed, size_t packed_bytes,
                         void* stream)
{
    size_t need = 0;
    tsd_status s = tsd_gemv_packed_bytes(wfmt, N, K, &need);
    if (s != TSD_OK) return s;
    if (!d_w || !d_packed) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "null buffer");
    if (w_bytes != canonical_matrix_bytes(wfmt, N, K)) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "canonical size mismatch");
    if (packed_bytes < need) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "packed buffer too small");
    hipError_t e = launch_pack(wfmt, d_w, N, K, d_packed, N, 0, PACK_IDENTITY, 64, (hipStream_t)stream);
    return e == hipSuccess ? TSD_OK : hip_fail(nullptr, e, "pack");
}

tsd_status tsd_gemv(int wfmt, const void* d_packed, int N, int K, int B, const float* d_x, const float* d_bias,
                    float* d_y, void* stream)
{
    if (!known_format(wfmt) || N <= 0 || K <= 0 || K % group_of(wfmt) || B < 1 || B > 4)
        return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "bad format or shape");
    if (!d_packed || !d_x || !d_y) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "null buffer");
    if (K > 4096 || !gemv_shape_ok(wfmt, K)) return fail(nullptr, TSD_ERR_UNSUPPORTED, "K has no GEMV lane mapping");
    PackedMat W = packed_view(wfmt, (void*)d_packed, N, K);
    for (int b = 0; b < B; ++b) {   // batch rows share nothing but the weights: one launch each
        ProArgs pa{};
        pa.src = d_x + (size_t)b * K;
        EpiArgs ea{};
        ea.y = d_y + (size_t)b * N;
        ea.bias = d_bias;
        hipError_t e = launch_gemv_stream(wfmt, W, pa, ea, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(nullptr, e, "gemv");
    }
    return TSD_OK;
}

tsd_status tsd_gemm_rows_packed_bytes(int N, int K, size_t* out)
{
    if (!out || !mm16_supported(N, K)) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "bad shape");
    *out = tiled_bytes(N, K);
    return TSD_OK;
}

tsd_status tsd_gemm_rows_pack(const void* d_w, size_t w_bytes, int N, int K, void* d_packed, size_t packed_bytes,
                              void* stream)
{
    size_t need = 0;
    tsd_status s = tsd_gemm_rows_packed_bytes(N, K, &need);
    if (s != TSD_OK) return s;
    if (!d_w || !d_packed) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "null buffer");
    if ((uintptr_t)d_packed % 256) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "packed buffer must be 256-byte aligned");
    if (w_bytes != canonical_matrix_bytes(TSD_W_AFFINE8_G64, N, K))
        return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "canonical size mismatch");
    if (packed_bytes < need) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "packed buffer too small");
    hipError_t e = launch_pack_tiled(d_w, N, K, d_packed, N, 0, PACK_IDENTITY, 64, (hipStream_t)stream);
    return e == hipSuccess ? TSD_OK : hip_fail(nullptr, e, "pack");
}

tsd_status tsd_gemm_rows_scratch_bytes(int N, int K, int splits, size_t* out)
{
    if (!out || !mm16_supported(N, K) || splits < 1 || splits > MM_MAX_SPLIT || splits > K / 64)
        return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "bad shape or split count");
    // the operand rows (fp16 hi and lo), then the split-K slices
    *out = align256((size_t)MM_ROWS * K * 4) + (splits == 1 ? 0 : (size_t)splits * MM_ROWS * N * 4);
    return TSD_OK;
}

tsd_status tsd_gemm_rows(const void* d_packed, int N, int K, int B, const float* d_x, float* d_y, int splits,
                         void* d_scratch, size_t scratch_bytes, void* stream)
{
    size_t need = 0;
    tsd_status s = tsd_gemm_rows_scratch_bytes(N, K, splits, &need);
    if (s != TSD_OK) return s;
    if (B < 1 || B > MM_ROWS) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "B must be 1..16");
    if (!d_packed || !d_x || !d_y || !d_scratch) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "null buffer");
    if ((uintptr_t)d_scratch % 256 || (uintptr_t)d_packed % 256)
        return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "packed matrix and scratch must be 256-byte aligned");
    if (scratch_bytes < need) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "scratch too small");
    hipStream_t st = (hipStream_t)stream;
    TiledMat W = tiled_view((void*)d_packed, N, K);
    RowPrep p{};
    p.src = ROW_MAJOR;
    p.rows_src = d_x;
    p.K = K;
    p.B = B;
    p.act.hi = (__half*)d_scratch;
    p.act.lo = (__half*)d_scratch + (size_t)MM_ROWS * K;
    hipError_t e = launch_row_prep(p, st);   // rows past B are written as zeros
    MmIn in{};
    in.a = p.act;
    in.rows = B;
    Mm16Out o{};
    o.rows = B;
    o.ldy = N;
    if (splits == 1) {
        o.y = d_y;
        if (e == hipSuccess) e = launch_mm16(MM_STORE, W, in, 1, o, st);
    } else {
        o.y = (float*)((uint8_t*)d_scratch + align256((size_t)MM_ROWS * K * 4));
        o.slice = (long long)MM_ROWS * N;
        if (e == hipSuccess) e = launch_mm16(MM_STORE, W, in, splits, o, st);
        if (e == hipSuccess) e = launch_sum_slices(o.y, splits, o.slice, d_y, (long long)B * N, st);
    }
    return e == hipSuccess ? TSD_OK : hip_fail(nullptr, e, "gemm rows");
}

tsd_status tsd_sample_topk(const float* d_logits, int n, int top_k, float temperature, uint64_t seed, int row, int pos,
                           int pass, int32_t* d_out, void* stream)
{
    if (!d_logits || !d_out) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "null buffer");
    if (n <= 0 || row < 0 || pos < 0 || pass < 0) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "bad size or counter");
    if (!(temperature > 0.f) || !std::isfinite(temperature))
        return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "temperature must be positive and finite");
    tsd_sampling sv{};
    sv.mode = 1;
    sv.top_k = top_k;
    sv.temperature = temperature;
    sv.seed = seed;
    return tsd_sample(d_logits, n, &sv, nullptr, 0, row, pos, pass, d_out, stream);
}

tsd_status tsd_sample(const float* d_logits, int n, const tsd_sampling* s, const int32_t* d_hist, int n_hist, int row,
                      int pos, int pass, int32_t* d_out, void* stream)
{
    if (!d_logits || !d_out || !s) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "null argument");
    if (n <= 0 || row < 0 || pos < 0 || pass < 0) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "bad size or counter");
    if (n_hist < 0 || (n_hist > 0 && !d_hist)) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "bad history");
    std::string msg;
    tsd_status st = check_sampling(s, msg);
    if (st != TSD_OK) return fail(nullptr, st, msg);
    if (s->cfg) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "guidance combines a model's two rows: not a standalone draw");
    SampChain ch{};
    int draw = 0;
    if (!chain_of(s, n, true, &ch, &draw)) return fail(nullptr, TSD_ERR_UNSUPPORTED, "k <= 1024 and n <= 12288");
    if (!draw) ch = SampChain{1.f, 1, 0.f, 0.f, 1.f, SAMP_ORDER_T3};   // greedy: the largest logit
    SampleArgs a{};
    a.logits = d_logits;
    a.n = n;
    a.ch = ch;
    a.seed = s->seed;
    a.row = row;
    a.pass = pass;
    a.pos_value = pos;
    a.out = d_out;
    a.seq = d_hist;
    a.seq_stride = 1;
    a.n_seq = n_hist;
    hipError_t e = launch_sample(a, (hipStream_t)stream);
    return e == hipSuccess ? TSD_OK : hip_fail(nullptr, e, "sample");
}

tsd_status tsd_attention_scratch_bytes(int B, int H, int n_ctx, int hd, size_t* out)
{
    if (!out || B <= 0 || H <= 0 || n_ctx <= 0 || (hd != 64 && hd != 128))
        return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "bad shape");
    *out = attn_part_bytes(B, H, n_ctx, hd);
    return TSD_OK;
}

tsd_status tsd_attention(const float* d_q, const uint16_t* d_k, const uint16_t* d_v, int B, int H, int Hkv, int hd,
                         int n_keys, int n_ctx, float* d_out, void* d_scratch, size_t scratch_bytes, void* stream)
{
    size_t need = 0;
    tsd_status s = tsd_attention_scratch_bytes(B, H, n_ctx, hd, &need);
    if (s != TSD_OK) return s;
    if (Hkv <= 0 || H % Hkv || n_keys < 1 || n_keys > n_ctx) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "bad shape");
    if (!d_q || !d_k || !d_v || !d_out || !d_scratch) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "null buffer");
    if (scratch_bytes < need) return fail(nullptr, TSD_ERR_INVALID_ARGUMENT, "scratch too small");
    hipStream_t st = (hipStream_t)stream;
    AttnArgs a{};
    a.q = d_q;
    a.ldq = H * hd;
    a.k = (const __half*)d_k;
    a.v = (const __half*)d_v;
    a.out = d_out;
    a.ldo = H * hd;
    a.part = (float*)d_scratch;
    a.B = B;
    a.H = H;
    a.Hkv = Hkv;
    a.hd = hd;
    a.n_ctx = n_ctx;
    a.pos = nullptr;
    a.n_keys = n_keys;
    hipError_t e = launch_attention(a, st);
    if (e == hipSuccess) e = launch_attention_merge(a, n_keys, st);
    return e == hipSuccess ? TSD_OK : hip_fail(nullptr, e, "attention");
}

}  // extern "C"
