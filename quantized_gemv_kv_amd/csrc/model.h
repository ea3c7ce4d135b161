// model.h — the model object behind the C ABI (internal; shared by model.hip, which runs the
// batch-1 GPT2/LLAMA step, and talker.hip, which runs the batched Talker + code-predictor frame).
#pragma once

#include <string>
#include <vector>

#include "frame.h"
#include "tsd.h"

namespace tsd {

struct LayerW {
    PackedMat qkv, o, fc, down;            // fc = fc (GPT-2) or interleaved gate/up (Llama, Talker)
    float *n1g = nullptr, *n1b = nullptr, *n2g = nullptr, *n2b = nullptr;
    float *bqkv = nullptr, *bo = nullptr, *bfc = nullptr, *bdown = nullptr;
    // GPT-2, for the persistent step: c = W g and d = W beta + bias of the two LayerNorm-fed
    // products (QKV with n1, FC with n2), so that the step can normalise after the dot product
    float *cqkv = nullptr, *dqkv = nullptr, *cfc = nullptr, *dfc = nullptr;
};

// bump planner over the workspace: the same walk sizes it and lays it out
struct Planner {
    uint8_t* base;
    size_t off = 0;
    explicit Planner(uint8_t* b) : base(b) {}
    void* take(size_t bytes)
    {
        off = align256(off);
        void* p = base ? base + off : nullptr;
        off += bytes;
        return p;
    }
    // move to the next device address that is a multiple of a (a power of two); when only sizing
    // (no base), reserve the most that can take
    void align_abs(size_t a)
    {
        off += base ? (a - ((size_t)(uintptr_t)base + off) % a) % a : a - 1;
    }
};

// a LLAMA-shaped layer of the batched frame: tiled matrices (qkv rows in RoPE pairs, gate/up
// interleaved), RMSNorm gains
struct TLayerW {
    TiledMat qkv, o, fc, down;
    float *n1g = nullptr, *n2g = nullptr;
};

inline TiledMat take_tiled(Planner& P, int N, int K)
{
    void* p = P.take(tiled_bytes(N, K));
    if (!p) {
        TiledMat m{};
        m.N = N;
        m.K = K;
        return m;
    }
    return tiled_view(p, N, K);
}

inline PackedMat take_mat(Planner& P, int f, int N, int K)
{
    PackedLayout L = packed_layout(f, N, K);
    void* p = P.take(L.total);
    if (!p) {
        PackedMat m{};
        m.N = N;
        m.K = K;
        return m;
    }
    return packed_view(f, p, N, K);
}

// the model's control words (64 words in the workspace): the epoch base (the persistent step:
// launches completed; TALKER_CP: frames completed, which tags the fused QKV + attention launches)
// and the sticky time-out word of the bounded waits; the sticky rejected-input word that every
// state-writing kernel checks (kernels.h launch_set_input)
enum { CTL_EPOCH = 0, CTL_ABORT = 1, CTL_BAD_INPUT = 2, CTL_WORDS = 64 };
constexpr long long STEP_SPIN_LIMIT = 2000000;   // 20 ms of the 100 MHz clock per wait

// kernel kinds a timing probe can bracket
enum { KIND_QKV = 0, KIND_ATTN = 1, KIND_OPROJ = 2, KIND_FC = 3, KIND_DOWN = 4, KIND_HEAD = 5, KIND_STEP = 6, TSD_KERNEL_KINDS = 7 };

struct Probe {
    int kind = -1;
    hipEvent_t* ev = nullptr;   // quadruples, consumed in launch order: empty bracket, kernel bracket
    int next = 0;
};

// brackets one launch with probe events when its kind is the probed one
struct Bracket {
    Probe* p;
    hipStream_t st;
    bool on;
    Bracket(Probe* pr, int kind, hipStream_t s) : p(pr), st(s), on(pr && pr->kind == kind)
    {
        if (!on) return;
        (void)hipEventRecord(p->ev[p->next], st);       // empty bracket: the cost of bracketing
        (void)hipEventRecord(p->ev[p->next + 1], st);
        (void)hipEventRecord(p->ev[p->next + 2], st);   // the kernel
    }
    ~Bracket()
    {
        if (on) (void)hipEventRecord(p->ev[p->next + 3], st), p->next += 4;
    }
};

}  // namespace tsd

struct tsd_model {
    tsd_config c{};
    tsd_sampling samp{};
    hipStream_t st = nullptr;
    uint8_t* ws = nullptr;
    size_t ws_bytes = 0;
    int tpp = 1;          // tokens per position
    int vmax = 0;
    int qkv_rows = 0;
    std::vector<tsd::LayerW> L;
    const float* emb[16] = {};
    int emb_rows[16] = {};
    const float* wpe = nullptr;
    float *nfg = nullptr, *nfb = nullptr;
    float *hc = nullptr, *hdv = nullptr;   // GPT-2: head W nfg and W nfb (as cqkv / dqkv)
    tsd::PackedMat head{};
    __half *kc = nullptr, *vc = nullptr;
    size_t kv_layer_elems = 0;
    float *x = nullptr, *qkv = nullptr, *attn = nullptr, *h = nullptr, *logits = nullptr, *part = nullptr;
    float2* rope = nullptr;
    int rope_rows = 0;
    unsigned long long* best = nullptr;   // per head-workgroup best keys
    int *pos = nullptr, *tok = nullptr, *hist = nullptr, *dbg_pos = nullptr;
    // persistent step: kernel (null: one launch per operator), grid, exchange state
    const void* step_fn = nullptr;
    int n_wg = 0;
    tsd::StepArgs sa{};
    tsd::StepArgs* d_sa = nullptr;    // sa in the workspace (the kernel reads it there)
    uint64_t* xbuf = nullptr;
    size_t xbuf_words = 0;
    uint32_t* ctl = nullptr;          // [0] epoch base (launches), [1] abort word
    uint64_t launches = 0, max_launches = 0;
    bool frame_fused = false;         // TALKER_CP: the QKV product and attention share a launch
    bool io_since_sync = false;       // a step or prompt since the last tsd_synchronize took or gave ids through caller buffers
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    // TALKER_CP: batch rows through the matrix-core GEMM; the code predictor's own layers,
    // norm, heads and cache; the graph of a frame without head and predictor (prefill)
    std::vector<tsd::TLayerW> Lt, Lc;   // Talker and predictor layers
    tsd::TiledMat t_head{};
    float* cp_nfg = nullptr;
    tsd::TiledMat cp_head[16] = {};
    __half *ckc = nullptr, *cvc = nullptr;
    size_t ckv_layer_elems = 0;
    float* xc = nullptr;              // predictor residual stream [16][d]
    tsd::Act16 act{}, act2{};         // GEMM operands, fp16 hi/lo of 16 rows (il_act layout): two,
                                      // so that an epilogue can write the next while others read one
    float* ssq = nullptr;             // partial row sums of squares of a norm's input [MM_MAX_SSQ][16]
    hipGraph_t graph_talker = nullptr;
    hipGraphExec_t exec_talker = nullptr;
    int kind_launches[tsd::TSD_KERNEL_KINDS] = {};
    // timing probes: events around every launch of one kernel kind
    std::vector<hipEvent_t> probe_ev[tsd::TSD_KERNEL_KINDS];
    int n_past = 0;
    int top_k = 0;                    // effective k of the main head's draw
    // the sampler chain as the kernels run it: the main head (token, or Talker code 0) and the
    // code predictor's heads (no repetition penalty); draw 0 = the greedy argmax
    tsd::SampChain chain{}, cp_chain{};
    int draw = 0, cp_draw = 0;
    int* seq = nullptr;               // [n_ctx][batch] the token (code 0) consumed at each position
    // prompt pass (GPT2/LLAMA): row buffers for up to pf_rows rows (batch rows x positions)
    int pf_rows = 0;
    float *pf_x = nullptr, *pf_q = nullptr;          // residual stream [rows][d], queries [rows][H hd]
    __half *pf_ahi = nullptr, *pf_alo = nullptr;     // operand [rows][max(d, H hd)]
    __half *pf_hhi = nullptr, *pf_hlo = nullptr;     // operand [rows][d_ff]
    std::string err;
};

namespace tsd {

tsd_status fail(tsd_model* m, tsd_status s, const std::string& msg);
tsd_status hip_fail(tsd_model* m, hipError_t e, const char* what);
// the scale group of a weight format along K (64 or 32), and the bytes of a canonical N x K blob
int group_of(int f);
size_t canonical_matrix_bytes(int f, int N, int K);

#define HIP_TRY(m, expr, what)                              \
    do {                                                    \
        hipError_t e_ = (expr);                             \
        if (e_ != hipSuccess) return hip_fail(m, e_, what); \
    } while (0)

// ---- TALKER_CP (talker.hip) -------------------------------------------------------------------
tsd_status talker_validate(const tsd_config* c, std::string& msg);
void talker_canonical_sizes(const tsd_config* c, size_t (*matrix_bytes)(int, int, int), std::vector<size_t>& sz);
size_t talker_plan(tsd_model* m, const tsd_config* c, uint8_t* base);
tsd_status talker_pack(tsd_model* m, const tsd_tensor* w);
// one frame: Talker layers, head and code c_0; with_cp: the predictor's passes for codes
// 1..C-1 and the history append.  Without: only the Talker's cache is advanced (prefill).
hipError_t talker_enqueue(tsd_model* m, hipStream_t st, bool with_cp, Probe* pr = nullptr);
// Talker layer l on the rows d_x ([batch][d] row-major) at *pos, the result left in m->x
// (tsd_layer_forward)
hipError_t talker_layer(tsd_model* m, int l, hipStream_t st, const float* d_x, const int* pos);
// launches of each kind in one frame
void talker_kind_launches(const tsd_model* m, int* out);

}  // namespace tsd
