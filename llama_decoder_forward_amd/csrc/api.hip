// The C ABI: validation, buffer carving and the launch sequence of prefill, decode and the
// single-layer call.  No device memory is allocated here; every buffer is the caller's.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <new>
#include <vector>

#include "llama_mi355x.h"
#include "launch.hpp"

namespace {

// Nothing here may throw across the C ABI: the message buffer is a fixed array, and the
// two containers that grow (the layer table, the profiling events) catch allocation failure.
thread_local char g_last_error[512];

llama_status fail(llama_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t v, size_t a = kAlign) { return (v + a - 1) / a * a; }

int seq_stride_of(const llama_config& c) { return (int)align_up((size_t)c.max_seq, 64); }
size_t elem_size(const llama_config& c) { return c.dtype == LLAMA_BF16 ? 2 : 4; }

// Workspace regions, in order, each 256-byte aligned.
struct Layout {
    size_t flags, rope, x, h, q, attn, g, logits, partials, kpart, tokbuf, argmax, total;
};

Layout layout_of(const llama_config& c) {
    const size_t es = elem_size(c);
    const size_t rows = (size_t)std::max(c.max_tokens, c.max_batch);
    const size_t D = c.dim, HD = (size_t)c.n_heads * c.head_dim;
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
    L.flags = take(256);
    L.rope = take((size_t)c.max_seq * (c.head_dim / 2) * sizeof(float2));
    // GEMM inputs: the packed activation layout of the few-row GEMMs pads to 64 rows
    const size_t arows = std::max<size_t>(rows, 64);
    L.x = take(rows * D * 4);
    L.h = take(arows * D * es);
    L.q = take(rows * HD * es);
    L.attn = take(arows * HD * es);
    L.g = take(arows * (size_t)c.ffn_hidden * es);
    L.logits = take((size_t)c.max_batch * c.vocab_size * 4);
    L.partials = take(lk::decode_partials_bytes(c.max_batch, c.n_heads, c.head_dim, seq_stride_of(c)));
    // split-K sums of the residual GEMMs: on the few-row path (at most 64 rows) and on the
    // tiled path (two splits of at most LLAMA_TILED_SPLIT_MAX_ROWS rows)
    L.kpart = take(std::max((size_t)lk::LLAMA_MAX_KSPLITS * 64 * D * 4,
                            (size_t)2 * std::min<size_t>(rows, lk::LLAMA_TILED_SPLIT_MAX_ROWS) * D * 4));
    L.tokbuf = take((size_t)c.max_batch * 4);
    L.argmax = take(lk::argmax_scratch_bytes(c.max_batch, c.vocab_size));
    L.total = off;
    return L;
}

llama_status validate_config(const llama_config* c) {
    if (!c) return fail(LLAMA_ERR_INVALID_ARG, "config is NULL");
    if (c->dtype != LLAMA_BF16 && c->dtype != LLAMA_F32)
        return fail(LLAMA_ERR_DTYPE, "unknown dtype %d", (int)c->dtype);
    if (c->dim <= 0 || c->n_layers <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 ||
        c->head_dim <= 0 || c->ffn_hidden <= 0 || c->vocab_size <= 0)
        return fail(LLAMA_ERR_SHAPE, "model sizes must be positive");
    if (c->max_batch <= 0 || c->max_seq <= 0 || c->max_tokens <= 0)
        return fail(LLAMA_ERR_SHAPE, "max_batch, max_seq and max_tokens must be positive");
    if (c->n_heads % c->n_kv_heads != 0)
        return fail(LLAMA_ERR_SHAPE, "n_heads %d is not a multiple of n_kv_heads %d", c->n_heads, c->n_kv_heads);
    if ((long long)c->n_heads * c->head_dim != c->dim)
        return fail(LLAMA_ERR_SHAPE, "dim %d != n_heads %d * head_dim %d", c->dim, c->n_heads, c->head_dim);
    if (c->head_dim % 4 != 0 || c->head_dim > 256)
        return fail(LLAMA_ERR_SHAPE, "head_dim %d must be a multiple of 4 and <= 256", c->head_dim);
    if (!(c->norm_eps >= 0.0f) || !(c->rope_theta > 0.0f))
        return fail(LLAMA_ERR_SHAPE, "norm_eps must be >= 0 and rope_theta > 0");
    if (c->dim % 8 != 0 || c->ffn_hidden % 4 != 0 || c->vocab_size % 4 != 0)
        return fail(LLAMA_ERR_SHAPE, "dim must be a multiple of 8, ffn_hidden and vocab_size of 4");
    if (c->dtype == LLAMA_BF16 && (c->dim % 64 || c->ffn_hidden % 64 || c->vocab_size % 64))
        return fail(LLAMA_ERR_SHAPE, "bf16 needs dim, ffn_hidden and vocab_size multiples of 64");
    if (c->dim > 16384)
        return fail(LLAMA_ERR_SHAPE, "dim %d above 16384", c->dim);
    const long long rows = std::max(c->max_tokens, c->max_batch);
    if (rows * std::max(c->ffn_hidden, c->vocab_size) >= (1LL << 40))
        return fail(LLAMA_ERR_CAPACITY, "max_tokens too large");
    return LLAMA_OK;
}

}  // namespace

// Scratch of llama_decode_step_noalloc: one array per GPU, part of the library's code object,
// held until the process ends.  Host code never uses this name as an address (on the host
// it is only a stand-in for the symbol): the device address comes from hipGetSymbolAddress.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

struct llama_model {
    llama_config cfg;
    std::vector<llama_layer_weights> layers;
    const void* tok_embeddings = nullptr;
    const void* norm = nullptr;
    const void* output = nullptr;
    char* kv = nullptr;
    char* ws = nullptr;
    Layout L{};
    lk::Dt dt = lk::Dt::BF16;
    size_t es = 2;
    int seq_stride = 0;
    bool rope_ready = false;
    // residual-stream trace (llama_trace_hidden): [n_layers + 1][trace_rows][dim] or NULL
    float* trace = nullptr;
    int trace_rows = 0;
    // kernel timing (llama_profile_kernel)
    int prof_kind = LLAMA_KERNEL_NONE;
    std::vector<hipEvent_t> prof_events;  // pairs: start, stop
    size_t prof_used = 0;

    uint32_t* deverr() { return reinterpret_cast<uint32_t*>(ws + L.flags); }
    int* pos_ctr() { return reinterpret_cast<int*>(ws + L.flags + 64); }
    int* step_ctr() { return reinterpret_cast<int*>(ws + L.flags + 128); }
    float2* rope() { return reinterpret_cast<float2*>(ws + L.rope); }
    float* x() { return reinterpret_cast<float*>(ws + L.x); }
    void* h() { return ws + L.h; }
    void* q() { return ws + L.q; }
    void* attn() { return ws + L.attn; }
    void* g() { return ws + L.g; }
    float* logits_scratch() { return reinterpret_cast<float*>(ws + L.logits); }
    float* partials() { return reinterpret_cast<float*>(ws + L.partials); }
    float* kpart() { return reinterpret_cast<float*>(ws + L.kpart); }
    int* tokbuf() { return reinterpret_cast<int*>(ws + L.tokbuf); }
    void* argmax_scratch() { return ws + L.argmax; }
    float* trace_slot(int l) {
        return trace ? trace + (size_t)l * trace_rows * cfg.dim : nullptr;
    }
    size_t kv_layer_elems() const {
        return (size_t)cfg.max_batch * cfg.n_kv_heads * seq_stride * cfg.head_dim;
    }
    char* kc(int l) { return kv + (size_t)l * 2 * kv_layer_elems() * es; }
    char* vc(int l) { return kc(l) + kv_layer_elems() * es; }
};

namespace {

#define HIP_TRY(expr)                                                                       \
    do {                                                                                    \
        hipError_t e_ = (expr);                                                             \
        if (e_ != hipSuccess) return fail(LLAMA_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

// First-use set-up on the caller's stream: device flags, the rotary table, and a zero fill
// of the KV cache.  Attention reads whole 64-position blocks of the cache and gives the
// positions past a sequence's context probability 0; with every cached value finite (zero
// or written by a layer) those positions add exactly 0 * V.
llama_status ensure_rope(llama_model* m, hipStream_t s) {
    if (m->rope_ready) return LLAMA_OK;
    // the set-up must run, not only be recorded: a graph made of it would leave every later
    // eager call without a rotary table or a cleared cache
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    HIP_TRY(hipStreamIsCapturing(s, &cs));
    if (cs != hipStreamCaptureStatusNone)
        return fail(LLAMA_ERR_INVALID_ARG,
                    "the first call on a model runs its one-time set-up and cannot be recorded "
                    "into a stream capture; make one call outside the capture first");
    HIP_TRY(lk::zero_u32(m->deverr(), 64, s));  // device flags and counters (first 256 bytes)
    HIP_TRY(lk::rope_table(m->rope(), m->cfg.max_seq, m->cfg.head_dim, m->cfg.rope_theta, s));
    HIP_TRY(lk::zero_bytes(m->kv, llama_kv_cache_bytes(&m->cfg), s));
    m->rope_ready = true;
    return LLAMA_OK;
}

// Event pair around launches of the profiled kernel class (skipped during stream capture).
struct ProfScope {
    llama_model* m;
    hipStream_t s;
    hipEvent_t stop = nullptr;
    ProfScope(llama_model* m_, int kind, hipStream_t s_) : m(m_), s(s_) {
        if (m->prof_kind != kind || kind == LLAMA_KERNEL_NONE) return;
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return;
        if (m->prof_used + 2 > m->prof_events.size()) {
            for (int i = 0; i < 2; ++i) {
                hipEvent_t e;
                if (hipEventCreate(&e) != hipSuccess) return;
                try {
                    m->prof_events.push_back(e);
                } catch (...) {  // no profiling for this launch
                    (void)hipEventDestroy(e);
                    return;
                }
            }
        }
        hipEvent_t start = m->prof_events[m->prof_used];
        stop = m->prof_events[m->prof_used + 1];
        if (hipEventRecord(start, s) != hipSuccess) { stop = nullptr; return; }
        m->prof_used += 2;
    }
    ~ProfScope() {
        if (stop) (void)hipEventRecord(stop, s);
    }
};

// A is in the activation layout act_pack(M, N, K) selects (written so by its producer).
lk::GemmArgs<void> gemm_args(llama_model* m, const void* A, int lda, const void* w, int M, int N,
                             int K) {
    lk::GemmArgs<void> g{};
    g.A = A; g.lda = lda;
    g.a_pack = lk::act_pack(m->dt, M, N, K);
    g.W = WeightRows<void>{w, w, w, N, N, K};
    g.W3 = g.W;
    g.M = M; g.N = N; g.K = K;
    return g;
}

// Split-K sums of a residual GEMM not yet added to the residual stream (kpart, `splits`
// slices of `stride` floats); the next RMSNorm of that stream adds them.
struct Pending {
    int splits = 0;
    size_t stride = 0;
};

// Scratch of one call: split-K sums of the few-row residual GEMMs, decode-attention split
// partials, argmax partials and the logits of a decode step whose caller wants none.  The
// model's workspace holds them (Scratch::of); llama_decode_step_noalloc points them into the
// library's static scratch array instead.
struct Scratch {
    float* kpart;
    float* partials;
    void* argmax;
    float* logits;
    static Scratch of(llama_model* m) {
        return Scratch{m->kpart(), m->partials(), m->argmax_scratch(), m->logits_scratch()};
    }
};

// One decoder layer on rows = B*S tokens (article, sections 构建Transformer层 to 前馈神经网络层).
// pend, if given: on entry the sums pending on xin (then xin is written, folded), on return
// those pending on xout.  Without it xout is complete on return.
// trace: if set, receives the layer's input rows (after pending sums are added).
llama_status run_layer(llama_model* m, int l, const float* xin, float* xout, int B, int S,
                       int start_pos, const int* pos_dev, int pos_stride, int max_ctx, bool decode,
                       Pending* pend, const Scratch& scr, float* trace, hipStream_t s) {
    const llama_config& c = m->cfg;
    const llama_layer_weights& w = m->layers[l];
    const int T = B * S, D = c.dim, H = c.n_heads, G = c.n_kv_heads, d = c.head_dim;
    const int Nq = H * d, Nk = G * d;
    // each GEMM input is written in the layout its GEMM reads
    const int pk_qkv = lk::act_pack(m->dt, T, Nq + 2 * Nk, D);
    const int pk_wo = lk::act_pack(m->dt, T, D, Nq);
    const int pk_up = lk::act_pack(m->dt, T, c.ffn_hidden, D);
    const int pk_down = lk::act_pack(m->dt, T, D, c.ffn_hidden);

    {
        ProfScope ps(m, LLAMA_KERNEL_RMSNORM, s);
        const Pending in = pend ? *pend : Pending{};
        // pending sums exist only on the library's own residual buffer, which is writable
        HIP_TRY(lk::rmsnorm_fold(m->dt, xin, scr.kpart, in.splits, in.stride,
                                 const_cast<float*>(xin), 1, 0, w.attention_norm, m->h(), pk_qkv,
                                 T, D, c.norm_eps, s));
    }
    if (trace) HIP_TRY(lk::copy_rows(xin, 1, 0, trace, T, D, s));

    lk::GemmArgs<void> qkv = gemm_args(m, m->h(), D, w.wq, T, Nq + 2 * Nk, D);
    qkv.W = WeightRows<void>{w.wq, w.wk, w.wv, Nq, Nq + Nk, D};
    EpiQKV<void> eq{m->q(), m->kc(l), m->vc(l), m->rope(), Nq, Nk, d, S, start_pos, G,
                    m->seq_stride, pos_dev, pos_stride, c.max_seq,
                    lk::kv_cache_packed(m->dt, H, G, d) ? 1 : 0};
    {
        ProfScope ps(m, LLAMA_KERNEL_QKV, s);
        HIP_TRY(lk::gemm_qkv(m->dt, qkv, eq, s));
    }

    lk::AttnArgs aa{m->q(), m->kc(l), m->vc(l), m->attn(), pk_wo, B, S, start_pos, H, G, d,
                    m->seq_stride, pos_dev, pos_stride, c.max_seq, scr.partials, max_ctx};
    {
        ProfScope ps(m, LLAMA_KERNEL_ATTENTION, s);
        if (decode) HIP_TRY(lk::attention_decode(m->dt, aa, s));
        else HIP_TRY(lk::attention_prefill(m->dt, aa, s));
    }
    // WO: x_out = x_in + attn WO, added by the FFN RMSNorm when split over K
    const int wo_splits = lk::residual_splits(m->dt, T, D, Nq);
    {
        ProfScope ps(m, LLAMA_KERNEL_WO, s);
        const lk::GemmArgs<void> ga = gemm_args(m, m->attn(), Nq, w.wo, T, D, Nq);
        if (wo_splits > 0) HIP_TRY(lk::gemm_residual_split(m->dt, ga, scr.kpart, wo_splits, s));
        else HIP_TRY(lk::gemm_residual(m->dt, ga, EpiResidual{xin, xout, D}, s));
    }
    {
        ProfScope ps(m, LLAMA_KERNEL_RMSNORM, s);
        if (wo_splits > 0)
            HIP_TRY(lk::rmsnorm_fold(m->dt, xin, scr.kpart, wo_splits, (size_t)T * D, xout, 1, 0,
                                     w.ffn_norm, m->h(), pk_up, T, D, c.norm_eps, s));
        else
            HIP_TRY(lk::rmsnorm(m->dt, xout, 1, 0, w.ffn_norm, m->h(), pk_up, T, D, c.norm_eps, s));
    }
    lk::GemmArgs<void> ff = gemm_args(m, m->h(), D, w.w1, T, c.ffn_hidden, D);
    ff.W3 = WeightRows<void>{w.w3, w.w3, w.w3, c.ffn_hidden, c.ffn_hidden, D};
    {
        ProfScope ps(m, LLAMA_KERNEL_FFN_UP, s);
        HIP_TRY(lk::gemm_swiglu(m->dt, ff, m->g(), c.ffn_hidden, pk_down, s));
    }
    // W2: x_out += g W2, left pending (split over K) when the caller takes pending sums.  A
    // call that takes none (llama_layer_forward) leaves none: on the few-row path its W2 is
    // not split; on the tiled path the split sums are added at once, by the same fold the
    // next layer's norm applies, so that its output equals a prefill's layer output bit for
    // bit (the fold's normalised rows land in the scratch activation buffer, unused).
    int w2_splits = lk::residual_splits(m->dt, T, D, c.ffn_hidden);
    const bool fold_now = !pend && w2_splits > 0 && T > 64;
    if (!pend && !fold_now) w2_splits = 0;
    {
        ProfScope ps(m, LLAMA_KERNEL_FFN_DOWN, s);
        const lk::GemmArgs<void> ga = gemm_args(m, m->g(), c.ffn_hidden, w.w2, T, D, c.ffn_hidden);
        if (w2_splits > 0) HIP_TRY(lk::gemm_residual_split(m->dt, ga, scr.kpart, w2_splits, s));
        else HIP_TRY(lk::gemm_residual(m->dt, ga, EpiResidual{xout, xout, D}, s));
    }
    if (fold_now) {
        ProfScope ps(m, LLAMA_KERNEL_RMSNORM, s);
        HIP_TRY(lk::rmsnorm_fold(m->dt, xout, scr.kpart, w2_splits, (size_t)T * D, xout, 1, 0,
                                 w.ffn_norm, m->h(), pk_up, T, D, c.norm_eps, s));
    }
    if (pend) *pend = Pending{w2_splits, (size_t)T * D};
    return LLAMA_OK;
}

// Final RMSNorm and vocabulary projection of `rows` rows of x taken every `step` rows
// starting at `offset` (article, section 预测下一个输出).
// `pend`: split-K sums still pending on x (added to the rows read).  With a trace, the rows
// read (after the pending sums) go to the last trace slot.
llama_status run_head(llama_model* m, int rows, int step, int offset, const Pending& pend,
                      const Scratch& scr, float* logits, hipStream_t s) {
    const llama_config& c = m->cfg;
    {
        ProfScope ps(m, LLAMA_KERNEL_RMSNORM, s);
        HIP_TRY(lk::rmsnorm_fold(m->dt, m->x(), scr.kpart, pend.splits, pend.stride, m->x(), step,
                                 offset, m->norm, m->h(),
                                 lk::act_pack(m->dt, rows, c.vocab_size, c.dim), rows, c.dim,
                                 c.norm_eps, s));
    }
    if (m->trace)
        HIP_TRY(lk::copy_rows(m->x(), step, offset, m->trace_slot(c.n_layers), rows, c.dim, s));
    {
        ProfScope ps(m, LLAMA_KERNEL_LM_HEAD, s);
        HIP_TRY(lk::gemm_store_f32(m->dt, gemm_args(m, m->h(), c.dim, m->output, rows, c.vocab_size, c.dim),
                                   EpiStoreF32{logits, c.vocab_size}, s));
    }
    return LLAMA_OK;
}

// One decode step of B rows; position from `pos` or, if pos_dev is set, from device memory.
llama_status run_decode_step(llama_model* m, const int32_t* tokens, int B, int pos,
                             const int* pos_dev, int pos_stride, int max_ctx, float* logits,
                             int32_t* next, int32_t* log_out, const int* step_ctr,
                             const Scratch& scr, hipStream_t s) {
    const llama_config& c = m->cfg;
    HIP_TRY(lk::embed(m->dt, tokens, m->tok_embeddings, m->x(), B, c.dim, c.vocab_size, m->deverr(), s));
    Pending pend;
    for (int l = 0; l < c.n_layers; ++l) {
        llama_status st = run_layer(m, l, m->x(), m->x(), B, 1, pos, pos_dev, pos_stride, max_ctx,
                                    true, &pend, scr, m->trace_slot(l), s);
        if (st != LLAMA_OK) return st;
    }
    float* lg = logits ? logits : scr.logits;
    llama_status st = run_head(m, B, 1, 0, pend, scr, lg, s);
    if (st != LLAMA_OK) return st;
    HIP_TRY(lk::argmax(lg, B, 1, 0, c.vocab_size, next, log_out, B, step_ctr, scr.argmax,
                       m->deverr(), s));
    return LLAMA_OK;
}

}  // namespace

extern "C" {

size_t llama_kv_cache_bytes(const llama_config* cfg) {
    if (validate_config(cfg) != LLAMA_OK) return 0;
    return (size_t)cfg->n_layers * 2 * cfg->max_batch * cfg->n_kv_heads *
           (size_t)seq_stride_of(*cfg) * cfg->head_dim * elem_size(*cfg);
}

size_t llama_workspace_bytes(const llama_config* cfg) {
    if (validate_config(cfg) != LLAMA_OK) return 0;
    return layout_of(*cfg).total;
}

llama_status llama_init_weights(const llama_config* cfg, const llama_weights* w, void* kv_cache,
                                size_t kv_bytes, void* workspace, size_t ws_bytes,
                                llama_model** out) {
    if (!out) return fail(LLAMA_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    llama_status st = validate_config(cfg);
    if (st != LLAMA_OK) return st;
    if (!w || !w->tok_embeddings || !w->layers || !w->norm || !w->output)
        return fail(LLAMA_ERR_INVALID_ARG, "weights struct or one of its pointers is NULL");
    for (int l = 0; l < cfg->n_layers; ++l) {
        const llama_layer_weights& lw = w->layers[l];
        if (!lw.attention_norm || !lw.wq || !lw.wk || !lw.wv || !lw.wo || !lw.ffn_norm ||
            !lw.w1 || !lw.w3 || !lw.w2)
            return fail(LLAMA_ERR_INVALID_ARG, "layer %d has a NULL weight pointer", l);
    }
    if (!kv_cache || !workspace) return fail(LLAMA_ERR_INVALID_ARG, "kv_cache or workspace is NULL");
    if (((uintptr_t)kv_cache % kAlign) || ((uintptr_t)workspace % kAlign))
        return fail(LLAMA_ERR_INVALID_ARG, "kv_cache and workspace must be 256-byte aligned");
    if (kv_bytes < llama_kv_cache_bytes(cfg))
        return fail(LLAMA_ERR_CAPACITY, "kv_cache has %zu bytes, needs %zu", kv_bytes, llama_kv_cache_bytes(cfg));
    if (ws_bytes < llama_workspace_bytes(cfg))
        return fail(LLAMA_ERR_CAPACITY, "workspace has %zu bytes, needs %zu", ws_bytes, llama_workspace_bytes(cfg));
    llama_model* m = new (std::nothrow) llama_model();
    if (!m) return fail(LLAMA_ERR_ALLOC, "handle allocation failed");
    m->cfg = *cfg;
    try {
        m->layers.assign(w->layers, w->layers + cfg->n_layers);
    } catch (...) {
        delete m;
        return fail(LLAMA_ERR_ALLOC, "layer table allocation failed");
    }
    m->tok_embeddings = w->tok_embeddings;
    m->norm = w->norm;
    m->output = w->output;
    m->kv = static_cast<char*>(kv_cache);
    m->ws = static_cast<char*>(workspace);
    m->L = layout_of(*cfg);
    m->dt = cfg->dtype == LLAMA_BF16 ? lk::Dt::BF16 : lk::Dt::F32;
    m->es = elem_size(*cfg);
    m->seq_stride = seq_stride_of(*cfg);
    *out = m;
    return LLAMA_OK;
}

llama_status llama_prefill_at(llama_model* m, const int32_t* tokens, int32_t B, int32_t S,
                              int32_t start_pos, float* logits, int32_t all_positions,
                              int32_t* next_tokens, hipStream_t s) {
    if (!m || !tokens || !logits) return fail(LLAMA_ERR_INVALID_ARG, "NULL model, tokens or logits");
    const llama_config& c = m->cfg;
    if (B <= 0 || S <= 0) return fail(LLAMA_ERR_SHAPE, "B and S must be positive (B=%d S=%d)", B, S);
    if (B > c.max_batch) return fail(LLAMA_ERR_CAPACITY, "B=%d > max_batch=%d", B, c.max_batch);
    if (start_pos < 0 || (long long)start_pos + S > c.max_seq)
        return fail(LLAMA_ERR_CAPACITY, "start_pos=%d + S=%d exceeds max_seq=%d", start_pos, S, c.max_seq);
    if ((long long)B * S > c.max_tokens)
        return fail(LLAMA_ERR_CAPACITY, "B*S=%lld > max_tokens=%d", (long long)B * S, c.max_tokens);
    if (m->trace && (long long)B * S > m->trace_rows)
        return fail(LLAMA_ERR_CAPACITY, "B*S=%lld > the trace's %d rows", (long long)B * S, m->trace_rows);
    llama_status st = ensure_rope(m, s);
    if (st != LLAMA_OK) return st;
    const int T = B * S;
    const Scratch scr = Scratch::of(m);
    HIP_TRY(lk::embed(m->dt, tokens, m->tok_embeddings, m->x(), T, c.dim, c.vocab_size, m->deverr(), s));
    Pending pend;
    for (int l = 0; l < c.n_layers; ++l) {
        st = run_layer(m, l, m->x(), m->x(), B, S, start_pos, nullptr, 0, start_pos + S, false,
                       &pend, scr, m->trace_slot(l), s);
        if (st != LLAMA_OK) return st;
    }
    st = all_positions ? run_head(m, T, 1, 0, pend, scr, logits, s)
                       : run_head(m, B, S, S - 1, pend, scr, logits, s);
    if (st != LLAMA_OK || !next_tokens) return st;
    // greedy choice of each sequence's last position (article, section 预测下一个输出)
    HIP_TRY(lk::argmax(logits, B, all_positions ? S : 1, all_positions ? S - 1 : 0, c.vocab_size,
                       next_tokens, nullptr, 0, nullptr, scr.argmax, m->deverr(), s));
    return LLAMA_OK;
}

llama_status llama_prefill(llama_model* m, const int32_t* tokens, int32_t B, int32_t S,
                           float* logits, int32_t all_positions, hipStream_t s) {
    return llama_prefill_at(m, tokens, B, S, 0, logits, all_positions, nullptr, s);
}

llama_status llama_decode_step(llama_model* m, const int32_t* tokens, int32_t B, int32_t pos,
                               float* logits, int32_t* next_tokens, hipStream_t s) {
    if (!m || !tokens || !next_tokens) return fail(LLAMA_ERR_INVALID_ARG, "NULL model, tokens or next_tokens");
    const llama_config& c = m->cfg;
    if (B <= 0) return fail(LLAMA_ERR_SHAPE, "B must be positive (B=%d)", B);
    if (B > c.max_batch) return fail(LLAMA_ERR_CAPACITY, "B=%d > max_batch=%d", B, c.max_batch);
    if (pos < 0 || pos >= c.max_seq) return fail(LLAMA_ERR_CAPACITY, "pos=%d outside [0, max_seq=%d)", pos, c.max_seq);
    if (m->trace && B > m->trace_rows)
        return fail(LLAMA_ERR_CAPACITY, "B=%d > the trace's %d rows", B, m->trace_rows);
    llama_status st = ensure_rope(m, s);
    if (st != LLAMA_OK) return st;
    return run_decode_step(m, tokens, B, pos, nullptr, 0, pos + 1, logits, next_tokens, nullptr,
                           nullptr, Scratch::of(m), s);
}

// Device address of the static scratch array on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

llama_status scratch_base(void** out) {
    int dev = -1;
    HIP_TRY(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(LLAMA_ERR_HIP, "device %d out of range", dev);
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        try {
            std::lock_guard<std::mutex> lock(g_scratch_mu);
            p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
            if (!p) {
                HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
                if (!p) return fail(LLAMA_ERR_HIP, "no device address for the scratch array");
                g_scratch_ptr[dev].store(p, std::memory_order_release);
            }
        } catch (...) {
            return fail(LLAMA_ERR_HIP, "scratch look-up failed");
        }
    }
    *out = p;
    return LLAMA_OK;
}

llama_status llama_decode_step_noalloc(llama_model* m, const int32_t* tokens, int32_t B,
                                       int32_t pos, float* logits, int32_t* next_tokens,
                                       hipStream_t s) {
    if (!m || !tokens || !next_tokens) return fail(LLAMA_ERR_INVALID_ARG, "NULL model, tokens or next_tokens");
    const llama_config& c = m->cfg;
    if (B <= 0) return fail(LLAMA_ERR_SHAPE, "B must be positive (B=%d)", B);
    if (B > c.max_batch) return fail(LLAMA_ERR_CAPACITY, "B=%d > max_batch=%d", B, c.max_batch);
    if (pos < 0 || pos >= c.max_seq) return fail(LLAMA_ERR_CAPACITY, "pos=%d outside [0, max_seq=%d)", pos, c.max_seq);
    if (m->trace && B > m->trace_rows)
        return fail(LLAMA_ERR_CAPACITY, "B=%d > the trace's %d rows", B, m->trace_rows);
    // carve the scratch this call needs; every region is written before it is read, so
    // nothing is cleared
    const int D = c.dim;
    const int splits = std::max(lk::residual_splits(m->dt, B, D, c.n_heads * c.head_dim),
                                lk::residual_splits(m->dt, B, D, c.ffn_hidden));
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
    const size_t o_kpart = take((size_t)splits * B * D * 4);
    const size_t o_part = take(lk::decode_partials_bytes(B, c.n_heads, c.head_dim, m->seq_stride));
    const size_t o_arg = take(lk::argmax_scratch_bytes(B, c.vocab_size));
    const size_t o_log = logits ? off : take((size_t)B * c.vocab_size * 4);
    if (off > kNoAllocScratchBytes)
        return fail(LLAMA_ERR_CAPACITY, "this step needs %zu bytes of scratch; the static array "
                    "holds %zu", off, kNoAllocScratchBytes);
    void* base = nullptr;
    llama_status st = scratch_base(&base);
    if (st != LLAMA_OK) return st;
    st = ensure_rope(m, s);
    if (st != LLAMA_OK) return st;
    char* sb = static_cast<char*>(base);
    const Scratch scr{reinterpret_cast<float*>(sb + o_kpart), reinterpret_cast<float*>(sb + o_part),
                      sb + o_arg, reinterpret_cast<float*>(sb + o_log)};
    return run_decode_step(m, tokens, B, pos, nullptr, 0, pos + 1, logits, next_tokens, nullptr,
                           nullptr, scr, s);
}

llama_status llama_decode_step_ragged(llama_model* m, const int32_t* tokens, int32_t B,
                                      const int32_t* positions, float* logits,
                                      int32_t* next_tokens, hipStream_t s) {
    if (!m || !tokens || !positions || !next_tokens)
        return fail(LLAMA_ERR_INVALID_ARG, "NULL model, tokens, positions or next_tokens");
    const llama_config& c = m->cfg;
    if (B <= 0) return fail(LLAMA_ERR_SHAPE, "B must be positive (B=%d)", B);
    if (B > c.max_batch) return fail(LLAMA_ERR_CAPACITY, "B=%d > max_batch=%d", B, c.max_batch);
    if (m->trace && B > m->trace_rows)
        return fail(LLAMA_ERR_CAPACITY, "B=%d > the trace's %d rows", B, m->trace_rows);
    llama_status st = ensure_rope(m, s);
    if (st != LLAMA_OK) return st;
    // positions live on the device: checked there (flag for llama_sync_status), and every
    // kernel replaces an out-of-range one by 0, so that no access leaves the cache
    HIP_TRY(lk::check_positions(positions, B, c.max_seq, m->deverr(), s));
    return run_decode_step(m, tokens, B, 0, positions, 1, c.max_seq, logits, next_tokens, nullptr,
                           nullptr, Scratch::of(m), s);
}

llama_status llama_generate(llama_model* m, const int32_t* tokens, int32_t B, int32_t pos,
                            int32_t n_steps, int32_t* out_tokens, float* logits, hipStream_t s) {
    if (!m || !tokens || !out_tokens) return fail(LLAMA_ERR_INVALID_ARG, "NULL model, tokens or out_tokens");
    const llama_config& c = m->cfg;
    if (B <= 0 || n_steps < 0) return fail(LLAMA_ERR_SHAPE, "B must be positive and n_steps >= 0");
    if (B > c.max_batch) return fail(LLAMA_ERR_CAPACITY, "B=%d > max_batch=%d", B, c.max_batch);
    if (pos < 0 || (long long)pos + n_steps > c.max_seq)
        return fail(LLAMA_ERR_CAPACITY, "pos=%d + n_steps=%d exceeds max_seq=%d", pos, n_steps, c.max_seq);
    if (n_steps == 0) return LLAMA_OK;
    if (m->trace && B > m->trace_rows)
        return fail(LLAMA_ERR_CAPACITY, "B=%d > the trace's %d rows", B, m->trace_rows);
    llama_status st = ensure_rope(m, s);
    if (st != LLAMA_OK) return st;
    const int max_ctx = pos + n_steps;
    HIP_TRY(lk::copy_tokens(tokens, m->tokbuf(), B, s));
    HIP_TRY(lk::set_counters(m->pos_ctr(), pos, m->step_ctr(), s));
    // The step reads its position and step index from device memory, so the same launch
    // sequence repeats with no host round trip; the argmax of each step feeds the next.
    for (int k = 0; k < n_steps; ++k) {
        st = run_decode_step(m, m->tokbuf(), B, 0, m->pos_ctr(), 0, max_ctx,
                             logits ? logits + (size_t)k * B * c.vocab_size : nullptr,
                             m->tokbuf(), out_tokens, m->step_ctr(), Scratch::of(m), s);
        if (st != LLAMA_OK) return st;
        HIP_TRY(lk::bump_counters(m->pos_ctr(), m->step_ctr(), s));
    }
    return LLAMA_OK;
}

llama_status llama_layer_forward(llama_model* m, int32_t layer, const float* x_in, float* x_out,
                                 int32_t B, int32_t S, int32_t start_pos, hipStream_t s) {
    if (!m || !x_in || !x_out) return fail(LLAMA_ERR_INVALID_ARG, "NULL model, x_in or x_out");
    const llama_config& c = m->cfg;
    if (layer < 0 || layer >= c.n_layers)
        return fail(LLAMA_ERR_INVALID_ARG, "layer %d outside [0, %d)", layer, c.n_layers);
    if (B <= 0 || S <= 0) return fail(LLAMA_ERR_SHAPE, "B and S must be positive (B=%d S=%d)", B, S);
    if (B > c.max_batch) return fail(LLAMA_ERR_CAPACITY, "B=%d > max_batch=%d", B, c.max_batch);
    if (start_pos < 0 || (long long)start_pos + S > c.max_seq)
        return fail(LLAMA_ERR_CAPACITY, "start_pos=%d + S=%d exceeds max_seq=%d", start_pos, S, c.max_seq);
    if ((long long)B * S > c.max_tokens)
        return fail(LLAMA_ERR_CAPACITY, "B*S=%lld > max_tokens=%d", (long long)B * S, c.max_tokens);
    llama_status st = ensure_rope(m, s);
    if (st != LLAMA_OK) return st;
    return run_layer(m, layer, x_in, x_out, B, S, start_pos, nullptr, 0, start_pos + S, false,
                     nullptr, Scratch::of(m), nullptr, s);
}

llama_status llama_trace_hidden(llama_model* m, float* hidden, int32_t max_rows) {
    if (!m) return fail(LLAMA_ERR_INVALID_ARG, "NULL model");
    if (hidden && max_rows <= 0) return fail(LLAMA_ERR_SHAPE, "max_rows must be positive");
    if (hidden && ((uintptr_t)hidden % 16))
        return fail(LLAMA_ERR_INVALID_ARG, "hidden must be 16-byte aligned");
    m->trace = hidden;
    m->trace_rows = hidden ? max_rows : 0;
    return LLAMA_OK;
}

llama_status llama_sync_status(llama_model* m, hipStream_t s) {
    if (!m) return fail(LLAMA_ERR_INVALID_ARG, "NULL model");
    HIP_TRY(hipStreamSynchronize(s));
    uint32_t flags = 0;
    HIP_TRY(hipMemcpy(&flags, m->deverr(), sizeof flags, hipMemcpyDeviceToHost));
    if (flags) {
        HIP_TRY(hipMemset(m->deverr(), 0, sizeof flags));
        HIP_TRY(hipDeviceSynchronize());
        return fail(LLAMA_ERR_INVALID_ARG, "device reported %s%s%s",
                    (flags & DEVERR_TOKEN_RANGE) ? "token id outside [0, vocab) " : "",
                    (flags & DEVERR_NAN_LOGIT) ? "NaN logits " : "",
                    (flags & DEVERR_POSITION_RANGE) ? "position outside [0, max_seq)" : "");
    }
    return LLAMA_OK;
}

llama_status llama_profile_kernel(llama_model* m, llama_kernel kind) {
    if (!m) return fail(LLAMA_ERR_INVALID_ARG, "NULL model");
    if ((int)kind < LLAMA_KERNEL_NONE || (int)kind > LLAMA_KERNEL_RMSNORM)
        return fail(LLAMA_ERR_INVALID_ARG, "unknown kernel class %d", (int)kind);
    m->prof_kind = kind;
    m->prof_used = 0;
    return LLAMA_OK;
}

llama_status llama_profile_read(llama_model* m, double* total_ms, int32_t* launches) {
    if (!m || !total_ms || !launches) return fail(LLAMA_ERR_INVALID_ARG, "NULL argument");
    double total = 0.0;
    for (size_t i = 0; i + 1 < m->prof_used; i += 2) {
        HIP_TRY(hipEventSynchronize(m->prof_events[i + 1]));
        float ms = 0.0f;
        HIP_TRY(hipEventElapsedTime(&ms, m->prof_events[i], m->prof_events[i + 1]));
        total += ms;
    }
    *total_ms = total;
    *launches = (int32_t)(m->prof_used / 2);
    m->prof_used = 0;
    return LLAMA_OK;
}

void llama_free(llama_model* m) {
    if (!m) return;
    for (hipEvent_t e : m->prof_events) (void)hipEventDestroy(e);
    delete m;
}

const char* llama_last_error(void) { return g_last_error; }

}  // extern "C"
