// qwen3_api.cpp -- the C ABI (include/qwen3.h): seat handle, host-side argument
// checks (all before the first enqueue), workspace layout and the per-layer
// launch sequence.
//
// Launch sequence of one forward call of T tokens ("maya2_mlx/backbone.py",
// Backbone.forward, with its deferred MLP residual `pend`):
//   layer 0:   y = RMSNorm(x)                              add_rmsnorm
//   layer l>0: h = rho(h + pend); y = RMSNorm(h)           add_rmsnorm (fused add; for T > 1 after a
//                                                          dense MLP the add already ran in down)
//              qkv = rho(y Wqkv^T)                         linear (GEMV / MFMA GEMM)
//              q, K[p], V[p] = norm + RoPE + cache write    qknorm_rope_kv (bf16, T large enough for
//                                                          256 x 128 tiles: the projection's epilogue)
//              a = attention(q, K[0..p], V[0..p])           split-K decode | flash prefill
//              h = rho(h + rho(a Wo^T))                    linear, residual epilogue
//              y2 = RMSNorm(h)                             add_rmsnorm
//              dense: m = swiglu(y2 Wgu^T)                 linear, SwiGLU epilogue
//                     pend = rho(m Wdown^T)                linear (T > 1: h = rho(h + pend) in its
//                                                          residual epilogue, same roundings)
//              MoE:   pend = moe(y2)                       router/top-k/sort/experts/combine
//   (in an MoE configuration a layer with a router is sparse, one without runs the dense MLP)
//   after the last layer: out = RMSNorm(rho(h + pend))     add_rmsnorm
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include "../../include/qwen3.h"
#include "../../include/qwen3_ops.h"
#include "kernels.h"

using namespace q3;

struct qwen3_handle {
    qwen3_config cfg;
    std::vector<qwen3_layer_weights> layers;
    const void *embed = nullptr, *final_norm = nullptr, *cos_t = nullptr, *sin_t = nullptr;
    char *kc = nullptr, *vc = nullptr;
    char *ws = nullptr;
    size_t ws_bytes = 0;
    hipStream_t stream = nullptr;
    int length = 0;
    std::string err;
    // workspace pieces
    void *h = nullptr, *h2 = nullptr, *y = nullptr, *qkv = nullptr, *q = nullptr, *a = nullptr, *m = nullptr, *pend = nullptr;
    void *tmp = nullptr;
    float *attn_ws = nullptr;
    int *dev_err = nullptr;
    unsigned long long *head_keys = nullptr;  // greedy-token keys, one per row
    int32_t *moe_idx = nullptr;
    void *moe_w = nullptr, *moe_ws = nullptr;
    // persistent decode step (the dense bf16 / 8-bit shapes and the MoE shape it supports)
    void *mk_ws = nullptr;
    bool mk_ready = false, mk_moe = false;
    int decode_path = 0;  // 0 auto, 1 separate kernels, 2 persistent kernel
    // measurement: event pairs around launches of one kernel kind
    static constexpr int NKIND = 6;
    bool timer_on[NKIND] = {};
    int timer_used[NKIND] = {};
    std::vector<std::pair<hipEvent_t, hipEvent_t>> timer_ev[NKIND];
    ~qwen3_handle() {
        for (auto &v : timer_ev)
            for (auto &p : v) {
                (void)hipEventDestroy(p.first);
                (void)hipEventDestroy(p.second);
            }
    }
};

namespace {

size_t al256(size_t b) { return (b + 255) & ~(size_t)255; }

struct Layout {
    size_t h, h2, y, qkv, q, a, m, pend, tmp, attn, cos_t, sin_t, err, head_keys, moe_idx, moe_w, moe_ws, mk, total;
};

size_t esize(const qwen3_config &c) { return c.dtype == QWEN3_BF16 ? 2 : 4; }

// A configuration the persistent MoE decode kernel is built for (its layers must all be MoE too)
bool moe_mk_config(const qwen3_config &c) {
    return c.n_experts > 0 && decode_moe_supported(c.n_layers, c.dtype, c.quant_bits, c.hidden, c.n_heads, c.n_kv_heads,
                                                   c.head_dim, c.n_experts, c.top_k, c.moe_intermediate, c.capacity);
}

Layout layout(const qwen3_config &c) {
    Layout L{};
    const size_t es = esize(c), Tm = (size_t)c.max_tokens, hid = (size_t)c.hidden;
    const size_t HD = (size_t)c.n_heads * c.head_dim, nqkv = (size_t)(c.n_heads + 2 * c.n_kv_heads) * c.head_dim;
    size_t o = 0;
    auto take = [&](size_t b) {
        const size_t r = o;
        o += al256(b);
        return r;
    };
    L.h = take(Tm * hid * es);
    L.h2 = take(Tm * hid * es);
    L.y = take(Tm * hid * es);
    L.qkv = take(Tm * nqkv * es);
    L.q = take(Tm * HD * es);
    L.a = take(Tm * HD * es);
    L.m = take(Tm * (size_t)(c.intermediate > 0 ? c.intermediate : 1) * es);
    L.pend = take(Tm * hid * es);
    L.tmp = take(Tm * hid * es);
    L.attn = take(attention_workspace(c.max_tokens, c.n_heads, c.n_kv_heads, c.head_dim, c.capacity));
    L.cos_t = take((size_t)c.capacity * c.head_dim * es);
    L.sin_t = take((size_t)c.capacity * c.head_dim * es);
    L.err = take(256);
    L.head_keys = take(Tm * 64 * 8);  // 64 key slots per row (kernels_head.hip)
    if (c.n_experts > 0) {
        L.moe_idx = take(Tm * c.top_k * 4);
        L.moe_w = take(Tm * c.top_k * es);
        L.moe_ws = take(moe_workspace(c.max_tokens, c.hidden, c.n_experts, c.top_k, c.moe_intermediate, c.dtype));
    }
    if (decode_mk_supported(c.n_layers, c.dtype, c.n_experts, c.quant_bits, c.hidden, c.n_heads, c.n_kv_heads, c.head_dim,
                            c.intermediate, c.capacity))
        L.mk = take(decode_mk_workspace(c.n_layers, c.n_heads, c.n_kv_heads, c.hidden, c.intermediate));
    else if (moe_mk_config(c))
        L.mk = take(decode_moe_workspace(c.n_layers, c.n_heads, c.n_kv_heads));
    L.total = o;
    return L;
}

int fail(qwen3_handle *h, int code, const char *fmt, ...) {
    if (h) {
        char buf[512];
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(buf, sizeof buf, fmt, ap);
        va_end(ap);
        h->err = buf;
    }
    return code;
}

// Configuration checks shared by qwen3_workspace_bytes and qwen3_init.
int check_config(const qwen3_config *c, std::string *why) {
    auto bad = [&](int code, const char *msg) {
        if (why) *why = msg;
        return code;
    };
    if (!c) return bad(QWEN3_ERR_ARG, "null config");
    if (c->dtype != QWEN3_BF16 && c->dtype != QWEN3_FP32)
        return bad(QWEN3_ERR_DTYPE, "dtype must be bf16 (production) or fp32 (strict)");
    if (c->n_layers < 1 || c->hidden < 1 || c->n_heads < 1 || c->n_kv_heads < 1 || c->capacity < 1 ||
        c->max_tokens < 1)
        return bad(QWEN3_ERR_ARG, "layer count, sizes, capacity and max_tokens must be positive");
    if (c->head_dim != 64 && c->head_dim != 128) return bad(QWEN3_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    if (c->n_heads % c->n_kv_heads) return bad(QWEN3_ERR_ARG, "n_heads must be a multiple of n_kv_heads");
    const int G = c->n_heads / c->n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8) return bad(QWEN3_ERR_UNSUPPORTED, "n_heads / n_kv_heads must be 1, 2, 4 or 8");
    if (c->hidden % 128) return bad(QWEN3_ERR_UNSUPPORTED, "hidden must be a multiple of 128");
    if (!(c->rms_eps >= 0.0f)) return bad(QWEN3_ERR_ARG, "rms_eps must be >= 0");
    if (!(c->rope_theta > 1.0)) return bad(QWEN3_ERR_ARG, "rope_theta must be > 1");
    if (c->sliding_window < 0) return bad(QWEN3_ERR_ARG, "sliding_window must be 0 (causal) or positive");
    if (c->n_experts > 0) {
        if (c->n_experts > 256 || c->top_k < 1 || c->top_k > 16 || c->top_k > c->n_experts)
            return bad(QWEN3_ERR_UNSUPPORTED, "MoE needs 1 <= top_k <= min(16, n_experts) and n_experts <= 256");
        if (c->moe_intermediate < 64 || c->moe_intermediate % 64)
            return bad(QWEN3_ERR_UNSUPPORTED, "moe_intermediate must be a positive multiple of 64");
        if (c->intermediate != 0 && (c->intermediate < 64 || c->intermediate % 64))
            return bad(QWEN3_ERR_UNSUPPORTED, "intermediate must be 0 or a positive multiple of 64");
    } else {
        if (c->intermediate < 64 || c->intermediate % 64)
            return bad(QWEN3_ERR_UNSUPPORTED, "intermediate must be a positive multiple of 64");
    }
    if (c->quant_bits != 0) {
        if (c->quant_bits != 8 || c->quant_group != 64)
            return bad(QWEN3_ERR_UNSUPPORTED, "quantised weights must be 8-bit in groups of 64");
        if (c->dtype != QWEN3_BF16) return bad(QWEN3_ERR_UNSUPPORTED, "quantised weights need the bf16 dtype");
        if (c->hidden > 8192 || c->n_heads * c->head_dim > 8192 || c->intermediate > 8192)
            return bad(QWEN3_ERR_UNSUPPORTED, "quantised projections need input widths <= 8192");
    }
    return QWEN3_OK;
}

bool is_q8(const qwen3_handle *h) { return h->cfg.quant_bits == 8; }

// Device buffers are read and written in 16-byte vector accesses (weight rows, cache rows,
// table rows, activation rows); NULL counts as aligned.
bool al16(const void *p) { return ((uintptr_t)p & 15) == 0; }
bool al_elem(const void *p, size_t es) { return ((uintptr_t)p & (es - 1)) == 0; }

// The first misaligned device pointer of the weights and caches, or nullptr.
const char *misaligned(const qwen3_config *cfg, const qwen3_weights *w, const void *kc, const void *vc) {
    if (!al16(kc)) return "k_cache";
    if (!al16(vc)) return "v_cache";
    if (!al16(w->embed)) return "embed";
    if (!al16(w->final_norm)) return "final_norm";
    if (!al16(w->rope_cos) || !al16(w->rope_sin)) return "rope table";
    static const char *names[] = {"in_norm",  "post_norm",     "q_norm",        "k_norm",     "qkv",
                                  "o",        "gate_up",       "down",          "qkv_s",      "qkv_b",
                                  "o_s",      "o_b",           "gate_up_s",     "gate_up_b",  "down_s",
                                  "down_b",   "router",        "exp_gate_up",   "exp_down",   "router_s",
                                  "router_b", "exp_gate_up_s", "exp_gate_up_b", "exp_down_s", "exp_down_b",
                                  "qkv_bias"};
    static_assert(sizeof(qwen3_layer_weights) == sizeof(names) / sizeof(names[0]) * sizeof(void *),
                  "every layer field is a pointer named above");
    for (int l = 0; l < cfg->n_layers; ++l) {
        const void *const *f = (const void *const *)&w->layers[l];
        for (size_t i = 0; i < sizeof(names) / sizeof(names[0]); ++i)
            if (!al16(f[i])) return names[i];
    }
    return nullptr;
}

// Layer kind: sparse MoE block iff the configuration has experts and the layer a router.
bool moe_layer(const qwen3_config &c, const qwen3_layer_weights &L) { return c.n_experts > 0 && L.router; }

MoeWeights moe_weights(const qwen3_handle *h, const qwen3_layer_weights &L) {
    return MoeWeights{L.router, L.router_s, L.router_b, L.exp_gate_up, L.exp_gate_up_s, L.exp_gate_up_b,
                      L.exp_down, L.exp_down_s, L.exp_down_b, is_q8(h)};
}

hipError_t moe(qwen3_handle *h, const qwen3_layer_weights &L, const void *x, int T, int32_t *idx, void *w, void *out) {
    const qwen3_config &c = h->cfg;
    return launch_moe(c.dtype, x, T, c.hidden, moe_weights(h, L), c.n_experts, c.top_k, c.norm_topk_prob,
                      c.moe_intermediate, idx, w, out, h->moe_ws, h->stream);
}

hipError_t linear(qwen3_handle *h, const void *x, int M, int K, const void *W, const void *Ws, const void *Wb, int N,
                  int epi, const void *res, void *out) {
    if (is_q8(h))
        return launch_linear_q8(x, M, K, (const uint8_t *)W, Ws, Wb, h->cfg.quant_group, N, epi, res, out, h->stream);
    return launch_linear(h->cfg.dtype, x, M, K, W, N, epi, res, out, h->stream);
}

enum { K_QKV = 0, K_O = 1, K_GU = 2, K_DOWN = 3, K_ATTN = 4, K_STEP = 5 };

// Record the start (begin = true) or end event of a timed launch of `kind`.
hipError_t mark(qwen3_handle *h, int kind, bool begin) {
    if (!h->timer_on[kind]) return hipSuccess;
    auto &v = h->timer_ev[kind];
    int &used = h->timer_used[kind];
    if (begin) {
        if ((size_t)used == v.size()) {
            hipEvent_t a, b;
            hipError_t e = hipEventCreate(&a);
            if (e != hipSuccess) return e;
            e = hipEventCreate(&b);
            if (e != hipSuccess) return e;
            v.push_back({a, b});
        }
        return hipEventRecord(v[used].first, h->stream);
    }
    const hipError_t e = hipEventRecord(v[used].second, h->stream);
    ++used;
    return e;
}

#define HIPCHECK(h, call)                                                                                    \
    do {                                                                                                     \
        hipError_t e_ = (call);                                                                              \
        if (e_ != hipSuccess) return fail(h, QWEN3_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_));       \
    } while (0)

hipError_t linear_norm(qwen3_handle *h, const void *h_in, const void *res, const void *nw, void *h_out, int K,
                       const void *W, const void *Ws, const void *Wb, int N, int epi, void *out) {
    if (is_q8(h))
        return launch_linear_q8_norm(h_in, res, nw, h->cfg.rms_eps, h_out, K, (const uint8_t *)W, Ws, Wb,
                                     h->cfg.quant_group, N, epi, out, h->stream);
    return launch_linear_norm(h->cfg.dtype, h_in, res, nw, h->cfg.rms_eps, h_out, K, W, N, epi, out, h->stream);
}

// T == 1: the norms ride in the projections' prologues and the per-head q/k norm, RoPE
// and cache write in the split-K attention kernel; two hidden-state buffers alternate so
// the block that writes h = rho(h + pend) never overwrites a row other blocks still read.
int run_decode(qwen3_handle *h, const void *x, void *out) {
    const qwen3_config &c = h->cfg;
    if (h->mk_ready && h->decode_path != 1) {
        HIPCHECK(h, mark(h, K_STEP, true));
        if (h->mk_moe)
            HIPCHECK(h, launch_decode_moe(h->mk_ws, c.n_layers, c.n_heads, c.n_kv_heads, c.n_experts, c.norm_topk_prob,
                                          is_q8(h), c.capacity, h->length, c.sliding_window, c.rms_eps, x, out, h->final_norm,
                                          h->cos_t, h->sin_t, h->kc, h->vc, h->dev_err, h->stream));
        else
            HIPCHECK(h, launch_decode_mk(h->mk_ws, c.n_layers, c.n_heads, c.n_kv_heads, c.hidden, c.intermediate,
                                         is_q8(h), c.capacity, h->length, c.sliding_window, c.rms_eps, x, out,
                                         h->final_norm, h->cos_t, h->sin_t, h->kc, h->vc, h->dev_err, h->stream));
        HIPCHECK(h, mark(h, K_STEP, false));
        return QWEN3_OK;
    }
    const int dt = c.dtype, hid = c.hidden, H = c.n_heads, KV = c.n_kv_heads, D = c.head_dim;
    const int nqkv = (H + 2 * KV) * D, p0 = h->length;
    const size_t es = esize(c), layer_kv = (size_t)KV * c.capacity * D * es;
    hipStream_t s = h->stream;
    void *hb[2] = {h->h, h->h2};
    void *hcur = nullptr;
    for (int l = 0; l < c.n_layers; ++l) {
        const qwen3_layer_weights &L = h->layers[l];
        void *hnext = l == 0 ? hb[0] : (hcur == hb[0] ? hb[1] : hb[0]);
        HIPCHECK(h, mark(h, K_QKV, true));
        if (l == 0)
            HIPCHECK(h, linear_norm(h, x, nullptr, L.in_norm, nullptr, hid, L.qkv, L.qkv_s, L.qkv_b, nqkv, EPI_STORE,
                                    h->qkv));
        else
            HIPCHECK(h, linear_norm(h, hcur, h->pend, L.in_norm, hnext, hid, L.qkv, L.qkv_s, L.qkv_b, nqkv, EPI_STORE,
                                    h->qkv));
        HIPCHECK(h, mark(h, K_QKV, false));
        HIPCHECK(h, mark(h, K_ATTN, true));
        HIPCHECK(h, launch_attention_decode_fused(dt, h->qkv, H, KV, D, L.q_norm, L.k_norm, L.qkv_bias, c.rms_eps,
                                                  h->cos_t, h->sin_t, p0, c.capacity, c.sliding_window,
                                                  h->kc + l * layer_kv, h->vc + l * layer_kv, h->a, h->attn_ws, s));
        HIPCHECK(h, mark(h, K_ATTN, false));
        HIPCHECK(h, mark(h, K_O, true));
        HIPCHECK(h, linear(h, h->a, 1, H * D, L.o, L.o_s, L.o_b, hid, EPI_RESID, l == 0 ? x : hnext, hnext));
        HIPCHECK(h, mark(h, K_O, false));
        hcur = hnext;
        if (moe_layer(c, L)) {  // post-attention norm in the router's and experts' prologues
            HIPCHECK(h, launch_moe_norm1(dt, hcur, L.post_norm, c.rms_eps, hid, moe_weights(h, L), c.n_experts,
                                         c.top_k, c.norm_topk_prob, c.moe_intermediate, h->moe_idx, h->moe_w,
                                         h->pend, h->moe_ws, s));
        } else {
            HIPCHECK(h, mark(h, K_GU, true));
            HIPCHECK(h, linear_norm(h, hcur, nullptr, L.post_norm, nullptr, hid, L.gate_up, L.gate_up_s, L.gate_up_b,
                                    c.intermediate, EPI_SWIGLU, h->m));
            HIPCHECK(h, mark(h, K_GU, false));
            HIPCHECK(h, mark(h, K_DOWN, true));
            HIPCHECK(h, linear(h, h->m, 1, c.intermediate, L.down, L.down_s, L.down_b, hid, EPI_STORE, nullptr,
                               h->pend));
            HIPCHECK(h, mark(h, K_DOWN, false));
        }
    }
    HIPCHECK(h, launch_add_rmsnorm(dt, hcur, h->pend, h->final_norm, nullptr, out, 1, hid, c.rms_eps, s));
    return QWEN3_OK;
}

int run_layers(qwen3_handle *h, const void *x, int T, void *out) {
    if (T == 1) return run_decode(h, x, out);
    const qwen3_config &c = h->cfg;
    const int dt = c.dtype, hid = c.hidden, H = c.n_heads, KV = c.n_kv_heads, D = c.head_dim;
    const int nqkv = (H + 2 * KV) * D, p0 = h->length;
    const size_t es = esize(c), layer_kv = (size_t)KV * c.capacity * D * es;
    hipStream_t s = h->stream;
    bool pend_live = false;  // the last MLP left its output in pend (MoE); dense layers add it in place
    for (int l = 0; l < c.n_layers; ++l) {
        const qwen3_layer_weights &L = h->layers[l];
        // deferred residual + input norm; layer 0 normalises x directly
        if (l == 0) HIPCHECK(h, launch_add_rmsnorm(dt, x, nullptr, L.in_norm, nullptr, h->y, T, hid, c.rms_eps, s));
        else HIPCHECK(h, launch_add_rmsnorm(dt, h->h, pend_live ? h->pend : nullptr, L.in_norm,
                                            pend_live ? h->h : nullptr, h->y, T, hid, c.rms_eps, s));
        HIPCHECK(h, mark(h, K_QKV, true));
        // the fused epilogue reads and writes 16 bytes at a time: the table, q and the caches
        // are 16-byte aligned (checked by qwen3_init; workspace pieces are 256-byte aligned)
        if (dt == QWEN3_BF16 && !is_q8(h) && gemm_qkv_fused_ok(T, hid, H, KV, D)) {
            // q/k norm, RoPE and the cache write in the projection's epilogue
            QkvEpi qe;
            qe.q_norm = L.q_norm;
            qe.k_norm = L.k_norm;
            qe.bias = L.qkv_bias;
            qe.cos_t = h->cos_t;
            qe.sin_t = h->sin_t;
            qe.eps = c.rms_eps;
            qe.H = H;
            qe.KV = KV;
            qe.p0 = p0;
            qe.cap = c.capacity;
            qe.q_out = h->q;
            qe.kc = h->kc + l * layer_kv;
            qe.vc = h->vc + l * layer_kv;
            HIPCHECK(h, launch_gemm_qkv_fused(h->y, T, hid, L.qkv, qe, s));
            HIPCHECK(h, mark(h, K_QKV, false));
        } else {
            HIPCHECK(h, linear(h, h->y, T, hid, L.qkv, L.qkv_s, L.qkv_b, nqkv, EPI_STORE, nullptr, h->qkv));
            HIPCHECK(h, mark(h, K_QKV, false));
            HIPCHECK(h, launch_qknorm_rope_kv(dt, h->qkv, T, H, KV, D, L.q_norm, L.k_norm, L.qkv_bias, c.rms_eps,
                                              h->cos_t, h->sin_t, p0, c.capacity, h->q, h->kc + l * layer_kv,
                                              h->vc + l * layer_kv, s));
        }
        HIPCHECK(h, mark(h, K_ATTN, true));
        HIPCHECK(h, launch_attention(dt, h->q, h->kc + l * layer_kv, h->vc + l * layer_kv, T, H, KV, D, c.capacity, p0,
                                     c.sliding_window, h->a, h->attn_ws, 0, s));
        HIPCHECK(h, mark(h, K_ATTN, false));
        HIPCHECK(h, mark(h, K_O, true));
        HIPCHECK(h, linear(h, h->a, T, H * D, L.o, L.o_s, L.o_b, hid, EPI_RESID, l == 0 ? x : h->h, h->h));
        HIPCHECK(h, mark(h, K_O, false));
        HIPCHECK(h, launch_add_rmsnorm(dt, h->h, nullptr, L.post_norm, nullptr, h->y, T, hid, c.rms_eps, s));
        pend_live = moe_layer(c, L);
        if (pend_live) {
            HIPCHECK(h, moe(h, L, h->y, T, h->moe_idx, h->moe_w, h->pend));
        } else {
            HIPCHECK(h, mark(h, K_GU, true));
            HIPCHECK(h, linear(h, h->y, T, hid, L.gate_up, L.gate_up_s, L.gate_up_b, c.intermediate, EPI_SWIGLU,
                               nullptr, h->m));
            HIPCHECK(h, mark(h, K_GU, false));
            // the deferred add h = rho(h + rho(m Wdown^T)) happens in the down projection's epilogue
            HIPCHECK(h, mark(h, K_DOWN, true));
            HIPCHECK(h, linear(h, h->m, T, c.intermediate, L.down, L.down_s, L.down_b, hid, EPI_RESID, h->h, h->h));
            HIPCHECK(h, mark(h, K_DOWN, false));
        }
    }
    HIPCHECK(h, launch_add_rmsnorm(dt, h->h, pend_live ? h->pend : nullptr, h->final_norm, nullptr, out, T, hid,
                                   c.rms_eps, s));
    return QWEN3_OK;
}

// B seats, one token each (B <= DECODE_MAXB): the leader's workspace and stream carry the
// activations [B][...]; the projections run once over the B rows; attention runs per seat on
// its own cache at its own position in one batched launch.
int run_batch(qwen3_handle *const *seats, int B, const void *x, void *out) {
    qwen3_handle *h = seats[0];
    const qwen3_config &c = h->cfg;
    const int dt = c.dtype, hid = c.hidden, H = c.n_heads, KV = c.n_kv_heads, D = c.head_dim;
    const int nqkv = (H + 2 * KV) * D;
    const size_t es = esize(c), layer_kv = (size_t)KV * c.capacity * D * es;
    hipStream_t s = h->stream;
    int pos[DECODE_MAXB];
    void *kc[DECODE_MAXB], *vc[DECODE_MAXB];
    for (int b = 0; b < B; ++b) pos[b] = seats[b]->length;
    bool pend_live = false;  // as in run_layers: only an MoE layer leaves its output in pend
    for (int l = 0; l < c.n_layers; ++l) {
        const qwen3_layer_weights &L = h->layers[l];
        if (l == 0) HIPCHECK(h, launch_add_rmsnorm(dt, x, nullptr, L.in_norm, nullptr, h->y, B, hid, c.rms_eps, s));
        else HIPCHECK(h, launch_add_rmsnorm(dt, h->h, pend_live ? h->pend : nullptr, L.in_norm,
                                            pend_live ? h->h : nullptr, h->y, B, hid, c.rms_eps, s));
        HIPCHECK(h, linear(h, h->y, B, hid, L.qkv, L.qkv_s, L.qkv_b, nqkv, EPI_STORE, nullptr, h->qkv));
        for (int b = 0; b < B; ++b) {
            kc[b] = seats[b]->kc + l * layer_kv;
            vc[b] = seats[b]->vc + l * layer_kv;
        }
        HIPCHECK(h, launch_attention_decode_batch(dt, h->qkv, B, H, KV, D, L.q_norm, L.k_norm, L.qkv_bias, c.rms_eps,
                                                  h->cos_t, h->sin_t, kc, vc, pos, c.capacity, c.sliding_window, h->a,
                                                  h->attn_ws, s));
        HIPCHECK(h, linear(h, h->a, B, H * D, L.o, L.o_s, L.o_b, hid, EPI_RESID, l == 0 ? x : h->h, h->h));
        HIPCHECK(h, launch_add_rmsnorm(dt, h->h, nullptr, L.post_norm, nullptr, h->y, B, hid, c.rms_eps, s));
        pend_live = moe_layer(c, L);
        if (pend_live) {
            HIPCHECK(h, moe(h, L, h->y, B, h->moe_idx, h->moe_w, h->pend));
        } else {
            HIPCHECK(h, linear(h, h->y, B, hid, L.gate_up, L.gate_up_s, L.gate_up_b, c.intermediate, EPI_SWIGLU,
                               nullptr, h->m));
            HIPCHECK(h, linear(h, h->m, B, c.intermediate, L.down, L.down_s, L.down_b, hid, EPI_RESID, h->h, h->h));
        }
    }
    HIPCHECK(h, launch_add_rmsnorm(dt, h->h, pend_live ? h->pend : nullptr, h->final_norm, nullptr, out, B, hid,
                                   c.rms_eps, s));
    return QWEN3_OK;
}

bool same_model(const qwen3_handle *a, const qwen3_handle *b) {
    const qwen3_config &x = a->cfg, &y = b->cfg;
    if (x.n_layers != y.n_layers || x.hidden != y.hidden || x.n_heads != y.n_heads || x.n_kv_heads != y.n_kv_heads ||
        x.head_dim != y.head_dim || x.intermediate != y.intermediate || x.capacity != y.capacity ||
        x.rms_eps != y.rms_eps || x.rope_theta != y.rope_theta || x.dtype != y.dtype || x.n_experts != y.n_experts ||
        x.top_k != y.top_k || x.moe_intermediate != y.moe_intermediate || x.norm_topk_prob != y.norm_topk_prob ||
        x.quant_bits != y.quant_bits || x.quant_group != y.quant_group || x.sliding_window != y.sliding_window)
        return false;
    if (a->final_norm != b->final_norm) return false;
    for (int l = 0; l < x.n_layers; ++l)
        if (memcmp(&a->layers[l], &b->layers[l], sizeof(qwen3_layer_weights)) != 0) return false;
    return true;
}

}  // namespace

extern "C" {

int qwen3_forward_batch(qwen3_handle *const *seats, int B, const void *x, void *out) {
    if (!seats || !seats[0]) return QWEN3_ERR_ARG;
    qwen3_handle *h = seats[0];
    h->err.clear();
    if (!x || !out) return fail(h, QWEN3_ERR_ARG, "null input or output");
    if (!al16(x) || !al16(out)) return fail(h, QWEN3_ERR_ARG, "input and output must be 16-byte aligned");
    if (B < 1 || B > DECODE_MAXB) return fail(h, QWEN3_ERR_ARG, "B=%d outside 1..%d", B, DECODE_MAXB);
    if (B > h->cfg.max_tokens) return fail(h, QWEN3_ERR_ARG, "B=%d exceeds the first seat's max_tokens=%d", B, h->cfg.max_tokens);
    for (int b = 0; b < B; ++b) {
        if (!seats[b]) return fail(h, QWEN3_ERR_ARG, "seat %d is null", b);
        for (int q = 0; q < b; ++q)
            if (seats[q] == seats[b]) return fail(h, QWEN3_ERR_ARG, "seat %d appears twice", b);
        if (!same_model(h, seats[b])) return fail(h, QWEN3_ERR_ARG, "seat %d has another configuration or weights", b);
        if (seats[b]->length + 1 > seats[b]->cfg.capacity)
            return fail(h, QWEN3_ERR_CAPACITY, "seat %d: context %d exceeds capacity %d", b, seats[b]->length + 1,
                        seats[b]->cfg.capacity);
    }
    const int rc = run_batch(seats, B, x, out);
    if (rc == QWEN3_OK)
        for (int b = 0; b < B; ++b) seats[b]->length += 1;
    return rc;
}


const char *qwen3_status_string(int code) {
    switch (code) {
    case QWEN3_OK: return "ok";
    case QWEN3_ERR_ARG: return "invalid argument";
    case QWEN3_ERR_DTYPE: return "unsupported dtype";
    case QWEN3_ERR_CAPACITY: return "context exceeds capacity";
    case QWEN3_ERR_NULL_WEIGHT: return "missing weight";
    case QWEN3_ERR_UNSUPPORTED: return "unsupported shape";
    case QWEN3_ERR_HIP: return "HIP error";
    case QWEN3_ERR_WORKSPACE: return "workspace too small";
    default: return "unknown error";
    }
}

size_t qwen3_workspace_bytes(const qwen3_config *cfg) {
    if (check_config(cfg, nullptr) != QWEN3_OK) return 0;
    return layout(*cfg).total;
}

int qwen3_init(const qwen3_config *cfg, const qwen3_weights *w, void *k_cache, void *v_cache, void *workspace,
               size_t ws_bytes, void *stream, qwen3_handle **out) {
    if (!out) return QWEN3_ERR_ARG;
    std::string why;
    int rc = check_config(cfg, &why);
    if (rc != QWEN3_OK) return rc;
    if (!w || !w->layers || !k_cache || !v_cache) return QWEN3_ERR_ARG;
    const Layout L = layout(*cfg);
    if (!workspace || ws_bytes < L.total || ((uintptr_t)workspace & 255)) return QWEN3_ERR_WORKSPACE;
    if (!w->final_norm) return QWEN3_ERR_NULL_WEIGHT;
    if ((w->rope_cos == nullptr) != (w->rope_sin == nullptr)) return QWEN3_ERR_ARG;
    if (misaligned(cfg, w, k_cache, v_cache)) return QWEN3_ERR_ARG;
    const bool q8 = cfg->quant_bits == 8, moe = cfg->n_experts > 0;
    for (int l = 0; l < cfg->n_layers; ++l) {
        const qwen3_layer_weights &Lw = w->layers[l];
        if (!Lw.in_norm || !Lw.post_norm || !Lw.qkv || !Lw.o) return QWEN3_ERR_NULL_WEIGHT;
        if ((Lw.q_norm == nullptr) != (Lw.k_norm == nullptr)) return QWEN3_ERR_NULL_WEIGHT;  // both or neither
        if (q8 && (!Lw.qkv_s || !Lw.qkv_b || !Lw.o_s || !Lw.o_b)) return QWEN3_ERR_NULL_WEIGHT;
        if (moe && Lw.router) {
            if (!Lw.exp_gate_up || !Lw.exp_down) return QWEN3_ERR_NULL_WEIGHT;
            if (q8 && (!Lw.router_s || !Lw.router_b || !Lw.exp_gate_up_s || !Lw.exp_gate_up_b || !Lw.exp_down_s ||
                       !Lw.exp_down_b))
                return QWEN3_ERR_NULL_WEIGHT;
        } else {  // dense MLP (every layer of a dense configuration; router-less layers of an MoE one)
            if (!Lw.gate_up || !Lw.down) return QWEN3_ERR_NULL_WEIGHT;
            if (cfg->intermediate < 64) return QWEN3_ERR_UNSUPPORTED;
            if (q8 && (!Lw.gate_up_s || !Lw.gate_up_b || !Lw.down_s || !Lw.down_b)) return QWEN3_ERR_NULL_WEIGHT;
        }
    }
    qwen3_handle *h = new qwen3_handle();
    h->cfg = *cfg;
    h->layers.assign(w->layers, w->layers + cfg->n_layers);
    h->embed = w->embed;
    h->final_norm = w->final_norm;
    h->kc = (char *)k_cache;
    h->vc = (char *)v_cache;
    h->ws = (char *)workspace;
    h->ws_bytes = ws_bytes;
    h->stream = (hipStream_t)stream;
    char *b = h->ws;
    h->h = b + L.h;
    h->h2 = b + L.h2;
    h->y = b + L.y;
    h->qkv = b + L.qkv;
    h->q = b + L.q;
    h->a = b + L.a;
    h->m = b + L.m;
    h->pend = b + L.pend;
    h->tmp = b + L.tmp;
    h->attn_ws = (float *)(b + L.attn);
    h->dev_err = (int *)(b + L.err);
    h->head_keys = (unsigned long long *)(b + L.head_keys);
    if (moe) {
        h->moe_idx = (int32_t *)(b + L.moe_idx);
        h->moe_w = b + L.moe_w;
        h->moe_ws = b + L.moe_ws;
    }
    hipError_t e = hipMemsetAsync(h->dev_err, 0, 256, h->stream);
    if (e == hipSuccess) {
        if (w->rope_cos) {
            h->cos_t = w->rope_cos;
            h->sin_t = w->rope_sin;
        } else {
            h->cos_t = b + L.cos_t;
            h->sin_t = b + L.sin_t;
            e = launch_rope_table(cfg->dtype, cfg->capacity, cfg->head_dim, cfg->rope_theta, (void *)h->cos_t,
                                  (void *)h->sin_t, h->stream);
        }
    }
    if (e == hipSuccess && decode_mk_supported(cfg->n_layers, cfg->dtype, cfg->n_experts, cfg->quant_bits, cfg->hidden,
                                               cfg->n_heads, cfg->n_kv_heads, cfg->head_dim, cfg->intermediate,
                                               cfg->capacity) &&
        decode_mk_max_blocks(cfg->hidden, cfg->intermediate, cfg->n_heads, cfg->n_kv_heads, q8) >= decode_mk_blocks()) {
        std::vector<const void *> ptrs, qptrs;
        for (int l = 0; l < cfg->n_layers; ++l) {
            const qwen3_layer_weights &Lw = w->layers[l];
            const void *row[9] = {Lw.in_norm,  Lw.post_norm, Lw.q_norm, Lw.k_norm,  Lw.qkv,
                                  Lw.o,        Lw.gate_up,   Lw.down,   Lw.qkv_bias};
            ptrs.insert(ptrs.end(), row, row + 9);
            const void *qrow[8] = {Lw.qkv_s, Lw.qkv_b, Lw.o_s, Lw.o_b, Lw.gate_up_s, Lw.gate_up_b, Lw.down_s, Lw.down_b};
            qptrs.insert(qptrs.end(), qrow, qrow + 8);
        }
        h->mk_ws = b + L.mk;
        e = decode_mk_init(h->mk_ws, cfg->n_layers, cfg->n_heads, cfg->n_kv_heads, cfg->hidden, cfg->intermediate,
                           ptrs.data(), q8 ? qptrs.data() : nullptr, h->stream);
        h->mk_ready = e == hipSuccess;
    } else if (e == hipSuccess && moe_mk_config(*cfg) && decode_moe_max_blocks(q8) >= decode_mk_blocks()) {
        bool all_moe = true;  // the persistent MoE step has no dense-MLP layers
        std::vector<const void *> ptrs, qptrs;
        for (int l = 0; l < cfg->n_layers; ++l) {
            const qwen3_layer_weights &Lw = w->layers[l];
            all_moe = all_moe && Lw.router;
            const void *row[10] = {Lw.in_norm, Lw.post_norm, Lw.q_norm,  Lw.k_norm,   Lw.qkv,
                                   Lw.o,       Lw.router,    Lw.exp_gate_up, Lw.exp_down, Lw.qkv_bias};
            ptrs.insert(ptrs.end(), row, row + 10);
            const void *qrow[10] = {Lw.qkv_s,      Lw.qkv_b,         Lw.o_s,           Lw.o_b,
                                    Lw.router_s,   Lw.router_b,      Lw.exp_gate_up_s, Lw.exp_gate_up_b,
                                    Lw.exp_down_s, Lw.exp_down_b};
            qptrs.insert(qptrs.end(), qrow, qrow + 10);
        }
        if (all_moe) {
            h->mk_ws = b + L.mk;
            e = decode_moe_init(h->mk_ws, cfg->n_layers, cfg->n_heads, cfg->n_kv_heads, ptrs.data(),
                                q8 ? qptrs.data() : nullptr, h->stream);
            h->mk_ready = h->mk_moe = e == hipSuccess;
        }
    }
    if (e != hipSuccess) {
        delete h;
        return QWEN3_ERR_HIP;
    }
    *out = h;
    return QWEN3_OK;
}

int qwen3_reset(qwen3_handle *h) {
    if (!h) return QWEN3_ERR_ARG;
    h->err.clear();
    const qwen3_config &c = h->cfg;
    const size_t bytes = (size_t)c.n_layers * c.n_kv_heads * c.capacity * c.head_dim * esize(c);
    HIPCHECK(h, hipMemsetAsync(h->kc, 0, bytes, h->stream));
    HIPCHECK(h, hipMemsetAsync(h->vc, 0, bytes, h->stream));
    h->length = 0;
    return QWEN3_OK;
}

int qwen3_forward_hidden(qwen3_handle *h, const void *x, int T, void *out) {
    if (!h) return QWEN3_ERR_ARG;
    h->err.clear();
    if (!x || !out) return fail(h, QWEN3_ERR_ARG, "null input or output");
    if (!al16(x) || !al16(out)) return fail(h, QWEN3_ERR_ARG, "input and output must be 16-byte aligned");
    if (T < 1 || T > h->cfg.max_tokens) return fail(h, QWEN3_ERR_ARG, "T=%d outside 1..max_tokens=%d", T, h->cfg.max_tokens);
    if (h->length + T > h->cfg.capacity)
        return fail(h, QWEN3_ERR_CAPACITY, "context %d exceeds capacity %d", h->length + T, h->cfg.capacity);
    const int rc = run_layers(h, x, T, out);
    if (rc == QWEN3_OK) h->length += T;
    return rc;
}

int qwen3_head(qwen3_handle *h, const void *hs, int T, const void *head, int V, float *logits, int32_t *argmax) {
    if (!h) return QWEN3_ERR_ARG;
    h->err.clear();
    if (!hs) return fail(h, QWEN3_ERR_ARG, "null hidden states");
    if (!logits && !argmax) return fail(h, QWEN3_ERR_ARG, "neither logits nor argmax requested");
    if (!al16(hs) || !al16(head) || !al_elem(logits, 4) || !al_elem(argmax, 4))
        return fail(h, QWEN3_ERR_ARG, "hidden states and head must be 16-byte aligned, logits and argmax 4-byte");
    if (T < 1 || T > h->cfg.max_tokens) return fail(h, QWEN3_ERR_ARG, "T=%d outside 1..max_tokens=%d", T, h->cfg.max_tokens);
    if (!head) {
        if (!h->embed || h->cfg.vocab < 1) return fail(h, QWEN3_ERR_NULL_WEIGHT, "no head and no embedding table");
        if (V != h->cfg.vocab) return fail(h, QWEN3_ERR_ARG, "V=%d differs from the tied embedding's vocab %d", V, h->cfg.vocab);
        head = h->embed;
    }
    if (V < 1) return fail(h, QWEN3_ERR_ARG, "V=%d must be positive", V);
    HIPCHECK(h, launch_head(h->cfg.dtype, hs, T, h->cfg.hidden, head, V, logits, argmax, h->head_keys, h->stream));
    return QWEN3_OK;
}

int qwen3_head_static(int dtype, const void *hs, int T, int hidden, const void *head, int V, float *logits,
                      int32_t *argmax, void *stream) {
    if (dtype != QWEN3_BF16 && dtype != QWEN3_FP32) return QWEN3_ERR_DTYPE;
    if (!hs || !head || (!logits && !argmax)) return QWEN3_ERR_ARG;
    if (T < 1 || T > QWEN3_HEAD_STATIC_MAX_T || V < 1 || hidden < 64 || hidden % 64) return QWEN3_ERR_ARG;
    if (!al16(hs) || !al16(head) || !al_elem(logits, 4) || !al_elem(argmax, 4)) return QWEN3_ERR_ARG;
    static_assert(QWEN3_HEAD_STATIC_MAX_T == HEAD_STATIC_MAX_T, "header and library agree on the limit");
    return launch_head_static(dtype, hs, T, hidden, head, V, logits, argmax, (hipStream_t)stream) == hipSuccess
               ? QWEN3_OK
               : QWEN3_ERR_HIP;
}

int qwen3_forward(qwen3_handle *h, const int32_t *tokens, int T, void *out) {
    if (!h) return QWEN3_ERR_ARG;
    h->err.clear();
    if (!tokens || !out) return fail(h, QWEN3_ERR_ARG, "null tokens or output");
    if (!al_elem(tokens, 4) || !al16(out)) return fail(h, QWEN3_ERR_ARG, "token ids must be 4-byte, the output 16-byte aligned");
    if (!h->embed || h->cfg.vocab < 1) return fail(h, QWEN3_ERR_NULL_WEIGHT, "no embedding table");
    if (T < 1 || T > h->cfg.max_tokens) return fail(h, QWEN3_ERR_ARG, "T=%d outside 1..max_tokens=%d", T, h->cfg.max_tokens);
    if (h->length + T > h->cfg.capacity)
        return fail(h, QWEN3_ERR_CAPACITY, "context %d exceeds capacity %d", h->length + T, h->cfg.capacity);
    HIPCHECK(h, launch_embed(h->cfg.dtype, tokens, T, h->embed, h->cfg.vocab, h->cfg.hidden, h->tmp, h->dev_err,
                             h->stream));
    const int rc = run_layers(h, h->tmp, T, out);
    if (rc == QWEN3_OK) h->length += T;
    return rc;
}

int qwen3_moe_block(qwen3_handle *h, int layer, const void *x, int T, void *out, int32_t *topk_idx, void *topk_w) {
    if (!h) return QWEN3_ERR_ARG;
    h->err.clear();
    const qwen3_config &c = h->cfg;
    if (c.n_experts <= 0) return fail(h, QWEN3_ERR_ARG, "not an MoE configuration");
    if (layer < 0 || layer >= c.n_layers) return fail(h, QWEN3_ERR_ARG, "layer %d out of range", layer);
    if (!x || !out) return fail(h, QWEN3_ERR_ARG, "null input or output");
    if (!al16(x) || !al16(out) || !al_elem(topk_idx, 4) || !al_elem(topk_w, esize(c)))
        return fail(h, QWEN3_ERR_ARG, "input and output must be 16-byte aligned, the routing outputs element-aligned");
    if (T < 1 || T > c.max_tokens) return fail(h, QWEN3_ERR_ARG, "T=%d outside 1..max_tokens=%d", T, c.max_tokens);
    const qwen3_layer_weights &L = h->layers[layer];
    if (!moe_layer(c, L)) return fail(h, QWEN3_ERR_ARG, "layer %d is a dense layer", layer);
    int32_t *idx = topk_idx ? topk_idx : h->moe_idx;
    void *w = topk_w ? topk_w : h->moe_w;
    HIPCHECK(h, moe(h, L, x, T, idx, w, out));
    return QWEN3_OK;
}

int qwen3_set_length(qwen3_handle *h, int length) {
    if (!h) return QWEN3_ERR_ARG;
    h->err.clear();
    if (length < 0 || length > h->cfg.capacity)
        return fail(h, QWEN3_ERR_ARG, "length %d outside 0..capacity=%d", length, h->cfg.capacity);
    h->length = length;
    return QWEN3_OK;
}

int qwen3_get_length(const qwen3_handle *h) { return h ? h->length : QWEN3_ERR_ARG; }

int qwen3_set_stream(qwen3_handle *h, void *stream) {
    if (!h) return QWEN3_ERR_ARG;
    h->stream = (hipStream_t)stream;
    return QWEN3_OK;
}

int qwen3_check_device_errors(qwen3_handle *h) {
    if (!h) return QWEN3_ERR_ARG;
    h->err.clear();
    int flag = 0;
    HIPCHECK(h, hipMemcpyAsync(&flag, h->dev_err, sizeof(int), hipMemcpyDeviceToHost, h->stream));
    HIPCHECK(h, hipStreamSynchronize(h->stream));
    if (flag) {
        HIPCHECK(h, hipMemsetAsync(h->dev_err, 0, sizeof(int), h->stream));
        if (flag & 2) return fail(h, QWEN3_ERR_HIP, "the persistent decode step timed out waiting for an exchange");
        return fail(h, QWEN3_ERR_ARG, "a token id was outside [0, vocab)");
    }
    return QWEN3_OK;
}

int qwen3_set_decode_path(qwen3_handle *h, int path) {
    if (!h) return QWEN3_ERR_ARG;
    h->err.clear();
    if (path < 0 || path > 2) return fail(h, QWEN3_ERR_ARG, "decode path must be 0, 1 or 2");
    if (path == 2 && !h->mk_ready)
        return fail(h, QWEN3_ERR_UNSUPPORTED, "no persistent decode kernel for this configuration or device");
    h->decode_path = path;
    return QWEN3_OK;
}

int qwen3_get_decode_path(const qwen3_handle *h) {
    if (!h) return QWEN3_ERR_ARG;
    return (h->mk_ready && h->decode_path != 1) ? 2 : 1;
}

int qwen3_kernel_timer(qwen3_handle *h, int kind, int enable) {
    if (!h || kind < 0 || kind >= qwen3_handle::NKIND) return QWEN3_ERR_ARG;
    h->timer_on[kind] = enable != 0;
    h->timer_used[kind] = 0;
    return QWEN3_OK;
}

int qwen3_kernel_timer_read(qwen3_handle *h, int kind, double *total_ms, int *count) {
    if (!h || kind < 0 || kind >= qwen3_handle::NKIND || !total_ms || !count) return QWEN3_ERR_ARG;
    h->err.clear();
    double tot = 0.0;
    for (int i = 0; i < h->timer_used[kind]; ++i) {
        const auto &p = h->timer_ev[kind][i];
        HIPCHECK(h, hipEventSynchronize(p.second));
        float ms = 0.f;
        HIPCHECK(h, hipEventElapsedTime(&ms, p.first, p.second));
        tot += ms;
    }
    *total_ms = tot;
    *count = h->timer_used[kind];
    return QWEN3_OK;
}

const char *qwen3_last_error(const qwen3_handle *h) { return h ? h->err.c_str() : "null handle"; }

void qwen3_destroy(qwen3_handle *h) { delete h; }

int qwen3_rope_table(int capacity, int head_dim, double theta, int dtype, void *cos_out, void *sin_out,
                     void *stream) {
    if (dtype != QWEN3_BF16 && dtype != QWEN3_FP32) return QWEN3_ERR_DTYPE;
    if (capacity < 1 || (head_dim != 64 && head_dim != 128) || !(theta > 1.0) || !cos_out || !sin_out)
        return QWEN3_ERR_ARG;
    return launch_rope_table(dtype, capacity, head_dim, theta, cos_out, sin_out, (hipStream_t)stream) == hipSuccess
               ? QWEN3_OK
               : QWEN3_ERR_HIP;
}

}  // extern "C"
