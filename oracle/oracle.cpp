/*
 * oracle.cpp -- CPU oracle (test infrastructure only; see oracle.h).
 *
 * A plain restatement of the Qwen3 decoder-layer forward and the Qwen3-MoE
 * block.  Loops follow the pages' order of operations; OpenMP only splits
 * independent outer loops (output rows, heads, tokens), which does not change
 * any result.  Build: -O2 -ffp-contract=off -fno-fast-math -fopenmp.
 */
#include "oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <numeric>
#include <vector>

static int g_threads = 0;

extern "C" void orc_set_threads(int n) {
    g_threads = n;
    if (n > 0) omp_set_num_threads(n);
}
extern "C" int orc_get_threads(void) { return g_threads > 0 ? g_threads : omp_get_max_threads(); }

/* ---------------------------------------------------------------- rounding */

/* bf16 round-to-nearest-even, from the IEEE-754 definition: keep the upper 16
 * bits of the binary32 pattern, rounding the dropped 16 bits to nearest with
 * ties to an even kept pattern.  NaN is kept NaN (quiet bit set). */
static float bf16_rne(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0) {
        u = (u | 0x00400000u) & 0xffff0000u;
    } else {
        uint32_t dropped = u & 0xffffu;
        uint32_t kept = u >> 16;
        if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;
        u = kept << 16;
    }
    float r;
    memcpy(&r, &u, 4);
    return r;
}

extern "C" float orc_round(float x, int mode) { return mode == ORC_BF16 ? bf16_rne(x) : x; }

extern "C" void orc_round_array(float *x, size_t n, int mode) {
    if (mode != ORC_BF16) return;
    for (size_t i = 0; i < n; ++i) x[i] = bf16_rne(x[i]);
}

static inline float rho(float x, int mode) { return mode == ORC_BF16 ? bf16_rne(x) : x; }

/* Exact-product dot in double, rounded once to fp32.  Every product of two
 * fp32 values is exact in double; the double sum is the "exact sum rounded
 * once" reading of an fp32-accumulated matmul. */
static float dot(const float *a, const float *b, int n) {
    double acc = 0.0;
#pragma omp simd reduction(+ : acc)
    for (int i = 0; i < n; ++i) acc += (double)a[i] * (double)b[i];
    return (float)acc;
}

/* ---------------------------------------------------------------- RMSNorm */

extern "C" void orc_rmsnorm(const float *v, const float *w, int n, float eps, int mode, float *out) {
    double ss = 0.0;
    for (int i = 0; i < n; ++i) ss += (double)v[i] * (double)v[i];
    float ms = (float)(ss / (double)n);
    float r = 1.0f / sqrtf(ms + eps);
    for (int i = 0; i < n; ++i) {
        float z = rho(v[i] * r, mode);  /* first rounding: the normalised value */
        out[i] = rho(w[i] * z, mode);   /* second rounding: times the weight */
    }
}

/* ---------------------------------------------------------------- linear */

extern "C" void orc_linear(const float *x, int T, int K, const float *W, int N, int mode, float *out) {
#pragma omp parallel for schedule(static) collapse(2)
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < N; ++j)
            out[(size_t)t * N + j] = rho(dot(x + (size_t)t * K, W + (size_t)j * K, K), mode);
}

/* ---------------------------------------------------------------- output head */

extern "C" void orc_head(const float *hs, int T, int K, const float *W, int V, int mode, float *logits, int *argmax) {
    std::vector<float> row(V);
    for (int t = 0; t < T; ++t) {
        orc_linear(hs + (size_t)t * K, 1, K, W, V, mode, row.data());
        int best = 0;
        for (int v = 1; v < V; ++v)  /* strictly larger only: ties keep the lower index */
            if (row[v] > row[best] || (row[best] != row[best] && row[v] == row[v])) best = v;
        argmax[t] = best;
        if (logits)
            for (int v = 0; v < V; ++v) logits[(size_t)t * V + v] = row[v];
    }
}

/* ---------------------------------------------------------------- RoPE */

extern "C" void orc_rope_table(int capacity, int D, double theta, int mode, float *cos_out,
                               float *sin_out) {
    const int half = D / 2;
    for (int j = 0; j < half; ++j) {
        /* inverse frequency theta^(-2j/D), rounded to fp32; the bf16 model
         * holds it as a bf16 buffer, so bf16 mode rounds it once more. */
        float inv = (float)(1.0 / pow(theta, (2.0 * j) / (double)D));
        inv = rho(inv, mode);
        for (int p = 0; p < capacity; ++p) {
            float ang = (float)p * inv;                 /* one fp32 product */
            float c = rho((float)cos((double)ang), mode);
            float s = rho((float)sin((double)ang), mode);
            cos_out[(size_t)p * D + j] = c;
            cos_out[(size_t)p * D + j + half] = c;
            sin_out[(size_t)p * D + j] = s;
            sin_out[(size_t)p * D + j + half] = s;
        }
    }
}

extern "C" void orc_rope(const float *x, int D, const float *c, const float *s, int mode, float *out) {
    const int half = D / 2;
    std::vector<float> o(D);
    for (int i = 0; i < half; ++i) {
        float x1 = x[i], x2 = x[i + half];
        float a = x1 * c[i];
        float b = x2 * s[i];
        o[i] = rho(a - b, mode);
        float a2 = x2 * c[i + half];
        float b2 = x1 * s[i + half];
        o[i + half] = rho(a2 + b2, mode);
    }
    memcpy(out, o.data(), sizeof(float) * D);
}

/* ---------------------------------------------------------------- attention */

extern "C" void orc_attention(const float *q, const float *K, const float *V, int T, int H, int KV,
                              int D, int cap, int p0, int window, int mode, float *out, float *probs) {
    const int group = H / KV;
    const float scale = (float)(1.0 / sqrt((double)D));
    const int nk = p0 + T;
#pragma omp parallel for schedule(dynamic) collapse(2)
    for (int t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h) {
            const int p = p0 + t;          /* absolute position of the query */
            const int lo = window > 0 ? std::max(0, p - window + 1) : 0; /* first visible key */
            const int g = h / group;       /* kv head read by q head h */
            const float *qv = q + ((size_t)t * H + h) * D;
            const float *Kg = K + (size_t)g * cap * D;
            const float *Vg = V + (size_t)g * cap * D;
            std::vector<float> s(p + 1), e(p + 1, 0.0f);
            float m = -INFINITY;
            for (int j = lo; j <= p; ++j) {
                s[j] = dot(qv, Kg + (size_t)j * D, D) * scale;
                m = std::max(m, s[j]);
            }
            double l = 0.0;
            for (int j = lo; j <= p; ++j) {
                e[j] = expf(s[j] - m);
                l += (double)e[j];
            }
            const float lf = (float)l;
            for (int d = 0; d < D; ++d) {
                double acc = 0.0;
                for (int j = lo; j <= p; ++j) acc += (double)e[j] * (double)Vg[(size_t)j * D + d];
                out[(size_t)t * H * D + (size_t)h * D + d] = rho((float)acc / lf, mode);
            }
            if (probs) {
                float *pr = probs + ((size_t)t * H + h) * nk;
                for (int j = 0; j < nk; ++j) pr[j] = (j >= lo && j <= p) ? e[j] / lf : 0.0f;
            }
        }
    }
}

/* ---------------------------------------------------------------- SwiGLU */

static inline float silu_rounded(float g, int mode) { return rho(g / (1.0f + expf(-g)), mode); }

extern "C" void orc_swiglu(const float *gu, int T, int I, int mode, float *out) {
    for (int t = 0; t < T; ++t)
        for (int i = 0; i < I; ++i) {
            float g = gu[(size_t)t * 2 * I + i];
            float u = gu[(size_t)t * 2 * I + I + i];
            out[(size_t)t * I + i] = rho(silu_rounded(g, mode) * u, mode);
        }
}

/* ---------------------------------------------------------------- MoE */

extern "C" void orc_router(const float *y2, int T, int hid, const float *Wr, int E, int k, int norm,
                           int mode, int32_t *idx, float *w, float *probs) {
    std::vector<float> logits((size_t)T * E);
    orc_linear(y2, T, hid, Wr, E, mode, logits.data());
    for (int t = 0; t < T; ++t) {
        const float *l = logits.data() + (size_t)t * E;
        /* softmax over all experts in fp32, rounded to the model dtype */
        float m = -INFINITY;
        for (int e = 0; e < E; ++e) m = std::max(m, l[e]);
        std::vector<float> ex(E), P(E);
        double z = 0.0;
        for (int e = 0; e < E; ++e) {
            ex[e] = expf(l[e] - m);
            z += (double)ex[e];
        }
        const float zf = (float)z;
        for (int e = 0; e < E; ++e) P[e] = rho(ex[e] / zf, mode);
        if (probs) memcpy(probs + (size_t)t * E, P.data(), sizeof(float) * E);
        /* top-k: descending P, ties to the lower expert index */
        std::vector<int> order(E);
        std::iota(order.begin(), order.end(), 0);
        std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return P[a] > P[b]; });
        double den = 0.0;
        for (int s = 0; s < k; ++s) den += (double)P[order[s]];
        const float denr = rho((float)den, mode);
        for (int s = 0; s < k; ++s) {
            idx[(size_t)t * k + s] = order[s];
            w[(size_t)t * k + s] = norm ? rho(P[order[s]] / denr, mode) : P[order[s]];
        }
    }
}

/* One expert's SwiGLU FFN on one row: y = rho(swiglu(rho(x Wgu^T)) Wd^T). */
static void expert_row(const float *x, int hid, int Ie, const float *Wgu, const float *Wd, int mode,
                       float *y) {
    std::vector<float> gu(2 * (size_t)Ie), m(Ie);
    for (int j = 0; j < 2 * Ie; ++j) gu[j] = rho(dot(x, Wgu + (size_t)j * hid, hid), mode);
    orc_swiglu(gu.data(), 1, Ie, mode, m.data());
    for (int j = 0; j < hid; ++j) y[j] = rho(dot(m.data(), Wd + (size_t)j * Ie, Ie), mode);
}

extern "C" void orc_moe_block(const float *y2, int T, int hid, const float *Wr, int E, int k, int Ie,
                              int norm, const float *Wgu_e, const float *Wd_e, int sorted, int mode,
                              float *out, int32_t *idx_out, float *w_out) {
    std::vector<int32_t> idx((size_t)T * k);
    std::vector<float> w((size_t)T * k);
    orc_router(y2, T, hid, Wr, E, k, norm, mode, idx.data(), w.data(), NULL);
    const size_t rows = (size_t)T * k;
    std::vector<float> y(rows * hid); /* expert output of row (t, slot), in token order */
    const size_t gu_stride = (size_t)2 * Ie * hid, d_stride = (size_t)hid * Ie;

    if (!sorted) {
        /* gather-matmul in token order */
#pragma omp parallel for schedule(dynamic)
        for (long r = 0; r < (long)rows; ++r) {
            const int e = idx[r];
            expert_row(y2 + (size_t)(r / k) * hid, hid, Ie, Wgu_e + e * gu_stride, Wd_e + e * d_stride,
                       mode, y.data() + (size_t)r * hid);
        }
    } else {
        /* stable sort of the flattened (token, slot) rows by expert, run in
         * that order, then scatter back through the inverse permutation */
        std::vector<int> order(rows), inverse(rows);
        std::iota(order.begin(), order.end(), 0);
        std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return idx[a] < idx[b]; });
        for (size_t i = 0; i < rows; ++i) inverse[order[i]] = (int)i;
        std::vector<float> ys(rows * hid);
#pragma omp parallel for schedule(dynamic)
        for (long i = 0; i < (long)rows; ++i) {
            const int r = order[i];
            const int e = idx[r];
            expert_row(y2 + (size_t)(r / k) * hid, hid, Ie, Wgu_e + e * gu_stride, Wd_e + e * d_stride,
                       mode, ys.data() + (size_t)i * hid);
        }
        for (size_t r = 0; r < rows; ++r)
            memcpy(y.data() + r * hid, ys.data() + (size_t)inverse[r] * hid, sizeof(float) * hid);
    }
    /* weighted sum over the slots */
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < hid; ++j) {
            double acc = 0.0;
            for (int s = 0; s < k; ++s) {
                const size_t r = (size_t)t * k + s;
                acc += (double)rho(y[r * hid + j] * w[r], mode);
            }
            out[(size_t)t * hid + j] = rho((float)acc, mode);
        }
    if (idx_out) memcpy(idx_out, idx.data(), sizeof(int32_t) * rows);
    if (w_out) memcpy(w_out, w.data(), sizeof(float) * rows);
}

/* ---------------------------------------------------------------- q8 */

extern "C" void orc_q8_dequant(const uint8_t *q, const float *s, const float *b, int N, int K,
                               int group, float *out) {
    const int ng = K / group;
    for (int j = 0; j < N; ++j)
        for (int kk = 0; kk < K; ++kk) {
            const float sc = s[(size_t)j * ng + kk / group], bi = b[(size_t)j * ng + kk / group];
            const float prod = sc * (float)q[(size_t)j * K + kk];
            out[(size_t)j * K + kk] = prod + bi;
        }
}

extern "C" void orc_q8_quantize(const float *w, int N, int K, int group, uint8_t *q, float *s, float *b) {
    const int ng = K / group;
    for (int j = 0; j < N; ++j)
        for (int g = 0; g < ng; ++g) {
            const float *wg = w + (size_t)j * K + (size_t)g * group;
            float lo = wg[0], hi = wg[0];
            for (int i = 1; i < group; ++i) {
                lo = std::min(lo, wg[i]);
                hi = std::max(hi, wg[i]);
            }
            const float sc = bf16_rne((hi - lo) / 255.0f);
            const float bi = bf16_rne(lo);
            s[(size_t)j * ng + g] = sc;
            b[(size_t)j * ng + g] = bi;
            for (int i = 0; i < group; ++i) {
                float c = sc > 0.0f ? nearbyintf((wg[i] - bi) / sc) : 0.0f;
                c = std::min(255.0f, std::max(0.0f, c));
                q[(size_t)j * K + (size_t)g * group + i] = (uint8_t)c;
            }
        }
}

/* ---------------------------------------------------------------- stack */

extern "C" int orc_forward(const orc_config *cfg, const orc_layer *layers, const float *final_norm,
                           const float *cos_tab, const float *sin_tab, float *kcache, float *vcache,
                           int *length, const float *x, int T, float *out) {
    if (!cfg || !layers || !length || !x || !out) return ORC_ERR_ARG;
    if (cfg->mode != ORC_BF16 && cfg->mode != ORC_FP32) return ORC_ERR_MODE;
    if (T < 1) return ORC_ERR_ARG;
    const int p0 = *length;
    if (p0 + T > cfg->capacity) return ORC_ERR_CAPACITY; /* before any write */

    const int hid = cfg->hidden, H = cfg->n_heads, KV = cfg->n_kv_heads, D = cfg->head_dim;
    const int I = cfg->intermediate, cap = cfg->capacity, mode = cfg->mode;
    const float eps = cfg->rms_eps;
    const int nqkv = (H + 2 * KV) * D;
    for (int l = 0; l < cfg->n_layers; ++l) { /* every layer has the weights of its kind */
        const orc_layer &L = layers[l];
        const bool moe = cfg->n_experts > 0 && L.router;
        if (moe ? (!L.exp_gate_up || !L.exp_down || cfg->top_k < 1 || cfg->top_k > cfg->n_experts)
                : (!L.gate_up || !L.down || I < 1))
            return ORC_ERR_ARG;
        if ((cfg->qk_norm && (!L.q_norm || !L.k_norm)) || (cfg->attention_bias && !L.qkv_bias))
            return ORC_ERR_ARG;
    }

    std::vector<float> h(x, x + (size_t)T * hid), pend((size_t)T * hid), y((size_t)T * hid);
    std::vector<float> qkv((size_t)T * nqkv), q((size_t)T * H * D), a((size_t)T * H * D);
    std::vector<float> o((size_t)T * hid), gu, m;
    bool have_pend = false;

    for (int l = 0; l < cfg->n_layers; ++l) {
        const orc_layer &L = layers[l];
        float *Kl = kcache + (size_t)l * KV * cap * D;
        float *Vl = vcache + (size_t)l * KV * cap * D;

        /* deferred residual of the previous layer's MLP: one rounding */
        if (have_pend)
            for (size_t i = 0; i < h.size(); ++i) h[i] = rho(h[i] + pend[i], mode);

        for (int t = 0; t < T; ++t)
            orc_rmsnorm(&h[(size_t)t * hid], L.in_norm, hid, eps, mode, &y[(size_t)t * hid]);
        orc_linear(y.data(), T, hid, L.qkv, nqkv, mode, qkv.data());
        if (cfg->attention_bias) /* [P2]: the bias is a separate add after the projection */
            for (int t = 0; t < T; ++t)
                for (int i = 0; i < nqkv; ++i)
                    qkv[(size_t)t * nqkv + i] = rho(qkv[(size_t)t * nqkv + i] + L.qkv_bias[i], mode);

        for (int t = 0; t < T; ++t) {
            const int p = p0 + t;
            const float *row = &qkv[(size_t)t * nqkv];
            const float *c = cos_tab + (size_t)p * D, *s = sin_tab + (size_t)p * D;
            for (int hh = 0; hh < H; ++hh) {
                float *qh = &q[((size_t)t * H + hh) * D];
                if (cfg->qk_norm) orc_rmsnorm(row + (size_t)hh * D, L.q_norm, D, eps, mode, qh);
                else memcpy(qh, row + (size_t)hh * D, sizeof(float) * D);
                orc_rope(qh, D, c, s, mode, qh);
            }
            for (int g = 0; g < KV; ++g) {
                std::vector<float> kg(D);
                if (cfg->qk_norm) orc_rmsnorm(row + (size_t)(H + g) * D, L.k_norm, D, eps, mode, kg.data());
                else memcpy(kg.data(), row + (size_t)(H + g) * D, sizeof(float) * D);
                orc_rope(kg.data(), D, c, s, mode, kg.data());
                memcpy(Kl + ((size_t)g * cap + p) * D, kg.data(), sizeof(float) * D);
                memcpy(Vl + ((size_t)g * cap + p) * D, row + (size_t)(H + KV + g) * D, sizeof(float) * D);
            }
        }
        orc_attention(q.data(), Kl, Vl, T, H, KV, D, cap, p0, cfg->window, mode, a.data(), NULL);

        orc_linear(a.data(), T, H * D, L.o, hid, mode, o.data());
        for (size_t i = 0; i < h.size(); ++i) h[i] = rho(h[i] + o[i], mode);

        for (int t = 0; t < T; ++t)
            orc_rmsnorm(&h[(size_t)t * hid], L.post_norm, hid, eps, mode, &y[(size_t)t * hid]);

        if (cfg->n_experts > 0 && L.router) {
            orc_moe_block(y.data(), T, hid, L.router, cfg->n_experts, cfg->top_k, cfg->moe_intermediate,
                          cfg->norm_topk_prob, L.exp_gate_up, L.exp_down, 0, mode, pend.data(), NULL, NULL);
        } else {
            gu.resize((size_t)T * 2 * I);
            m.resize((size_t)T * I);
            orc_linear(y.data(), T, hid, L.gate_up, 2 * I, mode, gu.data());
            orc_swiglu(gu.data(), T, I, mode, m.data());
            orc_linear(m.data(), T, I, L.down, hid, mode, pend.data());
        }
        have_pend = true;
    }
    for (size_t i = 0; i < h.size(); ++i) h[i] = rho(h[i] + pend[i], mode);
    *length = p0 + T;
    for (int t = 0; t < T; ++t) orc_rmsnorm(&h[(size_t)t * hid], final_norm, hid, eps, mode, out + (size_t)t * hid);
    return ORC_OK;
}
