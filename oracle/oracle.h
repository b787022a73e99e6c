/*
 * oracle.h -- CPU oracle for the Qwen3 decoder-layer forward over a static
 * per-seat KV cache, and for the Qwen3-MoE block.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, single-source C++
 * restatement of what the layer computes, written from the pages' text.  It is
 * used by the test-suite, by the package's smoke check and by the benchmark's
 * CPU-baseline leg, and by nothing else: the product path never links, loads
 * or calls it.  It shares no code, header, table or helper with the GPU
 * library.
 *
 * Sources (the pages):
 *  [P1] "maya2_mlx/backbone.py" (zone-1.cobraproject.com): the module
 *       docstring (rounding points), Backbone.__init__ (config, dtype gate,
 *       fused q|k|v and gate|up rows, RoPE table), reset(), _rope(),
 *       forward().  Authority for the arithmetic.
 *  [P2] "rlx_flow/blocks/qwen3_decoder.rs" (docs.rs, rlx-flow 0.2.11):
 *       Qwen3DecoderStage::emit and per_head_rms.  Op-order cross-check and the
 *       GQA mapping (repeat_kv with group = nh / nkv).
 *  [P3] "@mlx-bun/inference" qwen3-moe.ts / qwen3.ts (my.diffend.io page 97):
 *       Qwen3MoeSparseMoeBlock.forward, Qwen3UnsortedExperts,
 *       Qwen3SortedExperts, Qwen3Attention.forward.  Authority for the MoE
 *       block.
 *
 * Data model.  Every array is host memory holding float.  In bf16 mode
 * (ORC_BF16) every stored value is bf16-representable: inputs are exact
 * widenings of bf16 data and every rounding point rho() rounds to bf16
 * round-to-nearest-even.  In fp32 mode (ORC_FP32, [P1] "fp32 for the strict
 * gates") rho() is the identity.
 *
 * Arithmetic conventions (readings where the pages are silent):
 *  - every reduction (dot product, sum of squares, softmax denominator,
 *    probability-weighted value sum, MoE renormalisation and slot sum) is
 *    accumulated in double and rounded once to fp32; elementwise steps are
 *    fp32 operations as the pages state;
 *  - rho() is applied exactly where [P1]'s docstring and forward() round
 *    (each model-dtype array is one rounding);
 *  - no FMA contraction: built with -ffp-contract=off -fno-fast-math.
 *
 * Error convention: functions that can fail return 0 on success or a negative
 * ORC_ERR_* code, and change no output or state on failure ([P1] forward():
 * the capacity check raises before anything is written).
 */
#ifndef QWEN3_ORACLE_H
#define QWEN3_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_BF16 = 0, ORC_FP32 = 1 };
enum { ORC_OK = 0, ORC_ERR_ARG = -1, ORC_ERR_CAPACITY = -2, ORC_ERR_MODE = -3 };

/* rho: round one fp32 value to the model dtype (bf16 RNE in bf16 mode,
 * identity in fp32 mode).  NaN stays NaN (quiet), +-Inf stays +-Inf. */
float orc_round(float x, int mode);
void orc_round_array(float *x, size_t n, int mode);

/* RMSNorm with Qwen3's two roundings ([P1] docstring, mx.fast.rms_norm; [P2]
 * rms_norm with a zero beta):  ms = sum(v^2)/n, r = 1/sqrt(ms + eps),
 * z_i = rho(v_i * r), out_i = rho(w_i * z_i).  out may alias v. */
void orc_rmsnorm(const float *v, const float *w, int n, float eps, int mode, float *out);

/* out[t][j] = rho(sum_k x[t][k] * W[j][k]) for t < T, j < N; W row-major
 * [N][K] (the y @ W^T of [P1] Q.mm). */
void orc_linear(const float *x, int T, int K, const float *W, int N, int mode, float *out);

/* Output head and greedy token ([P1] Backbone.cb0_logits: the head projection in the model
 * dtype, then fp32; [P3] lmHead / the tied embedding used as a linear, then the greedy pick):
 * logits[t][v] = rho(sum_k hs[t][k] * W[v][k]) held in fp32, and argmax[t] = the lowest v
 * whose logit is the largest (a NaN logit is never the pick unless every logit is NaN, then
 * v = 0).  W row-major [V][K]; logits may be NULL. */
void orc_head(const float *hs, int T, int K, const float *W, int V, int mode, float *logits, int *argmax);

/* RoPE table, [P1] __init__ comment on the table and _rope():
 *   inv_j = fp32(theta^(-2j/D)) for j < D/2, rounded to bf16 in bf16 mode;
 *   angle = fp32(float(p) * inv_j);
 *   C[p][j] = C[p][j + D/2] = rho(fp32(cos(angle)))  (sin likewise).
 * cos/sin out: [capacity][D]. */
void orc_rope_table(int capacity, int D, double theta, int mode, float *cos_out, float *sin_out);

/* Rotate-half RoPE of one head vector at one position, fp32 maths, one
 * rounding ([P1] _rope):  o_i = rho(x_i c_i - x_{i+D/2} s_i),
 * o_{i+D/2} = rho(x_{i+D/2} c_{i+D/2} + x_i s_{i+D/2}).  out may alias x. */
void orc_rope(const float *x, int D, const float *cos_row, const float *sin_row, int mode, float *out);

/* Causal GQA attention ([P1] forward(): scaled_dot_product_attention with
 * mask "causal" when T > 1; docstring "attention over keys 0..pos (fp32
 * softmax, one rounding)"; [P2] repeat_kv group = H / KV; [P2]
 * Qwen3DecoderSpec mask: Causal or SlidingWindow(w)).
 *   q:   [T][H][D] (post-norm, post-RoPE)
 *   K,V: [KV][cap][D] cache of one layer (positions 0..p0+T-1 valid)
 *   query t sits at absolute position p = p0 + t and sees keys lo..p, where
 *   lo = 0 (window <= 0: causal) or max(0, p - window + 1) (a sliding window
 *   of the window most recent positions, the query's own included);
 *   q head h reads kv head h / (H/KV);
 *   s_j = fp32(q.K_j) * fp32(1/sqrt(D)); e_j = expf(s_j - max s);
 *   out[t][h*D + d] = rho(sum_j e_j V_j[d] / sum_j e_j).
 * probs (optional, may be NULL): [T][H][p0+T] receives e_j / sum e (0 outside lo..p). */
void orc_attention(const float *q, const float *K, const float *V, int T, int H, int KV, int D,
                   int cap, int p0, int window, int mode, float *out, float *probs);

/* SwiGLU on fused gate|up rows ([P1] forward(): silu in fp32 on the model
 * dtype gate, rounded once, then times up, rounded once):
 *   out[t][i] = rho(rho(g/(1+expf(-g))) * u), g = gu[t][i], u = gu[t][I+i]. */
void orc_swiglu(const float *gu, int T, int I, int mode, float *out);

/* MoE router ([P3] Qwen3MoeSparseMoeBlock.forward):
 *   l = rho(y2 . Wr[e]); P = rho(softmax_fp32(l)) over all E experts;
 *   S = the k largest P (ties -> lower expert index), in slot order of
 *   descending P then ascending index;
 *   if norm: den = rho(sum_{s in S} P_s), w_s = rho(P_s / den); else w_s = P_s.
 * idx [T][k], w [T][k]; probs (optional) [T][E] receives P. */
void orc_router(const float *y2, int T, int hid, const float *Wr, int E, int k, int norm,
                int mode, int32_t *idx, float *w, float *probs);

/* MoE block ([P3] forward + SwitchGLU experts): router as above, then for
 * each selected expert e: gu = rho(y2 . Wgu_e^T) with Wgu_e = [gate_e; up_e]
 * ([2*Ie][hid]), m = swiglu(gu), y_e = rho(m . Wd_e^T) (Wd_e [hid][Ie]);
 * out[t] = rho(sum_slots rho(y_e * w_s)).
 * sorted = 0 runs the experts in token order ([P3] Qwen3UnsortedExperts);
 * sorted = 1 sorts the (token, slot) rows by expert, runs them in that order
 * and un-permutes ([P3] Qwen3SortedExperts).  Both orders give the same
 * result bit for bit.  idx, w (optional) receive the routing. */
void orc_moe_block(const float *y2, int T, int hid, const float *Wr, int E, int k, int Ie,
                   int norm, const float *Wgu_e, const float *Wd_e, int sorted, int mode,
                   float *out, int32_t *idx, float *w);

/* 8-bit affine group quantisation along K (groups of `group`):
 * w_hat[j][k] = fp32(fp32(s[j][k/group] * q[j][k]) + b[j][k/group]). */
void orc_q8_dequant(const uint8_t *q, const float *s, const float *b, int N, int K, int group,
                    float *out);
/* Test-data quantiser: per group min/max, s = bf16((max-min)/255),
 * b = bf16(min), q = clamp(rne((w-b)/s), 0, 255), q = 0 where s == 0. */
void orc_q8_quantize(const float *w, int N, int K, int group, uint8_t *q, float *s, float *b);

typedef struct {
    int n_layers, hidden, n_heads, n_kv_heads, head_dim, intermediate, capacity;
    float rms_eps;
    int mode;                 /* ORC_BF16 or ORC_FP32 */
    int n_experts, top_k, moe_intermediate, norm_topk_prob; /* n_experts == 0: dense MLP */
    /* [P2] Qwen3DecoderSpec switches: qk_norm (1: per-head q/k RMSNorm before RoPE, Qwen3;
     * 0: RoPE on the projections, Qwen2), attention_bias (1: q/k/v bias added to the
     * projection, each add rounded: [P2] mm then add), window (0: causal; w > 0: the
     * SlidingWindow(w) mask of orc_attention). */
    int qk_norm, attention_bias, window;
} orc_config;
/* Layer kind ([P3] Qwen3MoeDecoderLayer: a layer runs the sparse MoE block unless its index is
 * in mlp_only_layers or (index + 1) is not a multiple of decoder_sparse_step, and the dense
 * MLP otherwise): with n_experts > 0, a layer whose router is NULL runs the dense MLP of
 * intermediate width from gate_up / down; the caller applies the index rule when it builds the
 * layers. */

typedef struct {
    const float *in_norm, *post_norm, *q_norm, *k_norm; /* [hid], [hid], [D], [D] */
    const float *qkv;      /* [(H+2KV)D][hid]: q rows, then k rows, then v rows */
    const float *o;        /* [hid][H*D] */
    const float *gate_up;  /* [2I][hid]: gate rows, then up rows (dense layers) */
    const float *down;     /* [hid][I] */
    const float *router;   /* [E][hid] (MoE layers; NULL: dense layer of an MoE stack) */
    const float *exp_gate_up; /* [E][2Ie][hid] */
    const float *exp_down;    /* [E][hid][Ie] */
    const float *qkv_bias;    /* [(H+2KV)D] (attention_bias) */
} orc_layer;

/* One forward call of the stack ([P1] Backbone.forward): x [T][hid] at
 * positions *length .. *length+T-1; writes the new K/V entries of every layer
 * into kcache/vcache ([n_layers][KV][capacity][D]), advances *length by T and
 * returns the final-norm hidden states in out [T][hid].
 * cos/sin: the [capacity][D] table from orc_rope_table.
 * Returns ORC_ERR_ARG for T < 1 or a layer without the weights of its kind
 * (dense: gate_up, down and intermediate >= 1; MoE: exp_gate_up, exp_down and
 * 1 <= top_k <= n_experts), ORC_ERR_CAPACITY when *length + T exceeds
 * capacity; then nothing is written. */
int orc_forward(const orc_config *cfg, const orc_layer *layers, const float *final_norm,
                const float *cos_tab, const float *sin_tab, float *kcache, float *vcache,
                int *length, const float *x, int T, float *out);

/* Threads the oracle's OpenMP loops use (0 = the OpenMP default). */
void orc_set_threads(int n);
int orc_get_threads(void);

#ifdef __cplusplus
}
#endif
#endif
