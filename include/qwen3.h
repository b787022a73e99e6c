/*
 * qwen3.h -- C ABI of the MI355X (gfx950) Qwen3 decoder-stack forward over a
 * static per-seat KV cache, with the Qwen3-MoE block and 8-bit affine group
 * quantised projections.
 *
 * What is computed (the pages):
 *  - "maya2_mlx/backbone.py", module docstring and Backbone.forward(): per
 *    layer h = h + pend (one rounding); y = RMSNorm(h) (two roundings);
 *    qkv = y [Wq;Wk;Wv]^T; per-head RMSNorm of q and k (two roundings); RoPE in
 *    fp32 on the model-dtype cos/sin table (one rounding); attention over keys
 *    0..pos with an fp32 softmax (one rounding); h = h + o_proj(attn);
 *    y2 = RMSNorm(h); pend = down(silu(g) * u) with silu in fp32 rounded once.
 *    After the last layer h = h + pend and the result is RMSNorm(h, norm).
 *    bf16 is the production dtype, fp32 the strict one.
 *  - "@mlx-bun/inference" qwen3-moe.ts, Qwen3MoeSparseMoeBlock.forward: router
 *    linear, softmax over all experts, top-k, renormalise, per-expert SwiGLU,
 *    weighted sum.
 *  - "rlx_flow/blocks/qwen3_decoder.rs", emit(): GQA, q head h reads kv head
 *    h / (n_heads / n_kv_heads).
 *
 * Rounding: "rho" below is round-to-nearest-even to bf16 in QWEN3_BF16 mode and
 * the identity in QWEN3_FP32 mode; the kernels accumulate in fp32.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless marked "host".  The library never
 *    allocates device memory: weights, the KV cache and the workspace are
 *    provided by the caller and BORROWED for the handle's lifetime; inputs are
 *    borrowed for the call; outputs are written into caller buffers.
 *  - All work is enqueued asynchronously on the handle's HIP stream; no call
 *    synchronises.  The caller synchronises the stream before reading outputs.
 *  - Every call returns QWEN3_OK (0) or a negative QWEN3_ERR_* code.  All
 *    argument checks run on the host before anything is enqueued, so a failed
 *    call leaves the cache, the seat length and all outputs unchanged (the
 *    capacity check of Backbone.forward raises before any state change).
 *    qwen3_last_error() then describes the failure.  A QWEN3_ERR_HIP from a
 *    launch can leave work partly enqueued.
 *  - A handle is one seat and is not thread-safe.
 *  - Alignment: the kernels move weight, cache, table and activation rows in
 *    16-byte vector accesses, so every device pointer qwen3_init takes (each
 *    weight, scale, bias and norm vector, the embedding and RoPE tables, both
 *    caches) and the hidden-state inputs and outputs of the forward calls must
 *    be 16-byte aligned; token ids, routing outputs, logits and argmax need
 *    their element alignment.  A misaligned pointer gives QWEN3_ERR_ARG before
 *    anything is enqueued (torch allocations are aligned; a view at an odd
 *    element offset may not be).
 *
 * Layouts (row-major, model dtype = bf16 or fp32 unless stated):
 *  - projection weights are [out][in]: q|k|v fused as [(H+2KV)*D][hidden]
 *    (q rows, then k rows, then v rows), o as [hidden][H*D], gate|up fused as
 *    [2*I][hidden] (gate rows first), down as [hidden][I] ("fuse_proj" of
 *    Backbone.__init__);
 *  - 8-bit projections (quant_bits == 8): u8 codes [out][in], plus bf16 scale
 *    and bias [out][in/quant_group]; w = scale * code + bias per group along
 *    the input axis; q|k|v and gate|up are quantised as the fused rows;
 *  - MoE: router [E][hidden], expert gate|up [E][2*Ie][hidden], expert down
 *    [E][hidden][Ie]; with quant_bits == 8 all three are u8 codes of those
 *    shapes with bf16 scale and bias [E][hidden/64], [E][2*Ie][hidden/64] and
 *    [E][hidden][Ie/64] ("@mlx-bun/inference" qwen3-moe.ts, the quantised gate
 *    Linear and QuantizedSwitchLinear experts of Qwen3SwitchWeights);
 *  - layer kind in an MoE configuration (n_experts > 0; qwen3-moe.ts,
 *    Qwen3MoeDecoderLayer: a layer is sparse unless its index is in
 *    mlp_only_layers or (index + 1) is not a multiple of decoder_sparse_step):
 *    a layer with a router runs the MoE block, a layer whose router is NULL
 *    runs the dense MLP (gate_up / down of width intermediate); the caller
 *    applies the index rule when it fills the layer array;
 *  - KV cache: K and V each [n_layers][n_kv_heads][capacity][head_dim]; the
 *    cache holds post-norm, post-RoPE keys and raw values (Backbone.reset and
 *    forward).  Entries at positions >= the seat length are never read;
 *  - RoPE table: cos and sin each [capacity][head_dim], halves duplicated.
 */
#ifndef QWEN3_H
#define QWEN3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { QWEN3_BF16 = 0, QWEN3_FP32 = 1 } qwen3_dtype;

enum {
    QWEN3_OK = 0,
    QWEN3_ERR_ARG = -1,         /* bad argument: null pointer, T < 1, bad layer index, ... */
    QWEN3_ERR_DTYPE = -2,       /* dtype neither bf16 nor fp32 (Backbone.__init__ dtype gate) */
    QWEN3_ERR_CAPACITY = -3,    /* length + T exceeds capacity (Backbone.forward) */
    QWEN3_ERR_NULL_WEIGHT = -4, /* a weight the configuration needs is NULL */
    QWEN3_ERR_UNSUPPORTED = -5, /* a shape the kernels do not handle (see qwen3_init) */
    QWEN3_ERR_HIP = -6,         /* a HIP runtime call or kernel launch failed */
    QWEN3_ERR_WORKSPACE = -7    /* workspace missing or smaller than qwen3_workspace_bytes() */
};

typedef struct {
    int n_layers, hidden, n_heads, n_kv_heads, head_dim, intermediate, vocab, capacity;
    float rms_eps;
    double rope_theta;
    int dtype;                 /* qwen3_dtype */
    int n_experts, top_k, moe_intermediate, norm_topk_prob; /* n_experts == 0: dense MLP */
    int quant_bits, quant_group; /* 0 (plain weights) or 8 with quant_group 64 */
    int max_tokens;            /* largest T per call; sizes the workspace */
    int sliding_window;        /* 0: causal (keys 0..p); w > 0: SlidingWindow(w), keys max(0, p-w+1)..p
                                  ("rlx_flow/blocks/qwen3_decoder.rs", Qwen3DecoderSpec mask) */
} qwen3_config;

typedef struct {
    const void *in_norm, *post_norm, *q_norm, *k_norm; /* [hidden], [hidden], [D], [D]; q_norm and
                                                          k_norm both NULL: no per-head q/k RMSNorm
                                                          (Qwen3DecoderSpec qk_norm off, Qwen2) */
    const void *qkv, *o, *gate_up, *down;               /* plain weights, or u8 codes if quantised */
    const void *qkv_s, *qkv_b, *o_s, *o_b;              /* bf16 per-group scale and bias (quantised) */
    const void *gate_up_s, *gate_up_b, *down_s, *down_b;
    const void *router, *exp_gate_up, *exp_down;        /* MoE layers (u8 codes if quantised) */
    const void *router_s, *router_b;                    /* bf16 per-group scale and bias of the */
    const void *exp_gate_up_s, *exp_gate_up_b;          /* quantised MoE weights */
    const void *exp_down_s, *exp_down_b;
    const void *qkv_bias;     /* [(H+2KV)*D] model dtype or NULL (Qwen2 attention_bias: q|k|v each
                                 become rho(x + b) after the projection) */
} qwen3_layer_weights;

typedef struct {
    const void *embed;        /* [vocab][hidden]; may be NULL when only qwen3_forward_hidden is used */
    const void *final_norm;   /* [hidden] */
    const void *rope_cos, *rope_sin; /* [capacity][D] each, or both NULL: built by qwen3_init */
    const qwen3_layer_weights *layers; /* HOST array [n_layers]; copied by qwen3_init */
} qwen3_weights;

typedef struct qwen3_handle qwen3_handle;

/* Bytes of device workspace qwen3_init needs for this configuration (0 when
 * the configuration is invalid).  The workspace holds activations, attention
 * partials, MoE routing buffers and, when not supplied, the RoPE table. */
size_t qwen3_workspace_bytes(const qwen3_config *cfg);

/* Create a seat (Backbone.__init__ + reset without the zeroing: the caller's
 * cache is used as is and the seat length starts at 0).
 *   cfg, w: host structs, copied; the device buffers they point to are borrowed.
 *   k_cache, v_cache: [n_layers][n_kv_heads][capacity][head_dim] each.
 *   workspace: ws_bytes >= qwen3_workspace_bytes(cfg), 256-byte aligned.
 *   stream: hipStream_t for every enqueue (NULL = the null stream).
 * Supported: head_dim 64 or 128; n_heads a multiple of n_kv_heads; hidden,
 * intermediate and moe_intermediate multiples of 64 (intermediate may be 0 in
 * an MoE configuration without dense layers); quant_group 64.  Returns
 * QWEN3_ERR_UNSUPPORTED otherwise, QWEN3_ERR_DTYPE for another dtype,
 * QWEN3_ERR_NULL_WEIGHT for a missing weight.  *out is set only on success. */
int qwen3_init(const qwen3_config *cfg, const qwen3_weights *w, void *k_cache, void *v_cache,
               void *workspace, size_t ws_bytes, void *stream, qwen3_handle **out);

/* Zero the K/V cache of every layer and set the length to 0 (Backbone.reset). */
int qwen3_reset(qwen3_handle *h);

/* Forward T token ids (device int32 [T], each in [0, vocab)) at positions
 * length..length+T-1: embedding gather (Backbone.embed_tokens), then
 * qwen3_forward_hidden.  out: [T][hidden] final-norm hidden states.
 * QWEN3_ERR_NULL_WEIGHT when the handle has no embedding table.  Ids are not
 * range-checked on the host (they live on the device); the gather clamps an
 * out-of-range id to 0 and sets the handle's device error flag, which
 * qwen3_check_device_errors reports. */
int qwen3_forward(qwen3_handle *h, const int32_t *tokens, int T, void *out);

/* Forward hidden states x [T][hidden] (model dtype) at positions
 * length..length+T-1 through every layer (Backbone.forward): writes the new
 * K/V entries, advances the length by T and writes the final-norm hidden
 * states to out [T][hidden].  T == 1 takes the decode kernels (split-K
 * attention), T > 1 the prefill kernels (causal attention: the query at
 * position p sees keys 0..p).  Errors: QWEN3_ERR_ARG (T < 1 or T > max_tokens),
 * QWEN3_ERR_CAPACITY (length + T > capacity). */
int qwen3_forward_hidden(qwen3_handle *h, const void *x, int T, void *out);

/* The MoE block of layer `layer` on already-normalised rows x [T][hidden]
 * (Qwen3MoeSparseMoeBlock.forward): out [T][hidden].  topk_idx (int32 [T][top_k])
 * and topk_w (model dtype [T][top_k]) receive the routing when not NULL: the
 * selected experts in slot order of descending probability, ties to the lower
 * expert index.  Does not touch the cache or the length.  Errors:
 * QWEN3_ERR_ARG (not an MoE configuration, layer out of range or a dense
 * layer, T < 1 or T > max_tokens). */
int qwen3_moe_block(qwen3_handle *h, int layer, const void *x, int T, void *out, int32_t *topk_idx,
                    void *topk_w);

/* One decode step for B seats at once (page 3 "decode": one new token per sequence; page 2
 * batch): row b of x [B][hidden] (model dtype) is seat b's next token at position
 * seats[b]'s length; out [B][hidden] gets the final-norm hidden states and every seat's
 * length advances by 1.  seats: host array of B distinct handles with the same configuration
 * (all shape fields, capacity, eps, theta, dtype, MoE and quantisation fields) and the same
 * weight pointers; each keeps its own cache and length.  The projections read each weight
 * once for the B rows; attention runs per seat in one batched launch.  The activations and
 * the stream are seats[0]'s (its max_tokens must be >= B).  1 <= B <= 16.  Errors:
 * QWEN3_ERR_ARG (B out of range, a null or repeated seat, a seat of another model),
 * QWEN3_ERR_CAPACITY (a seat is full); on error no seat changes. */
int qwen3_forward_batch(qwen3_handle *const *seats, int B, const void *x, void *out);

/* Output head and greedy token ("maya2_mlx/backbone.py" Backbone.cb0_logits: the head
 * projection in the model dtype, then fp32; "@mlx-bun/inference" qwen3.ts lmHead or the tied
 * embedding used as a linear) on final-norm hidden states hs [T][hidden] (model dtype):
 *   logits[t][v] = fp32(rho(hs[t] . head[v]))  (fp32 [T][V], may be NULL)
 *   argmax[t]    = the lowest v with the largest logit; a NaN logit is never picked unless
 *                  every logit is NaN (then 0)  (int32 [T], may be NULL)
 * head: [V][hidden] in the model dtype, or NULL for the handle's embedding table (tied
 * weights, V must equal vocab).  All pointers are device memory; the call enqueues on the
 * handle's stream and does not touch the cache or the length.  Errors: QWEN3_ERR_ARG (null
 * hs, neither output requested, T outside 1..max_tokens, V < 1 or V != vocab when tied),
 * QWEN3_ERR_NULL_WEIGHT (no head and no embedding table). */
int qwen3_head(qwen3_handle *h, const void *hs, int T, const void *head, int V, float *logits, int32_t *argmax);

/* qwen3_head without a handle or workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same logits and greedy token as qwen3_head, for hs [T][hidden] and head [V][hidden] in
 * `dtype`, enqueued on `stream` (which must belong to the current device; NULL = the null
 * stream).  The per-row greedy-token keys live in a static array the library keeps on each
 * device for the rest of the process (QWEN3_HEAD_STATIC_MAX_T * 64 64-bit words, 128 KB);
 * nothing is allocated, and the call clears the keys itself.  Calls that overlap on one
 * device (other streams, other threads) share that array and race: serialise them.
 * Errors: QWEN3_ERR_DTYPE; QWEN3_ERR_ARG for a null or misaligned pointer, neither output
 * requested, T outside 1..QWEN3_HEAD_STATIC_MAX_T, V < 1, or hidden not a positive multiple
 * of 64; QWEN3_ERR_HIP when the array's address cannot be found or a launch fails. */
#define QWEN3_HEAD_STATIC_MAX_T 256
int qwen3_head_static(int dtype, const void *hs, int T, int hidden, const void *head, int V, float *logits,
                      int32_t *argmax, void *stream);

/* Set the seat length (0 <= length <= capacity): a pre-filled cache, or a
 * rewind.  Entries at positions >= length are never read and are overwritten
 * by the next forward. */
int qwen3_set_length(qwen3_handle *h, int length);
int qwen3_get_length(const qwen3_handle *h);

/* Use another HIP stream for later calls. */
int qwen3_set_stream(qwen3_handle *h, void *stream);

/* Kernel structure of T == 1 steps.  path 0: automatic (default) -- the persistent decode
 * kernel when the configuration and device support it, on a device that holds 256
 * co-resident blocks of 704 threads: dense bf16 stacks with bf16 or 8-bit group-quantised
 * projection weights (quant_group 64), head_dim 128, hidden 2048 = n_heads * head_dim,
 * intermediate 6144, 2 query heads per kv head, capacity <= 8192; or MoE stacks (bf16 or
 * 8-bit weights, router and experts included) whose every layer has a router, with hidden
 * 2048, 32 q / 4 kv heads of 128, 8 to 128 experts, top 8, moe_intermediate 768, capacity
 * <= 8192 -- else one kernel per
 * step of the layer; 1: always one kernel per step; 2: require the persistent kernel
 * (QWEN3_ERR_UNSUPPORTED when unavailable).  Both compute the same values up to fp32
 * summation order.  qwen3_get_decode_path returns the path T == 1 calls take (1 or 2).
 * The persistent kernel's blocks wait on each other's results, so all 256 must run at once:
 * an eager call launches it cooperatively (the runtime guarantees co-residency or fails the
 * launch), but a launch recorded into a HIP graph is a plain launch, and co-residency then
 * rests on the occupancy check qwen3_init made and on no other work holding CUs while the
 * graph runs (the GPU used by this process alone, no kernels on other streams overlapping
 * the step).  If blocks cannot all run, every wait gives up after about a second: the call
 * still returns QWEN3_OK (it only enqueues), the step's outputs are invalid, and only
 * qwen3_check_device_errors reports it (QWEN3_ERR_HIP). */
int qwen3_set_decode_path(qwen3_handle *h, int path);
int qwen3_get_decode_path(const qwen3_handle *h);

/* Synchronise the handle's stream and report device-side errors raised since
 * the last check: an out-of-range token id (QWEN3_ERR_ARG) or a persistent decode
 * step that timed out waiting for another block's results (QWEN3_ERR_HIP; the
 * step's outputs are invalid).  The flags are then cleared.  Together with
 * qwen3_init (which synchronises once to upload the persistent kernel's layer
 * table), the only entry points that synchronise. */
int qwen3_check_device_errors(qwen3_handle *h);

/* Text of the last failure on this handle ("" when none); valid until the
 * next call on the handle.  qwen3_status_string names a return code. */
const char *qwen3_last_error(const qwen3_handle *h);
const char *qwen3_status_string(int code);

/* Free the handle (host memory only; borrowed buffers stay the caller's). */
void qwen3_destroy(qwen3_handle *h);

/* Build the RoPE table (Backbone.__init__ table comment, _rope):
 * inv_j = fp32(theta^(-2j/D)), rounded to bf16 in bf16 mode;
 * angle = fp32(p * inv_j); cos[p][j] = cos[p][j + D/2] = rho(fp32(cos(angle))),
 * sin likewise.  cos, sin: [capacity][head_dim] in `dtype`. */
int qwen3_rope_table(int capacity, int head_dim, double theta, int dtype, void *cos_out, void *sin_out,
                     void *stream);

#ifdef __cplusplus
}
#endif
#endif
