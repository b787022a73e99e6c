/*
 * qwen3_ops.h -- single-kernel entry points of libqwen3, for per-kernel parity
 * tests.  Not the user API (that is qwen3.h).  Same conventions: device
 * pointers, asynchronous on `stream` (a hipStream_t, NULL = null stream),
 * QWEN3_OK or a negative QWEN3_ERR_* code, host-side argument checks before
 * any enqueue.  `dtype` is QWEN3_BF16 or QWEN3_FP32 for every model-dtype
 * buffer.
 */
#ifndef QWEN3_OPS_H
#define QWEN3_OPS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Rows t < T of width n ("maya2_mlx/backbone.py" docstring: h = h + pend with
 * one rounding; RMSNorm with two roundings): h = res ? rho(h_in + res) : h_in,
 * written to h_out when res and h_out are both given; y = rho(w * rho(h * r)),
 * r = 1/sqrt(mean(h^2) + eps).  n must be a multiple of 8. */
int qwen3_op_add_rmsnorm(int dtype, const void *h_in, const void *res, const void *w, void *h_out, void *y, int T,
                         int n, float eps, void *stream);

/* Projection x [M][K] . W^T with an epilogue (Backbone.forward's Q.mm calls):
 * epilogue 0: out[m][n] = rho(acc), W [N][K];
 * epilogue 1: out[m][n] = rho(res[m][n] + rho(acc)) (o_proj + residual);
 * epilogue 2: W [2N][K] = gate rows then up rows,
 *             out[m][n] = rho(rho(silu(rho(g))) * rho(u)) (silu in fp32).
 * K must be a multiple of 64; for M > 16 N must be a multiple of 128
 * (epilogue 2: of 64) in bf16. */
int qwen3_op_linear(int dtype, const void *x, int M, int K, const void *W, int N, int epilogue, const void *res,
                    void *out, void *stream);

/* The same with 8-bit affine group weights (bf16 activations): codes u8 [rows][K],
 * scale and bias bf16 [rows][K/64]; w = scale * code + bias, kept in fp32.
 * QWEN3_ERR_UNSUPPORTED for M <= 16 with K > 8192. */
int qwen3_op_linear_q8(const void *x, int M, int K, const uint8_t *codes, const void *scale, const void *bias,
                       int N, int epilogue, const void *res, void *out, void *stream);

/* Per token t < T and head: per-head RMSNorm over head_dim D with q_norm / k_norm
 * (two roundings), rotate-half RoPE at position p0 + t from the cos/sin table
 * [cap][D] (fp32 maths, one rounding); q heads to q_out [T][H][D]; k heads and
 * the raw v rows into the cache [KV][cap][D] at position p0 + t
 * (Backbone._rope and forward).  qkv: [T][(H+2KV)D]. */
int qwen3_op_qknorm_rope_kv(int dtype, const void *qkv, int T, int H, int KV, int D, const void *q_norm,
                            const void *k_norm, float eps, const void *cos_t, const void *sin_t, int p0, int cap,
                            void *q_out, void *k_cache, void *v_cache, void *stream);

/* Causal GQA attention: queries q [T][H][D] at positions p0..p0+T-1, keys and
 * values 0..p0+T-1 of the cache [KV][cap][D]; out [T][H*D].  T == 1 runs the
 * split-K decode kernels, T > 1 the prefill kernel.  ws: fp32 scratch of
 * qwen3_op_attention_workspace() bytes. */
size_t qwen3_op_attention_workspace(int T, int H, int KV, int D, int cap);
int qwen3_op_attention(int dtype, const void *q, const void *k_cache, const void *v_cache, int T, int H, int KV, int D,
                       int cap, int p0, void *out, void *ws, size_t ws_bytes, void *stream);

/* MoE block on normalised rows x [T][hid] ("@mlx-bun/inference" qwen3-moe.ts,
 * Qwen3MoeSparseMoeBlock.forward): idx int32 [T][k], w [T][k] (model dtype),
 * out [T][hid].  ws: qwen3_op_moe_workspace() bytes.  E <= 256, k <= 16,
 * Ie a multiple of 64. */
size_t qwen3_op_moe_workspace(int dtype, int T, int hid, int E, int k, int Ie);
int qwen3_op_moe(int dtype, const void *x, int T, int hid, const void *router, int E, int k, int norm, int Ie,
                 const void *exp_gate_up, const void *exp_down, int32_t *idx, void *w, void *out, void *ws,
                 size_t ws_bytes, void *stream);

/* Streaming-read probe, for the measured HBM read peak reported beside the published one
 * (not part of the layer): reads src[0 .. bytes) with 16-byte non-temporal loads.  Thread t of
 * the 256 x 256-thread grid reads the 16-byte words t, t + 65536, t + 2 * 65536, ... and
 * writes to out[t] the XOR of their 32-bit words.  bytes: a positive multiple of 16; src
 * 16-byte aligned; out: 65536 words (256 KiB), 4-byte aligned.  QWEN3_ERR_ARG otherwise,
 * before any launch. */
int qwen3_op_stream_read(const void *src, size_t bytes, uint32_t *out, void *stream);

/* Kernel timing for measurement.  While enabled for a kind (0 q|k|v projection,
 * 1 o_proj, 2 gate|up projection, 3 down projection, 4 attention, 5 the persistent
 * decode kernel of a whole T == 1 step), every launch of
 * that kind by qwen3_forward / qwen3_forward_hidden on handle h is bracketed by two
 * HIP events recorded on the handle's stream.  qwen3_kernel_timer_read synchronises
 * on those events and returns the summed duration in ms and the launch count since
 * the timer was (re)enabled.  Enabling resets the sums. */
typedef struct qwen3_handle qwen3_handle;
int qwen3_kernel_timer(qwen3_handle *h, int kind, int enable);
int qwen3_kernel_timer_read(qwen3_handle *h, int kind, double *total_ms, int *count);

#ifdef __cplusplus
}
#endif
#endif
