// kernels.h -- host-side launchers of the gfx950 kernels (internal to libqwen3).
// Every launcher validates nothing the host layer already checked; it returns
// the hipError_t of the launch.  Pointers are device pointers; `dt` selects
// bf16 or fp32 storage for every model-dtype buffer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace q3 {

enum Epi { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_QKV = 3 };

// What the fused q|k|v epilogue (EPI_QKV) needs besides the GEMM operands: per-head q/k RMSNorm
// weights (both null: no q/k norm), q|k|v bias (or null), the RoPE table, the first position
// p0 of the call, and the destinations: q [T][H][D], the layer's K and V caches [KV][cap][D].
struct QkvEpi {
    const void *q_norm = nullptr, *k_norm = nullptr, *bias = nullptr, *cos_t = nullptr, *sin_t = nullptr;
    float eps = 0.f;
    int H = 0, KV = 0, p0 = 0, cap = 0;
    void *q_out = nullptr, *kc = nullptr, *vc = nullptr;
};

// out[t] = E[ids[t]] (ids outside [0, vocab) read row 0 and set *err).
hipError_t launch_embed(int dt, const int32_t *ids, int T, const void *E, int vocab, int hid, void *out,
                        int *err, hipStream_t s);

// Per row t < T: h = res ? rho(h_in + res) : h_in (written to h_out when res and h_out);
// y = rho(w * rho(h * r)), r = 1/sqrt(mean(h^2) + eps).
// Streaming read of `bytes` (a multiple of 16) for the measured HBM read peak; out: 256 * 256 words.
hipError_t launch_stream_read(const void *src, size_t bytes, void *out, hipStream_t s);
hipError_t launch_add_rmsnorm(int dt, const void *h_in, const void *res, const void *w, void *h_out, void *y,
                              int T, int n, float eps, hipStream_t s);

// RoPE table [cap][D] (cos, sin) in storage dt.
hipError_t launch_rope_table(int dt, int cap, int D, double theta, void *cos_t, void *sin_t, hipStream_t s);

// Per token t and head: bias add (bias [(H+2KV)D] or NULL), per-head RMSNorm (q_norm / k_norm
// weights; both NULL: no norm), RoPE at p0 + t, q to q_out [T][H][D]; k and v (plus bias)
// written to the cache at position p0 + t.
hipError_t launch_qknorm_rope_kv(int dt, const void *qkv, int T, int H, int KV, int D, const void *q_norm,
                                 const void *k_norm, const void *bias, float eps, const void *cos_t,
                                 const void *sin_t, int p0, int cap, void *q_out, void *k_cache, void *v_cache,
                                 hipStream_t s);

// out = epilogue(x [M][K] . W^T), W [rows][K] row-major.
//  EPI_STORE:  out[m][n] = rho(acc), n < N (W has N rows)
//  EPI_RESID:  out[m][n] = rho(res[m][n] + rho(acc))
//  EPI_SWIGLU: W has 2N rows (gate rows then up rows);
//              out[m][n] = rho(rho(silu(rho(g))) * rho(u))
hipError_t launch_linear(int dt, const void *x, int M, int K, const void *W, int N, int epi, const void *res,
                         void *out, hipStream_t s);

// Decode projection (M == 1) with the RMSNorm prologue:
//   h = res ? rho(h_in + res) : h_in   (written to h_out by one block when res and h_out)
//   y = rho(nw * rho(h * r)), out = epilogue(y . W^T) with EPI_STORE or EPI_SWIGLU.
// h_out must not alias h_in or res.
hipError_t launch_linear_norm(int dt, const void *h_in, const void *res, const void *nw, float eps, void *h_out,
                              int K, const void *W, int N, int epi, void *out, hipStream_t s);
hipError_t launch_linear_q8_norm(const void *h_in, const void *res, const void *nw, float eps, void *h_out, int K,
                                 const uint8_t *codes, const void *scale, const void *bias, int group, int N,
                                 int epi, void *out, hipStream_t s);

// Same with 8-bit affine group weights: codes u8 [rows][K], scale/bias bf16 [rows][K/64]
// (group must be 64); x, res and out are bf16.  Dequantised weights stay fp32.
hipError_t launch_linear_q8(const void *x, int M, int K, const uint8_t *codes, const void *scale,
                            const void *bias, int group, int N, int epi, const void *res, void *out, hipStream_t s);

// Causal GQA attention of T queries at positions p0..p0+T-1 against cache entries
// 0..p0+T-1: q [T][H][D] -> out [T][H*D].  ws: fp32 scratch of attention_workspace() bytes.
// window: 0 causal (query at p sees keys 0..p) or w > 0, a sliding window (keys max(0, p-w+1)..p).
hipError_t launch_attention(int dt, const void *q, const void *k_cache, const void *v_cache, int T, int H, int KV,
                            int D, int cap, int p0, int window, void *out, float *ws, size_t ws_bytes, hipStream_t s);
size_t attention_workspace(int T, int H, int KV, int D, int cap);
// Decode step (T == 1) at position p0 fused with the bias add (bias or NULL), the per-head
// q/k RMSNorm (q_norm and k_norm, or both NULL), RoPE and the cache write: qkv [(H+2KV)D] of
// the token -> out [H*D]; writes K/V at p0; window as for launch_attention.  The scratch of
// attention_workspace(T, ...) holds min(T, DECODE_MAXB) seats' partials.
hipError_t launch_attention_decode_fused(int dt, const void *qkv, int H, int KV, int D, const void *q_norm,
                                         const void *k_norm, const void *bias, float eps, const void *cos_t,
                                         const void *sin_t, int p0, int cap, int window, void *k_cache,
                                         void *v_cache, void *out, float *ws, hipStream_t s);
// The same for B <= DECODE_MAXB seats at once (one token each, the same weights): seat b's
// q|k|v row b of qkv [B][(H+2KV)D], its layer cache kc[b] / vc[b] ([KV][cap][D]) and position
// p[b]; out row b of [B][H*D].
constexpr int DECODE_MAXB = 16;
struct DecodeBatch {
    void *kc[DECODE_MAXB], *vc[DECODE_MAXB];
    int p[DECODE_MAXB], lo[DECODE_MAXB], chunk[DECODE_MAXB], nsplit[DECODE_MAXB];
};
hipError_t launch_attention_decode_batch(int dt, const void *qkv, int B, int H, int KV, int D, const void *q_norm,
                                         const void *k_norm, const void *bias, float eps, const void *cos_t,
                                         const void *sin_t, void *const *k_cache, void *const *v_cache, const int *p,
                                         int cap, int window, void *out, float *ws, hipStream_t s);

// ---- MoE block: router logits rho(x . Wr^T), rho(softmax) over all E experts, top-k
// (ties to the lower index, slot order descending probability), renormalised weights
// w [T][k] (storage dt), expert SwiGLU FFNs and out [T][hid] = rho(sum_s rho(y_s * w_s)).
// idx: int32 [T][k].  ws: moe_workspace() bytes.  Requires E <= 256, k <= 16.
// Weights: router [E][hid], gate|up [E][2*Ie][hid], down [E][hid][Ie] in the model dtype, or
// (q8, bf16 only) u8 codes of those shapes with bf16 scale and bias [rows][in/64] each.
struct MoeWeights {
    const void *router, *router_s, *router_b;
    const void *gate_up, *gate_up_s, *gate_up_b;
    const void *down, *down_s, *down_b;
    bool q8;
};
size_t moe_workspace(int T, int hid, int E, int k, int Ie, int dt);
hipError_t launch_moe(int dt, const void *x, int T, int hid, const MoeWeights &W, int E, int k, int norm, int Ie,
                      int32_t *idx, void *w, void *out, void *ws, hipStream_t s);
// One token with the RMSNorm in front: y = rho(nw * rho(h * r)) (the post-attention norm of a
// decode step), then the MoE block of y; out, idx, w and ws as for launch_moe with T = 1.
hipError_t launch_moe_norm1(int dt, const void *h, const void *nw, float eps, int hid, const MoeWeights &W, int E,
                            int k, int norm, int Ie, int32_t *idx, void *w, void *out, void *ws, hipStream_t s);

// ---- output head + greedy token (kernels_head.hip): logits fp32 [T][V] and/or argmax int32 [T];
// keys: 64 T 64-bit words of scratch
hipError_t launch_head(int dt, const void *hs, int T, int K, const void *W, int V, float *logits, int32_t *argmax,
                       unsigned long long *keys, hipStream_t s);
// The same with the keys in the library's per-device static array (no workspace, nothing
// allocated): T <= HEAD_STATIC_MAX_T rows; the stream must belong to the current device.
constexpr int HEAD_STATIC_MAX_T = 256;
hipError_t launch_head_static(int dt, const void *hs, int T, int K, const void *W, int V, float *logits,
                              int32_t *argmax, hipStream_t s);

// ---- MFMA projections for M > 16 (kernels_gemm.hip): LDS-DMA pipeline, K % 64 == 0 (bf16
// weights) or K % 128 == 0 and 4-byte aligned scale/bias (8-bit weights)
bool gemm_dma_ok(int M, int K, int N);
hipError_t launch_gemm_dma(const void *x, int M, int K, const void *W, int N, int epi, const void *res, void *out,
                           hipStream_t s);
// q|k|v projection of T > 1 tokens with the per-head q/k RMSNorm, RoPE and K/V cache write in
// the epilogue (bf16, head_dim 128): true when the tiling it needs fills the chip at this M.
bool gemm_qkv_fused_ok(int M, int K, int H, int KV, int D);
hipError_t launch_gemm_qkv_fused(const void *x, int M, int K, const void *W, const QkvEpi &qe, hipStream_t s);
bool gemm_q8_dma_ok(int M, int K, int N, const void *scale, const void *bias);
hipError_t launch_gemm_q8_dma(const void *x, int M, int K, const uint8_t *codes, const void *scale, const void *bias,
                              int N, int epi, const void *res, void *out, hipStream_t s);

// ---- persistent decode step (kernels_decode_mk.hip): dense bf16 stacks of supported shape,
// bf16 or 8-bit (groups of 64) weights
bool decode_mk_supported(int n_layers, int dt, int n_experts, int quant_bits, int hid, int H, int KV, int D, int I, int cap);
size_t decode_mk_workspace(int n_layers, int H, int KV, int hid, int I);
// Copies the per-layer weight pointers (host array of 9 pointers per layer: in_norm, post_norm,
// q_norm, k_norm, qkv, o, gate_up, down, qkv_bias; q/k norm and bias may be null; with 8-bit
// weights the projections are the code arrays and layer_q8_ptrs holds 8 pointers per layer:
// qkv, o, gate_up, down scale then bias; else null) into ws and clears the exchange buffers;
// synchronises s.
hipError_t decode_mk_init(void *ws, int n_layers, int H, int KV, int hid, int I, const void *layer_ptrs,
                          const void *layer_q8_ptrs, hipStream_t s);
hipError_t launch_decode_mk(void *ws, int n_layers, int H, int KV, int hid, int I, bool q8, int cap, int p, int window,
                            float eps, const void *x, void *out, const void *final_norm, const void *cos_t,
                            const void *sin_t, void *kc, void *vc, int *err, hipStream_t s);
int decode_mk_max_blocks(int hid, int I, int H, int KV, bool q8);
int decode_mk_blocks();
// ---- persistent decode step for Qwen3-MoE stacks (kernels_decode_moe.hip): bf16 model with bf16
// or 8-bit (groups of 64) weights, hidden 2048, 32 q / 4 kv heads of 128, E <= 128 experts, top 8,
// expert intermediate 768, every layer MoE.  layer_ptrs: n_layers rows of {in_norm, post_norm,
// q_norm, k_norm, qkv, o, router, exp_gate_up, exp_down, qkv_bias} (code arrays with 8-bit
// weights); layer_q8_ptrs (8-bit, else null): n_layers rows of scale then bias of {qkv, o, router,
// exp_gate_up, exp_down}.
bool decode_moe_supported(int n_layers, int dt, int quant_bits, int hid, int H, int KV, int D, int E, int k, int Ie,
                          int cap);
size_t decode_moe_workspace(int n_layers, int H, int KV);
hipError_t decode_moe_init(void *ws, int n_layers, int H, int KV, const void *layer_ptrs, const void *layer_q8_ptrs,
                           hipStream_t s);
hipError_t launch_decode_moe(void *ws, int n_layers, int H, int KV, int E, int norm_topk, bool q8, int cap, int p,
                             int window, float eps, const void *x, void *out, const void *final_norm, const void *cos_t,
                             const void *sin_t, void *kc, void *vc, int *err, hipStream_t s);
int decode_moe_max_blocks(bool q8);

}  // namespace q3
