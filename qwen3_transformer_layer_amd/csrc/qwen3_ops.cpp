// qwen3_ops.cpp -- single-kernel entry points (include/qwen3_ops.h) for
// per-kernel parity tests.  Arguments are checked on the host before launch.
#include "../../include/qwen3.h"
#include "../../include/qwen3_ops.h"
#include "kernels.h"

using namespace q3;

namespace {
bool dt_ok(int dt) { return dt == QWEN3_BF16 || dt == QWEN3_FP32; }
int hip_rc(hipError_t e) { return e == hipSuccess ? QWEN3_OK : QWEN3_ERR_HIP; }
}  // namespace

extern "C" {

int qwen3_op_add_rmsnorm(int dtype, const void *h_in, const void *res, const void *w, void *h_out, void *y, int T,
                         int n, float eps, void *stream) {
    if (!dt_ok(dtype)) return QWEN3_ERR_DTYPE;
    if (!h_in || !w || !y || T < 1 || n < 8 || n % 8 || n > 16384) return QWEN3_ERR_ARG;
    return hip_rc(launch_add_rmsnorm(dtype, h_in, res, w, h_out, y, T, n, eps, (hipStream_t)stream));
}

int qwen3_op_stream_read(const void *src, size_t bytes, uint32_t *out, void *stream) {
    if (!src || !out || bytes < 16 || bytes % 16 || ((uintptr_t)src & 15) || ((uintptr_t)out & 3)) return QWEN3_ERR_ARG;
    return hip_rc(launch_stream_read(src, bytes, out, (hipStream_t)stream));
}

int qwen3_op_linear(int dtype, const void *x, int M, int K, const void *W, int N, int epilogue, const void *res,
                    void *out, void *stream) {
    if (!dt_ok(dtype)) return QWEN3_ERR_DTYPE;
    if (!x || !W || !out || M < 1 || K < 64 || K % 64 || N < 1 || epilogue < 0 || epilogue > 2) return QWEN3_ERR_ARG;
    if (epilogue == EPI_RESID && !res) return QWEN3_ERR_ARG;
    return hip_rc(launch_linear(dtype, x, M, K, W, N, epilogue, res, out, (hipStream_t)stream));
}

int qwen3_op_linear_q8(const void *x, int M, int K, const uint8_t *codes, const void *scale, const void *bias,
                       int N, int epilogue, const void *res, void *out, void *stream) {
    if (!x || !codes || !scale || !bias || !out || M < 1 || K < 64 || K % 64 || N < 1 || epilogue < 0 || epilogue > 2)
        return QWEN3_ERR_ARG;
    if (epilogue == EPI_RESID && !res) return QWEN3_ERR_ARG;
    if (M <= 16 && K > 8192) return QWEN3_ERR_UNSUPPORTED;  // the GEMV keeps a whole row in flight
    return hip_rc(launch_linear_q8(x, M, K, codes, scale, bias, 64, N, epilogue, res, out, (hipStream_t)stream));
}

int qwen3_op_qknorm_rope_kv(int dtype, const void *qkv, int T, int H, int KV, int D, const void *q_norm,
                            const void *k_norm, float eps, const void *cos_t, const void *sin_t, int p0, int cap,
                            void *q_out, void *k_cache, void *v_cache, void *stream) {
    if (!dt_ok(dtype)) return QWEN3_ERR_DTYPE;
    if (!qkv || !q_norm || !k_norm || !cos_t || !sin_t || !q_out || !k_cache || !v_cache) return QWEN3_ERR_ARG;
    if (T < 1 || H < 1 || KV < 1 || H % KV || (D != 64 && D != 128) || p0 < 0 || p0 + T > cap) return QWEN3_ERR_ARG;
    return hip_rc(launch_qknorm_rope_kv(dtype, qkv, T, H, KV, D, q_norm, k_norm, nullptr, eps, cos_t, sin_t, p0, cap, q_out,
                                        k_cache, v_cache, (hipStream_t)stream));
}

size_t qwen3_op_attention_workspace(int T, int H, int KV, int D, int cap) {
    return attention_workspace(T, H, KV, D, cap);
}

int qwen3_op_attention(int dtype, const void *q, const void *k_cache, const void *v_cache, int T, int H, int KV, int D,
                       int cap, int p0, void *out, void *ws, size_t ws_bytes, void *stream) {
    if (!dt_ok(dtype)) return QWEN3_ERR_DTYPE;
    if (!q || !k_cache || !v_cache || !out || T < 1 || H < 1 || KV < 1 || H % KV || p0 < 0 || p0 + T > cap)
        return QWEN3_ERR_ARG;
    const int G = H / KV;
    if ((D != 64 && D != 128) || (G != 1 && G != 2 && G != 4 && G != 8)) return QWEN3_ERR_UNSUPPORTED;
    if (T == 1 && (!ws || ws_bytes < attention_workspace(T, H, KV, D, cap))) return QWEN3_ERR_WORKSPACE;
    return hip_rc(launch_attention(dtype, q, k_cache, v_cache, T, H, KV, D, cap, p0, 0, out, (float *)ws, ws_bytes,
                                   (hipStream_t)stream));
}

size_t qwen3_op_moe_workspace(int dtype, int T, int hid, int E, int k, int Ie) {
    return moe_workspace(T, hid, E, k, Ie, dtype);
}

int qwen3_op_moe(int dtype, const void *x, int T, int hid, const void *router, int E, int k, int norm, int Ie,
                 const void *exp_gate_up, const void *exp_down, int32_t *idx, void *w, void *out, void *ws,
                 size_t ws_bytes, void *stream) {
    if (!dt_ok(dtype)) return QWEN3_ERR_DTYPE;
    if (!x || !router || !exp_gate_up || !exp_down || !idx || !w || !out || !ws) return QWEN3_ERR_ARG;
    if (T < 1 || hid < 64 || hid % 64 || E < 1 || E > 256 || k < 1 || k > 16 || k > E || Ie < 64 || Ie % 64)
        return QWEN3_ERR_ARG;
    if (ws_bytes < moe_workspace(T, hid, E, k, Ie, dtype)) return QWEN3_ERR_WORKSPACE;
    const MoeWeights W{router, nullptr, nullptr, exp_gate_up, nullptr, nullptr, exp_down, nullptr, nullptr, false};
    return hip_rc(launch_moe(dtype, x, T, hid, W, E, k, norm, Ie, idx, w, out, ws, (hipStream_t)stream));
}

}  // extern "C"
