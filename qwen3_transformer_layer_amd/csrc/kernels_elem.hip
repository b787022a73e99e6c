// kernels_elem.hip -- row-wise and per-head kernels: embedding gather, fused
// residual add + RMSNorm, the RoPE table, and the fused per-head q/k RMSNorm +
// RoPE + KV-cache write.
//
// Arithmetic ("maya2_mlx/backbone.py", module docstring, _rope and forward):
// RMSNorm rounds twice (after normalising and after the weight), RoPE is fp32
// maths on the table values with one rounding, the residual add rounds once.
#include "common.h"
#include "kernels.h"

namespace q3 {

// ------------------------------------------------------------ embedding gather
template <typename T>
__global__ void __launch_bounds__(256) embed_kernel(const int32_t *__restrict__ ids, const T *__restrict__ E,
                                                    int vocab, int hid, T *__restrict__ out, int *err) {
    const int t = blockIdx.x;
    int id = ids[t];
    if (id < 0 || id >= vocab) {
        if (threadIdx.x == 0 && err) atomicOr(err, 1);
        id = 0;
    }
    const T *src = E + (size_t)id * hid;
    T *dst = out + (size_t)t * hid;
    for (int i = threadIdx.x; i < hid; i += blockDim.x) dst[i] = src[i];
}

hipError_t launch_embed(int dt, const int32_t *ids, int T, const void *E, int vocab, int hid, void *out, int *err,
                        hipStream_t s) {
    if (dt == DT_BF16)
        embed_kernel<bf16><<<T, 256, 0, s>>>(ids, (const bf16 *)E, vocab, hid, (bf16 *)out, err);
    else
        embed_kernel<float><<<T, 256, 0, s>>>(ids, (const float *)E, vocab, hid, (float *)out, err);
    return hipGetLastError();
}

// ------------------------------------------------------------ add + RMSNorm
// One block per row with 16-byte vector accesses; the (added) row is kept in LDS as fp32
// between the sum-of-squares pass and the normalising pass.
template <typename T>
__global__ void __launch_bounds__(256) add_rmsnorm_kernel(const T *__restrict__ h_in, const T *__restrict__ res,
                                                          const T *__restrict__ w, T *__restrict__ h_out,
                                                          T *__restrict__ y, int n, float eps) {
    constexpr int VN = Vec<T>::N;
    extern __shared__ float hv[];
    __shared__ float red[8];
    const size_t row = blockIdx.x;
    const T *hi = h_in + row * n;
    const int nc = n / VN;
    float ss = 0.f;
    for (int c = threadIdx.x; c < nc; c += blockDim.x) {
        float v[VN];
        Vec<T>::expand(ld16(hi + (size_t)c * VN), v);
        if (res) {
            float r[VN];
            Vec<T>::expand(ld16(res + row * n + (size_t)c * VN), r);
#pragma unroll
            for (int e = 0; e < VN; ++e) v[e] = rho<T>(v[e] + r[e]);
            if (h_out) {
#pragma unroll
                for (int e = 0; e < VN; ++e) h_out[row * n + (size_t)c * VN + e] = from_f<T>(v[e]);
            }
        }
#pragma unroll
        for (int e = 0; e < VN; ++e) {
            hv[c * VN + e] = v[e];
            ss += v[e] * v[e];
        }
    }
    const float r = 1.0f / sqrtf(block_sum(ss, red) / (float)n + eps);
    for (int c = threadIdx.x; c < nc; c += blockDim.x) {
        float wv[VN];
        Vec<T>::expand(ld16(w + (size_t)c * VN), wv);
#pragma unroll
        for (int e = 0; e < VN; ++e) y[row * n + (size_t)c * VN + e] = from_f<T>(wv[e] * rho<T>(hv[c * VN + e] * r));
    }
}

hipError_t launch_add_rmsnorm(int dt, const void *h_in, const void *res, const void *w, void *h_out, void *y,
                              int T, int n, float eps, hipStream_t s) {
    const size_t lds = (size_t)n * sizeof(float);
    if (dt == DT_BF16)
        add_rmsnorm_kernel<bf16><<<T, 256, lds, s>>>((const bf16 *)h_in, (const bf16 *)res, (const bf16 *)w,
                                                     (bf16 *)h_out, (bf16 *)y, n, eps);
    else
        add_rmsnorm_kernel<float><<<T, 256, lds, s>>>((const float *)h_in, (const float *)res, (const float *)w,
                                                      (float *)h_out, (float *)y, n, eps);
    return hipGetLastError();
}

// ------------------------------------------------------------ RoPE table
// inv_j = fp32(theta^(-2j/D)) (rounded to the storage type: the bf16 model holds
// the inverse frequencies as a bf16 buffer); angle = fp32(p * inv_j);
// value = rho(fp32(cos(angle))) from double-precision cos/sin of the fp32 angle.
template <typename T>
__global__ void rope_table_kernel(int cap, int D, double theta, T *__restrict__ cos_t, T *__restrict__ sin_t) {
    const int half = D / 2;
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)cap * half) return;
    const int p = (int)(idx / half), j = (int)(idx % half);
    float inv = (float)(1.0 / pow(theta, (2.0 * j) / (double)D));
    inv = rho<T>(inv);
    const float ang = (float)p * inv;
    const T c = from_f<T>((float)cos((double)ang));
    const T sn = from_f<T>((float)sin((double)ang));
    cos_t[(size_t)p * D + j] = c;
    cos_t[(size_t)p * D + j + half] = c;
    sin_t[(size_t)p * D + j] = sn;
    sin_t[(size_t)p * D + j + half] = sn;
}

hipError_t launch_rope_table(int dt, int cap, int D, double theta, void *cos_t, void *sin_t, hipStream_t s) {
    const long n = (long)cap * (D / 2);
    const int grid = (int)((n + 255) / 256);
    if (dt == DT_BF16)
        rope_table_kernel<bf16><<<grid, 256, 0, s>>>(cap, D, theta, (bf16 *)cos_t, (bf16 *)sin_t);
    else
        rope_table_kernel<float><<<grid, 256, 0, s>>>(cap, D, theta, (float *)cos_t, (float *)sin_t);
    return hipGetLastError();
}

// ------------------------------------------------------------ q/k RMSNorm + RoPE + KV write
// One block per token, its waves looping over the heads.  Lane i owns the rotate-half
// pair (i, i + D/2), so the norm's sum of squares is one wave reduction and the rotation needs no
// exchange.  Heads 0..H-1 are query heads (written to q_out), H..H+KV-1 key
// heads (written to the cache with their value rows).
template <typename T>
__global__ void __launch_bounds__(256) qknorm_rope_kv_kernel(
    const T *__restrict__ qkv, int H, int KV, int D, const T *__restrict__ q_norm, const T *__restrict__ k_norm,
    float eps, const T *__restrict__ cos_t, const T *__restrict__ sin_t, int p0, int cap, T *__restrict__ q_out,
    T *__restrict__ kc, T *__restrict__ vc) {
    const int t = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = D / 2, nqkv = (H + 2 * KV) * D;
    const int p = p0 + t;
    const bool on = lane < half;
    float c1 = 0.f, s1 = 0.f, c2 = 0.f, s2 = 0.f;
    if (on) {
        c1 = to_f(cos_t[(size_t)p * D + lane]);
        s1 = to_f(sin_t[(size_t)p * D + lane]);
        c2 = to_f(cos_t[(size_t)p * D + lane + half]);
        s2 = to_f(sin_t[(size_t)p * D + lane + half]);
    }
    for (int hh = wave; hh < H + KV; hh += blockDim.x >> 6) {
        const T *row = qkv + (size_t)t * nqkv + (size_t)hh * D;
        float x1 = 0.f, x2 = 0.f;
        if (on) {
            x1 = to_f(row[lane]);
            x2 = to_f(row[lane + half]);
        }
        const float ss = wave_sum(x1 * x1 + x2 * x2);
        const float r = 1.0f / sqrtf(ss / (float)D + eps);
        if (!on) continue;
        const T *wn = hh < H ? q_norm : k_norm;
        const float n1 = rho<T>(to_f(wn[lane]) * rho<T>(x1 * r));
        const float n2 = rho<T>(to_f(wn[lane + half]) * rho<T>(x2 * r));
        const T o1 = from_f<T>(n1 * c1 - n2 * s1);
        const T o2 = from_f<T>(n2 * c2 + n1 * s2);
        if (hh < H) {
            T *dst = q_out + ((size_t)t * H + hh) * D;
            dst[lane] = o1;
            dst[lane + half] = o2;
        } else {
            const int g = hh - H;
            T *kd = kc + ((size_t)g * cap + p) * D;
            kd[lane] = o1;
            kd[lane + half] = o2;
            const T *vrow = qkv + (size_t)t * nqkv + (size_t)(H + KV + g) * D;
            T *vd = vc + ((size_t)g * cap + p) * D;
            vd[lane] = vrow[lane];
            vd[lane + half] = vrow[lane + half];
        }
    }
}

hipError_t launch_qknorm_rope_kv(int dt, const void *qkv, int T, int H, int KV, int D, const void *q_norm,
                                 const void *k_norm, float eps, const void *cos_t, const void *sin_t, int p0,
                                 int cap, void *q_out, void *k_cache, void *v_cache, hipStream_t s) {
    const dim3 grid(T);
    if (dt == DT_BF16)
        qknorm_rope_kv_kernel<bf16><<<grid, 256, 0, s>>>((const bf16 *)qkv, H, KV, D, (const bf16 *)q_norm,
                                                        (const bf16 *)k_norm, eps, (const bf16 *)cos_t,
                                                        (const bf16 *)sin_t, p0, cap, (bf16 *)q_out,
                                                        (bf16 *)k_cache, (bf16 *)v_cache);
    else
        qknorm_rope_kv_kernel<float><<<grid, 256, 0, s>>>((const float *)qkv, H, KV, D, (const float *)q_norm,
                                                         (const float *)k_norm, eps, (const float *)cos_t,
                                                         (const float *)sin_t, p0, cap, (float *)q_out,
                                                         (float *)k_cache, (float *)v_cache);
    return hipGetLastError();
}

}  // namespace q3
