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

// 16 bytes of type T from VN fp32 values (each rounded once).
template <typename T> __device__ __forceinline__ void store_vec(T *dst, const float *v);
template <> __device__ __forceinline__ void store_vec<bf16>(bf16 *dst, const float *v) {
    *(u32x4 *)dst = u32x4{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7])};
}
template <> __device__ __forceinline__ void store_vec<float>(float *dst, const float *v) {
    *(f32x4 *)dst = f32x4{v[0], v[1], v[2], v[3]};
}

// The same with the row held in registers (n <= 256 * VN * MAXC): each thread keeps its
// chunks c = tid + 256 i, and every store is 16 bytes.  Same arithmetic and order as above.
template <typename T, int MAXC>
__global__ void __launch_bounds__(256) add_rmsnorm_reg_kernel(const T *__restrict__ h_in, const T *__restrict__ res,
                                                              const T *__restrict__ w, T *__restrict__ h_out,
                                                              T *__restrict__ y, int n, float eps) {
    constexpr int VN = Vec<T>::N;
    __shared__ float red[8];
    const size_t row = blockIdx.x;
    const int nc = n / VN;
    float v[MAXC][VN];
    float ss = 0.f;
    u32x4 wraw[MAXC];  // the norm weights are loaded with h, not after the reduction
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
        const int c = threadIdx.x + 256 * i;
        if (c < nc) wraw[i] = ld16(w + (size_t)c * VN);
    }
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
        const int c = threadIdx.x + 256 * i;
        if (c < nc) {
            Vec<T>::expand(ld16(h_in + row * n + (size_t)c * VN), v[i]);
            if (res) {
                float r[VN];
                Vec<T>::expand(ld16(res + row * n + (size_t)c * VN), r);
#pragma unroll
                for (int e = 0; e < VN; ++e) v[i][e] = rho<T>(v[i][e] + r[e]);
                if (h_out) store_vec<T>(h_out + row * n + (size_t)c * VN, v[i]);
            }
#pragma unroll
            for (int e = 0; e < VN; ++e) ss += v[i][e] * v[i][e];
        }
    }
    const float r = 1.0f / sqrtf(block_sum(ss, red) / (float)n + eps);
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
        const int c = threadIdx.x + 256 * i;
        if (c < nc) {
            float wv[VN], o[VN];
            Vec<T>::expand(wraw[i], wv);
#pragma unroll
            for (int e = 0; e < VN; ++e) o[e] = wv[e] * rho<T>(v[i][e] * r);
            store_vec<T>(y + row * n + (size_t)c * VN, o);
        }
    }
}

hipError_t launch_add_rmsnorm(int dt, const void *h_in, const void *res, const void *w, void *h_out, void *y,
                              int T, int n, float eps, hipStream_t s) {
    const size_t lds = (size_t)n * sizeof(float);
    if (dt == DT_BF16 && n <= 256 * 8 * 4) {
        add_rmsnorm_reg_kernel<bf16, 4><<<T, 256, 0, s>>>((const bf16 *)h_in, (const bf16 *)res, (const bf16 *)w,
                                                         (bf16 *)h_out, (bf16 *)y, n, eps);
        return hipGetLastError();
    }
    if (dt == DT_FP32 && n <= 256 * 4 * 4) {
        add_rmsnorm_reg_kernel<float, 4><<<T, 256, 0, s>>>((const float *)h_in, (const float *)res,
                                                          (const float *)w, (float *)h_out, (float *)y, n, eps);
        return hipGetLastError();
    }
    if (dt == DT_BF16)
        add_rmsnorm_kernel<bf16><<<T, 256, lds, s>>>((const bf16 *)h_in, (const bf16 *)res, (const bf16 *)w,
                                                     (bf16 *)h_out, (bf16 *)y, n, eps);
    else
        add_rmsnorm_kernel<float><<<T, 256, lds, s>>>((const float *)h_in, (const float *)res, (const float *)w,
                                                      (float *)h_out, (float *)y, n, eps);
    return hipGetLastError();
}

// ------------------------------------------------------------ streaming read probe
// The measured-peak figure beside the published 8 TB/s: a plain read of n16 16-byte words with
// non-temporal 16-byte loads, eight in flight per thread per round, consecutive lanes on
// consecutive words, one block of 4 waves per CU.  Each thread XORs what it read and writes one
// word (so the loads are not dead); out holds SR_BLOCKS * 256 words.  Over a 4 GiB buffer
// (one box, graph replays): 256 blocks x 8 loads 7.18 TB/s; 512 x 4 7.05; 1024 x 4 5.73;
// 8192 x 4 6.45; plain (cached) loads 5.6.
constexpr int SR_BLOCKS = 256, SR_U = 8;
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4 *__restrict__ src, size_t n16,
                                                          uint32_t *__restrict__ out) {
    const size_t stride = (size_t)SR_BLOCKS * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (SR_U - 1) * stride < n16; i += SR_U * stride) {
        u32x4 v[SR_U];
#pragma unroll
        for (int k = 0; k < SR_U; ++k) v[k] = __builtin_nontemporal_load(src + i + k * stride);
#pragma unroll
        for (int k = 0; k < SR_U; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
    }
    for (; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(src + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

hipError_t launch_stream_read(const void *src, size_t bytes, void *out, hipStream_t s) {
    stream_read_kernel<<<SR_BLOCKS, 256, 0, s>>>((const u32x4 *)src, bytes / 16, (uint32_t *)out);
    return hipGetLastError();
}

// ------------------------------------------------------------ RoPE table
// inv_j = fp32(theta^(-2j/D)) (rounded to the storage type: the bf16 model holds
// the inverse frequencies as a bf16 buffer); angle = fp32(p * inv_j);
// value = rho(fp32(cos(angle))) from double-precision cos/sin of the fp32 angle.
// The fp32 value is what gets rounded to the table type: without the empty asm the compiler
// fuses "double -> fp32 -> bf16" into one rounding straight from double, which differs from
// the two roundings on a few entries.
__device__ __forceinline__ float pin_f32(float f) {
    __asm__ volatile("" : "+v"(f));
    return f;
}

template <typename T>
__global__ void rope_table_kernel(int cap, int D, double theta, T *__restrict__ cos_t, T *__restrict__ sin_t) {
    const int half = D / 2;
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)cap * half) return;
    const int p = (int)(idx / half), j = (int)(idx % half);
    float inv = pin_f32((float)(1.0 / pow(theta, (2.0 * j) / (double)D)));
    inv = rho<T>(inv);
    const float ang = (float)p * inv;
    const T c = from_f<T>(pin_f32((float)cos((double)ang)));
    const T sn = from_f<T>(pin_f32((float)sin((double)ang)));
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
// Page 2's switches ("rlx_flow/blocks/qwen3_decoder.rs", Qwen3DecoderSpec): with a bias
// [(H+2KV)D] every q, k and v element first becomes rho(x + b) (the add after the
// projection, rounded); with q_norm == k_norm == NULL (Qwen2) RoPE takes the projection
// (plus bias) as it is.
// One block per token, its waves looping over the heads.  Lane i owns the rotate-half
// pair (i, i + D/2), so the norm's sum of squares is one wave reduction and the rotation needs no
// exchange.  Heads 0..H-1 are query heads (written to q_out), H..H+KV-1 key
// heads (written to the cache with their value rows).
template <typename T>
__global__ void __launch_bounds__(256) qknorm_rope_kv_kernel(
    const T *__restrict__ qkv, int H, int KV, int D, const T *__restrict__ q_norm, const T *__restrict__ k_norm,
    const T *__restrict__ bias, float eps, const T *__restrict__ cos_t, const T *__restrict__ sin_t, int p0, int cap,
    T *__restrict__ q_out, T *__restrict__ kc, T *__restrict__ vc) {
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
            if (bias) {
                x1 = rho<T>(x1 + to_f(bias[(size_t)hh * D + lane]));
                x2 = rho<T>(x2 + to_f(bias[(size_t)hh * D + lane + half]));
            }
        }
        const float ss = wave_sum(x1 * x1 + x2 * x2);
        const float r = 1.0f / sqrtf(ss / (float)D + eps);
        if (!on) continue;
        const T *wn = hh < H ? q_norm : k_norm;
        const float n1 = wn ? rho<T>(to_f(wn[lane]) * rho<T>(x1 * r)) : x1;
        const float n2 = wn ? rho<T>(to_f(wn[lane + half]) * rho<T>(x2 * r)) : x2;
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
            if (bias) {
                const T *vb = bias + (size_t)(H + KV + g) * D;
                vd[lane] = from_f<T>(to_f(vrow[lane]) + to_f(vb[lane]));
                vd[lane + half] = from_f<T>(to_f(vrow[lane + half]) + to_f(vb[lane + half]));
            } else {
                vd[lane] = vrow[lane];
                vd[lane + half] = vrow[lane + half];
            }
        }
    }
}

// The same with D/8 lanes per head: lane li of a head owns elements 4 li .. 4 li + 3 and their
// rotate-half partners 4 li + D/2 .., so every access is 8 bytes (bf16), a wave holds 512 / D
// heads, and the norm's sum of squares is a butterfly over the head's lanes.  The table row
// and the norm weights are read once per token.
template <int D>
__global__ void __launch_bounds__(256) qknorm_rope_kv_vec_kernel(
    const bf16 *__restrict__ qkv, int H, int KV, const bf16 *__restrict__ q_norm, const bf16 *__restrict__ k_norm,
    const bf16 *__restrict__ bias, float eps, const bf16 *__restrict__ cos_t, const bf16 *__restrict__ sin_t, int p0,
    int cap, bf16 *__restrict__ q_out, bf16 *__restrict__ kc, bf16 *__restrict__ vc) {
    constexpr int LPH = D / 8, HPW = 64 / LPH, half = D / 2;  // lanes per head, heads per wave
    const int t = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane % LPH, sub = lane / LPH, e1 = 4 * li, e2 = e1 + half;
    const int nqkv = (H + 2 * KV) * D, p = p0 + t;
    float c1[4], s1[4], c2[4], s2[4], wq1[4], wq2[4], wk1[4], wk2[4];
    auto ld4 = [](const bf16 *src, float *o) {
        const uint2 u = *(const uint2 *)src;
        o[0] = bf_lo(u.x); o[1] = bf_hi(u.x); o[2] = bf_lo(u.y); o[3] = bf_hi(u.y);
    };
    ld4(cos_t + (size_t)p * D + e1, c1);
    ld4(sin_t + (size_t)p * D + e1, s1);
    ld4(cos_t + (size_t)p * D + e2, c2);
    ld4(sin_t + (size_t)p * D + e2, s2);
    const bool nrm = q_norm != nullptr;
    if (nrm) {
        ld4(q_norm + e1, wq1);
        ld4(q_norm + e2, wq2);
        ld4(k_norm + e1, wk1);
        ld4(k_norm + e2, wk2);
    }
    const int nh = H + KV;
    for (int hb = wave * HPW; hb < nh; hb += HPW * (blockDim.x >> 6)) {
        const int hh = hb + sub;
        const bool on = hh < nh;
        float x1[4] = {0.f, 0.f, 0.f, 0.f}, x2[4] = {0.f, 0.f, 0.f, 0.f};
        if (on) {
            ld4(qkv + (size_t)t * nqkv + (size_t)hh * D + e1, x1);
            ld4(qkv + (size_t)t * nqkv + (size_t)hh * D + e2, x2);
            if (bias) {
                float b1[4], b2[4];
                ld4(bias + (size_t)hh * D + e1, b1);
                ld4(bias + (size_t)hh * D + e2, b2);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x1[e] = rho<bf16>(x1[e] + b1[e]);
                    x2[e] = rho<bf16>(x2[e] + b2[e]);
                }
            }
        }
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) ss += x1[e] * x1[e] + x2[e] * x2[e];
#pragma unroll
        for (int o = 1; o < LPH; o <<= 1) ss += __shfl_xor(ss, o, 64);
        const float r = 1.0f / sqrtf(ss / (float)D + eps);
        if (!on) continue;
        const bool isq = hh < H;
        float o1[4], o2[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float n1 = nrm ? rho<bf16>((isq ? wq1[e] : wk1[e]) * rho<bf16>(x1[e] * r)) : x1[e];
            const float n2 = nrm ? rho<bf16>((isq ? wq2[e] : wk2[e]) * rho<bf16>(x2[e] * r)) : x2[e];
            o1[e] = n1 * c1[e] - n2 * s1[e];
            o2[e] = n2 * c2[e] + n1 * s2[e];
        }
        const uint2 w1 = {pack_bf2(o1[0], o1[1]), pack_bf2(o1[2], o1[3])};
        const uint2 w2 = {pack_bf2(o2[0], o2[1]), pack_bf2(o2[2], o2[3])};
        if (isq) {
            bf16 *dst = q_out + ((size_t)t * H + hh) * D;
            *(uint2 *)(dst + e1) = w1;
            *(uint2 *)(dst + e2) = w2;
        } else {
            const int g = hh - H;
            bf16 *kd = kc + ((size_t)g * cap + p) * D;
            *(uint2 *)(kd + e1) = w1;
            *(uint2 *)(kd + e2) = w2;
            const bf16 *vrow = qkv + (size_t)t * nqkv + (size_t)(H + KV + g) * D;
            bf16 *vd = vc + ((size_t)g * cap + p) * D;
            if (bias) {
                float v1[4], v2[4], b1[4], b2[4];
                ld4(vrow + e1, v1);
                ld4(vrow + e2, v2);
                ld4(bias + (size_t)(H + KV + g) * D + e1, b1);
                ld4(bias + (size_t)(H + KV + g) * D + e2, b2);
                *(uint2 *)(vd + e1) = uint2{pack_bf2(v1[0] + b1[0], v1[1] + b1[1]), pack_bf2(v1[2] + b1[2], v1[3] + b1[3])};
                *(uint2 *)(vd + e2) = uint2{pack_bf2(v2[0] + b2[0], v2[1] + b2[1]), pack_bf2(v2[2] + b2[2], v2[3] + b2[3])};
            } else {
                *(uint2 *)(vd + e1) = *(const uint2 *)(vrow + e1);
                *(uint2 *)(vd + e2) = *(const uint2 *)(vrow + e2);
            }
        }
    }
}

hipError_t launch_qknorm_rope_kv(int dt, const void *qkv, int T, int H, int KV, int D, const void *q_norm,
                                 const void *k_norm, const void *bias, float eps, const void *cos_t,
                                 const void *sin_t, int p0, int cap, void *q_out, void *k_cache, void *v_cache,
                                 hipStream_t s) {
    if ((q_norm == nullptr) != (k_norm == nullptr)) return hipErrorInvalidValue;
    const dim3 grid(T);
    if (dt == DT_BF16 && (D == 128 || D == 64)) {
        const bf16 *a = (const bf16 *)qkv, *qn = (const bf16 *)q_norm, *kn = (const bf16 *)k_norm;
        const bf16 *b = (const bf16 *)bias, *ct = (const bf16 *)cos_t, *st = (const bf16 *)sin_t;
        if (D == 128)
            qknorm_rope_kv_vec_kernel<128><<<grid, 256, 0, s>>>(a, H, KV, qn, kn, b, eps, ct, st, p0, cap,
                                                                 (bf16 *)q_out, (bf16 *)k_cache, (bf16 *)v_cache);
        else
            qknorm_rope_kv_vec_kernel<64><<<grid, 256, 0, s>>>(a, H, KV, qn, kn, b, eps, ct, st, p0, cap,
                                                                (bf16 *)q_out, (bf16 *)k_cache, (bf16 *)v_cache);
        return hipGetLastError();
    }
    if (dt == DT_BF16)
        qknorm_rope_kv_kernel<bf16><<<grid, 256, 0, s>>>((const bf16 *)qkv, H, KV, D, (const bf16 *)q_norm,
                                                        (const bf16 *)k_norm, (const bf16 *)bias, eps,
                                                        (const bf16 *)cos_t, (const bf16 *)sin_t, p0, cap,
                                                        (bf16 *)q_out, (bf16 *)k_cache, (bf16 *)v_cache);
    else
        qknorm_rope_kv_kernel<float><<<grid, 256, 0, s>>>((const float *)qkv, H, KV, D, (const float *)q_norm,
                                                         (const float *)k_norm, (const float *)bias, eps,
                                                         (const float *)cos_t, (const float *)sin_t, p0, cap,
                                                         (float *)q_out, (float *)k_cache, (float *)v_cache);
    return hipGetLastError();
}

}  // namespace q3
