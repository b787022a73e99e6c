// kernels_attn.hip -- causal GQA attention over the static KV cache.
//
// What is computed ("maya2_mlx/backbone.py", forward and docstring; the GQA
// mapping of "rlx_flow/blocks/qwen3_decoder.rs", emit/repeat_kv): the query at
// absolute position p attends keys 0..p of its kv head g = h / (H/KV) with
// scores fp32(q.k) * D^-1/2, an fp32 softmax and one rounding of the output.
//
//  - attn_decode_kernel + attn_combine_kernel (T == 1): split-K flash-decode.
//    Block (split s, kv head g) scores its chunk of keys for all G query heads
//    of the group (each K/V row is read from HBM once per step), keeps
//    un-normalised partial sums (max, sum of exp, exp-weighted V) in fp32,
//    and a combine kernel merges the splits with the usual log-sum-exp scaling.
//  - attn_prefill_mfma_kernel (T > 1, bf16): causal flash attention on MFMA.
//    Computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (q and k are bf16
//    values, so the products are exact and the sums fp32), an online fp32
//    softmax, and O^T += V^T P^T where the fp32 P is split into bf16 hi + lo
//    parts so the probability weights keep ~16 bits instead of bf16's 8.
//  - attn_rowwise_kernel (T > 1, fp32 strict mode): one wave per (query, head),
//    online softmax over key blocks of 64.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace q3 {

static inline int decode_chunk(int nkeys, int KV) {
    int c = (nkeys * KV + 511) / 512;
    c = (c + 31) / 32 * 32;
    if (c < 32) c = 32;
    if (c > 1024) c = 1024;
    return c;
}

size_t attention_workspace(int T, int H, int KV, int D, int cap) {
    (void)T;
    (void)KV;
    const size_t nsplit_max = (size_t)(cap + 31) / 32;
    return (size_t)H * nsplit_max * (D + 2) * sizeof(float);
}

// ------------------------------------------------------------ split-K decode
template <typename T, int D, int G>
__global__ void __launch_bounds__(256) attn_decode_kernel(const T *__restrict__ q, const T *__restrict__ Kc,
                                                          const T *__restrict__ Vc, int cap, int nkeys, int chunk,
                                                          float scale, float *__restrict__ part, int nsplit) {
    constexpr int VN = Vec<T>::N;
    constexpr int LPK = D / VN;    // lanes per key row
    constexpr int KPW = 64 / LPK;  // keys per wave step
    constexpr int KPB = KPW * 4;   // keys per block step
    extern __shared__ float smem[];
    float *sc = smem;                    // [G][chunk] scores, then exp(score - max)
    float *red = smem + G * chunk;       // [4][G][D] per-wave partial outputs
    __shared__ float mrow[G], lrow[G];

    const int s = blockIdx.x, g = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % LPK, kslot = lane / LPK;
    const int j0 = s * chunk;
    const int j1 = min(nkeys, j0 + chunk);
    const int nj = j1 - j0;
    const T *Kg = Kc + (size_t)g * cap * D;
    const T *Vg = Vc + (size_t)g * cap * D;

    float qf[G][VN];
#pragma unroll
    for (int i = 0; i < G; ++i) Vec<T>::expand(ld16(q + (size_t)(g * G + i) * D + sub * VN), qf[i]);

    for (int jb = j0 + wave * KPW; jb < j1; jb += KPB) {
        const int j = jb + kslot;
        const bool valid = j < j1;
        float kf[VN];
        Vec<T>::expand(valid ? ld16(Kg + (size_t)j * D + sub * VN) : u32x4{0, 0, 0, 0}, kf);
#pragma unroll
        for (int i = 0; i < G; ++i) {
            float p = 0.f;
#pragma unroll
            for (int e = 0; e < VN; ++e) p += qf[i][e] * kf[e];
#pragma unroll
            for (int o = LPK / 2; o > 0; o >>= 1) p += __shfl_xor(p, o, 64);
            if (sub == 0 && valid) sc[i * chunk + (j - j0)] = p * scale;
        }
    }
    __syncthreads();
    for (int i = wave; i < G; i += 4) {
        float m = -INFINITY;
        for (int j = lane; j < nj; j += 64) m = fmaxf(m, sc[i * chunk + j]);
        m = wave_max(m);
        float l = 0.f;
        for (int j = lane; j < nj; j += 64) {
            const float e = __expf(sc[i * chunk + j] - m);
            sc[i * chunk + j] = e;
            l += e;
        }
        l = wave_sum(l);
        if (lane == 0) {
            mrow[i] = m;
            lrow[i] = l;
        }
    }
    __syncthreads();

    float o[G][VN];
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
        for (int e = 0; e < VN; ++e) o[i][e] = 0.f;
    for (int jb = j0 + wave * KPW; jb < j1; jb += KPB) {
        const int j = jb + kslot;
        if (j < j1) {
            float vf[VN];
            Vec<T>::expand(ld16(Vg + (size_t)j * D + sub * VN), vf);
#pragma unroll
            for (int i = 0; i < G; ++i) {
                const float e = sc[i * chunk + (j - j0)];
#pragma unroll
                for (int x = 0; x < VN; ++x) o[i][x] += e * vf[x];
            }
        }
    }
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
        for (int x = 0; x < VN; ++x) {
            float v = o[i][x];
#pragma unroll
            for (int off = LPK; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
            o[i][x] = v;
        }
    if (kslot == 0) {
#pragma unroll
        for (int i = 0; i < G; ++i)
#pragma unroll
            for (int x = 0; x < VN; ++x) red[(wave * G + i) * D + sub * VN + x] = o[i][x];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += 256) {
        const int i = idx / D, d = idx % D;
        const float v = red[(0 * G + i) * D + d] + red[(1 * G + i) * D + d] + red[(2 * G + i) * D + d] +
                        red[(3 * G + i) * D + d];
        part[((size_t)(g * G + i) * nsplit + s) * (D + 2) + 2 + d] = v;
    }
    if (threadIdx.x < G) {
        float *pp = part + ((size_t)(g * G + threadIdx.x) * nsplit + s) * (D + 2);
        pp[0] = mrow[threadIdx.x];
        pp[1] = lrow[threadIdx.x];
    }
}

template <typename T>
__global__ void attn_combine_kernel(const float *__restrict__ part, int nsplit, int D, T *__restrict__ out) {
    const int h = blockIdx.x, d = threadIdx.x;
    const float *ph = part + (size_t)h * nsplit * (D + 2);
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ph[(size_t)s * (D + 2)]);
    float L = 0.f, acc = 0.f;
    for (int s = 0; s < nsplit; ++s) {
        const float *p = ph + (size_t)s * (D + 2);
        const float f = __expf(p[0] - M);
        L += p[1] * f;
        acc += p[2 + d] * f;
    }
    out[(size_t)h * D + d] = from_f<T>(acc / L);
}

// ------------------------------------------------------------ fp32 / fallback row-wise kernel
template <typename T>
__global__ void __launch_bounds__(64) attn_rowwise_kernel(const T *__restrict__ q, const T *__restrict__ Kc,
                                                          const T *__restrict__ Vc, int H, int KV, int D, int cap,
                                                          int p0, float scale, T *__restrict__ out) {
    __shared__ float qs[128];
    __shared__ float es[64];
    const int t = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
    const int g = h / (H / KV), p = p0 + t;
    const T *Kg = Kc + (size_t)g * cap * D;
    const T *Vg = Vc + (size_t)g * cap * D;
    for (int d = lane; d < D; d += 64) qs[d] = to_f(q[((size_t)t * H + h) * D + d]);
    __syncthreads();
    float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
    for (int jb = 0; jb <= p; jb += 64) {
        const int j = jb + lane;
        float sj = -INFINITY;
        if (j <= p) {
            float dotv = 0.f;
            for (int d = 0; d < D; ++d) dotv += qs[d] * to_f(Kg[(size_t)j * D + d]);
            sj = dotv * scale;
        }
        const float mn = fmaxf(m, wave_max(sj));
        const float alpha = __expf(m - mn);
        const float e = j <= p ? __expf(sj - mn) : 0.f;
        l = l * alpha + wave_sum(e);
        es[lane] = e;
        __syncthreads();
        o0 *= alpha;
        o1 *= alpha;
        const int nkb = min(64, p + 1 - jb);
        for (int jj = 0; jj < nkb; ++jj) {
            const float w = es[jj];
            o0 += w * to_f(Vg[(size_t)(jb + jj) * D + lane]);
            if (D > 64) o1 += w * to_f(Vg[(size_t)(jb + jj) * D + 64 + lane]);
        }
        __syncthreads();
        m = mn;
    }
    T *dst = out + (size_t)t * H * D + (size_t)h * D;
    if (lane < D) dst[lane] = from_f<T>(o0 / l);
    if (D > 64) dst[64 + lane] = from_f<T>(o1 / l);
}

// ------------------------------------------------------------ bf16 MFMA causal flash prefill
// Block: 64 queries (4 waves x 16) of one query head, over key tiles of 64.
template <int D>
__global__ void __launch_bounds__(256) attn_prefill_mfma_kernel(const bf16 *__restrict__ q,
                                                                const bf16 *__restrict__ Kc,
                                                                const bf16 *__restrict__ Vc, int T, int H, int KV,
                                                                int cap, int p0, float scale,
                                                                bf16 *__restrict__ out) {
    constexpr int KP = D + 8;   // K tile pitch (elements)
    constexpr int VP = 64 + 8;  // V^T tile pitch
    __shared__ __attribute__((aligned(16))) uint16_t Ks[64 * KP];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VP];
    const int ntiles = (T + 63) / 64;
    const int qt = ntiles - 1 - blockIdx.x;  // heaviest (latest) query tiles first
    const int h = blockIdx.y, g = h / (H / KV);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = qt * 64, wq0 = t0 + wave * 16;
    const int col = lane & 15, quad = lane >> 4;
    const int tq = wq0 + col;                          // this lane's query (B-operand column)
    const int qpos = p0 + min(tq, T - 1);              // padded queries behave like the last one
    const int kmax = p0 + min(t0 + 63, T - 1);         // last key any query of the block sees
    const bf16 *Kg = Kc + (size_t)g * cap * D;
    const bf16 *Vg = Vc + (size_t)g * cap * D;

    bf16x8 qf[D / 32];
    {
        const int tl = min(tq, T - 1);
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            u32x4 v = ld16(q + ((size_t)tl * H + h) * D + ks * 32 + quad * 8);
            qf[ks] = *(bf16x8 *)&v;
        }
    }
    f32x4 acc_o[D / 16];
#pragma unroll
    for (int i = 0; i < D / 16; ++i) acc_o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    const int nkt = kmax / 64 + 1;
    for (int kt = 0; kt < nkt; ++kt) {
        const int k0 = kt * 64;
        __syncthreads();
        // stage K (row-major) and V (transposed) for keys k0..k0+63; rows past kmax are zero
        for (int c = tid; c < 64 * (D / 8); c += 256) {
            const int r = c / (D / 8), d8 = (c % (D / 8)) * 8;
            const int kp = k0 + r;
            u32x4 kv = u32x4{0, 0, 0, 0}, vv = u32x4{0, 0, 0, 0};
            if (kp <= kmax) {
                kv = ld16(Kg + (size_t)kp * D + d8);
                vv = ld16(Vg + (size_t)kp * D + d8);
            }
            *(u32x4 *)&Ks[r * KP + d8] = kv;
            const uint32_t w4[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Vt[(d8 + 2 * e) * VP + r] = (uint16_t)(w4[e] & 0xffffu);
                Vt[(d8 + 2 * e + 1) * VP + r] = (uint16_t)(w4[e] >> 16);
            }
        }
        __syncthreads();
        if (k0 > p0 + min(wq0 + 15, T - 1)) continue;  // whole tile is in this wave's future

        // S^T (16 keys x 16 queries per sub-tile): row key = 4*quad + a, column query = col
        f32x4 sacc[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
                const bf16x8 kf = *(const bf16x8 *)&Ks[(kb * 16 + col) * KP + ks * 32 + quad * 8];
                sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], sacc[kb], 0, 0, 0);
            }
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int kp = k0 + kb * 16 + quad * 4 + a;
                const float sv = kp <= qpos ? sacc[kb][a] * scale : -INFINITY;
                sacc[kb][a] = sv;
                tmax = fmaxf(tmax, sv);
            }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = __expf(m_run - m_new);
        float psum = 0.f;
        bf16x8 phi[2], plo[2];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const float pv = __expf(sacc[2 * kc + half][a] - m_new);
                    psum += pv;
                    const uint32_t hb = f2bf_bits(pv);
                    const float hf = __uint_as_float(hb << 16);
                    const uint32_t lb = f2bf_bits(pv - hf);
                    uint16_t hs = (uint16_t)hb, ls = (uint16_t)lb;
                    phi[kc][half * 4 + a] = *(__bf16 *)&hs;
                    plo[kc][half * 4 + a] = *(__bf16 *)&ls;
                }
            }
        }
        psum += __shfl_xor(psum, 16, 64);
        psum += __shfl_xor(psum, 32, 64);
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
#pragma unroll
            for (int a = 0; a < 4; ++a) acc_o[dt][a] *= alpha;
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                const uint16_t *vr = &Vt[(dt * 16 + col) * VP + kc * 32 + quad * 4];
                bf16x8 vf;
                const uint2 lo4 = *(const uint2 *)vr;
                const uint2 hi4 = *(const uint2 *)(vr + 16);
                uint32_t *vw = (uint32_t *)&vf;
                vw[0] = lo4.x;
                vw[1] = lo4.y;
                vw[2] = hi4.x;
                vw[3] = hi4.y;
                acc_o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, phi[kc], acc_o[dt], 0, 0, 0);
                acc_o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, plo[kc], acc_o[dt], 0, 0, 0);
            }
        }
    }
    if (tq < T) {
        const float inv = 1.0f / l_run;
        bf16 *dst = out + (size_t)tq * H * D + (size_t)h * D;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            uint2 w;
            w.x = pack_bf2(acc_o[dt][0] * inv, acc_o[dt][1] * inv);
            w.y = pack_bf2(acc_o[dt][2] * inv, acc_o[dt][3] * inv);
            *(uint2 *)&dst[dt * 16 + quad * 4] = w;
        }
    }
}

// ------------------------------------------------------------ dispatch
template <typename T, int D>
static hipError_t decode_t(const void *q, const void *kc, const void *vc, int H, int KV, int cap, int nkeys,
                           void *out, float *ws, hipStream_t s) {
    const int G = H / KV;
    const int chunk = decode_chunk(nkeys, KV);
    const int nsplit = (nkeys + chunk - 1) / chunk;
    const float scale = (float)(1.0 / sqrt((double)D));
    const size_t lds = ((size_t)G * chunk + 4 * (size_t)G * D) * sizeof(float);
    const dim3 grid(nsplit, KV);
    const T *qq = (const T *)q, *kk = (const T *)kc, *vv = (const T *)vc;
    switch (G) {
    case 1: attn_decode_kernel<T, D, 1><<<grid, 256, lds, s>>>(qq, kk, vv, cap, nkeys, chunk, scale, ws, nsplit); break;
    case 2: attn_decode_kernel<T, D, 2><<<grid, 256, lds, s>>>(qq, kk, vv, cap, nkeys, chunk, scale, ws, nsplit); break;
    case 4: attn_decode_kernel<T, D, 4><<<grid, 256, lds, s>>>(qq, kk, vv, cap, nkeys, chunk, scale, ws, nsplit); break;
    case 8: attn_decode_kernel<T, D, 8><<<grid, 256, lds, s>>>(qq, kk, vv, cap, nkeys, chunk, scale, ws, nsplit); break;
    default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    attn_combine_kernel<T><<<H, D, 0, s>>>(ws, nsplit, D, (T *)out);
    return hipGetLastError();
}

hipError_t launch_attention(int dt, const void *q, const void *k_cache, const void *v_cache, int T, int H, int KV,
                            int D, int cap, int p0, void *out, float *ws, size_t ws_bytes, hipStream_t s) {
    (void)ws_bytes;
    const float scale = (float)(1.0 / sqrt((double)D));
    if (T == 1) {
        const int nkeys = p0 + 1;
        if (dt == DT_BF16)
            return D == 128 ? decode_t<bf16, 128>(q, k_cache, v_cache, H, KV, cap, nkeys, out, ws, s)
                            : decode_t<bf16, 64>(q, k_cache, v_cache, H, KV, cap, nkeys, out, ws, s);
        return D == 128 ? decode_t<float, 128>(q, k_cache, v_cache, H, KV, cap, nkeys, out, ws, s)
                        : decode_t<float, 64>(q, k_cache, v_cache, H, KV, cap, nkeys, out, ws, s);
    }
    if (dt == DT_BF16) {
        const dim3 grid((T + 63) / 64, H);
        const bf16 *qq = (const bf16 *)q, *kk = (const bf16 *)k_cache, *vv = (const bf16 *)v_cache;
        if (D == 128)
            attn_prefill_mfma_kernel<128><<<grid, 256, 0, s>>>(qq, kk, vv, T, H, KV, cap, p0, scale, (bf16 *)out);
        else
            attn_prefill_mfma_kernel<64><<<grid, 256, 0, s>>>(qq, kk, vv, T, H, KV, cap, p0, scale, (bf16 *)out);
        return hipGetLastError();
    }
    attn_rowwise_kernel<float><<<dim3(T, H), 64, 0, s>>>((const float *)q, (const float *)k_cache,
                                                          (const float *)v_cache, H, KV, D, cap, p0, scale,
                                                          (float *)out);
    return hipGetLastError();
}

}  // namespace q3
