// kernels_moe.hip -- the Qwen3-MoE block on the GPU.
//
// What is computed ("@mlx-bun/inference" qwen3-moe.ts, Qwen3MoeSparseMoeBlock.forward
// and the two expert orders Qwen3UnsortedExperts / Qwen3SortedExperts): router
// logits x . Wr^T, softmax over all experts in fp32 rounded to the model dtype,
// the top-k experts (ties to the lower index; slot order descending probability),
// renormalised weights, per-expert SwiGLU FFN (gate|up rows, silu in fp32 rounded
// once, times up rounded once, down projection), and the weighted sum over slots.
//
// Layout of the work:
//  1. router logits: the shared projection kernels (GEMV / MFMA GEMM);
//  2. moe_topk_kernel: one wave per token does softmax, k arg-max rounds and the
//     renormalisation;
//  3. moe_sort_kernel: stable counting sort of the T*k (token, slot) rows by
//     expert (one thread per expert scans the rows in order), giving per-expert
//     row ranges, the sorted-to-row permutation, its inverse and the list of
//     experts that received rows;
//  4. moe_expert_kernel: grid (output column block, active expert); each wave
//     streams one weight row (a gate/up pair in the first pass) of its expert
//     once per group of 8 routed rows, so every hit expert's weights are read
//     from HBM once for up to 8 tokens;
//  5. moe_combine_kernel: out[t] = rho(sum_s rho(y[t,s] * w[t,s])), slot order.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace q3 {

namespace {
inline size_t al(size_t b) { return (b + 255) & ~(size_t)255; }
struct MoeWs {
    size_t logits, offsets, perm, inv, active, m, y, total;
};
MoeWs moe_layout(int T, int hid, int E, int k, int Ie, int dt) {
    const size_t es = dt == DT_BF16 ? 2 : 4, rows = (size_t)T * k;
    MoeWs w{};
    size_t o = 0;
    w.logits = o; o += al((size_t)T * E * es);
    w.offsets = o; o += al((size_t)(E + 1) * 4);
    w.perm = o; o += al(rows * 4);
    w.inv = o; o += al(rows * 4);
    w.active = o; o += al((size_t)(E + 1) * 4);
    w.m = o; o += al(rows * Ie * es);
    w.y = o; o += al(rows * hid * es);
    w.total = o;
    return w;
}
}  // namespace

size_t moe_workspace(int T, int hid, int E, int k, int Ie, int dt) { return moe_layout(T, hid, E, k, Ie, dt).total; }

// ------------------------------------------------------------ softmax + top-k + renormalise
template <typename T>
__global__ void __launch_bounds__(64) moe_topk_kernel(const T *__restrict__ logits, int E, int k, int norm,
                                                      int32_t *__restrict__ idx, T *__restrict__ wout) {
    constexpr int EPL = 4;  // experts per lane (E <= 256)
    const int t = blockIdx.x, lane = threadIdx.x;
    const T *l = logits + (size_t)t * E;
    float v[EPL];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E ? to_f(l[e]) : -INFINITY;
        m = fmaxf(m, v[i]);
    }
    m = wave_max(m);
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E ? __expf(v[i] - m) : 0.f;
        z += v[i];
    }
    z = wave_sum(z);
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E ? rho<T>(v[i] / z) : -INFINITY;  // probabilities in the model dtype
    }
    // k rounds of (largest value, lowest index) selection among the experts not taken yet.
    // Only experts e < E are candidates and a NaN probability ranks as -inf, so every round
    // picks a valid expert (k <= E) whatever the logits hold.
    float psel[16];
    int isel[16];
    unsigned taken = 0;  // bit i: expert lane + 64 i is selected or does not exist
#pragma unroll
    for (int i = 0; i < EPL; ++i)
        if (lane + 64 * i >= E) taken |= 1u << i;
    for (int s = 0; s < k; ++s) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            const float x = v[i] == v[i] ? v[i] : -INFINITY;
            if (!((taken >> i) & 1u) && (x > bv || (x == bv && e < bi))) {
                bv = x;
                bi = e;
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float ov = __shfl_xor(bv, o, 64);
            const int oi = __shfl_xor(bi, o, 64);
            if (ov > bv || (ov == bv && oi < bi)) {
                bv = ov;
                bi = oi;
            }
        }
        psel[s] = bv;
        isel[s] = bi;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (lane + 64 * i == bi) taken |= 1u << i;
    }
    if (lane == 0) {
        float den = 0.f;
        for (int s = 0; s < k; ++s) den += psel[s];
        const float denr = rho<T>(den);
        for (int s = 0; s < k; ++s) {
            idx[(size_t)t * k + s] = isel[s];
            wout[(size_t)t * k + s] = from_f<T>(norm ? psel[s] / denr : psel[s]);
        }
    }
}

// ------------------------------------------------------------ stable counting sort by expert
__global__ void __launch_bounds__(256) moe_sort_kernel(const int32_t *__restrict__ idx, int rows, int E,
                                                       int32_t *__restrict__ offsets, int32_t *__restrict__ perm,
                                                       int32_t *__restrict__ inv, int32_t *__restrict__ active) {
    __shared__ int cnt[257];
    __shared__ int start[257];
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int c = 0;
        for (int r = 0; r < rows; ++r) c += idx[r] == e;
        cnt[e] = c;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int acc = 0, na = 0;
        for (int e = 0; e < E; ++e) {
            start[e] = acc;
            offsets[e] = acc;
            acc += cnt[e];
            if (cnt[e] > 0) active[1 + na++] = e;
        }
        offsets[E] = acc;
        active[0] = na;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int pos = start[e];
        for (int r = 0; r < rows; ++r)
            if (idx[r] == e) {
                perm[pos] = r;
                inv[r] = pos;
                ++pos;
            }
    }
}

// ------------------------------------------------------------ grouped expert projections
// PASS 0: m[i] = swiglu(x[row(i)] . Wgu_e^T)  (Wgu_e [2*Ie][hid], output Ie columns)
// PASS 1: y[i] = rho(m[i] . Wd_e^T)           (Wd_e [hid][Ie], output hid columns)
// i runs over the sorted rows of expert e; row(i) = perm[i] / k for PASS 0.
template <typename T, int PASS>
__global__ void __launch_bounds__(256) moe_expert_kernel(const T *__restrict__ xin, const T *__restrict__ W,
                                                         int K, int N, int k, const int32_t *__restrict__ offsets,
                                                         const int32_t *__restrict__ perm,
                                                         const int32_t *__restrict__ active, T *__restrict__ out) {
    constexpr int VN = Vec<T>::N;
    constexpr int MR = 8;
    const int slot = blockIdx.y;
    if (slot >= active[0]) return;
    const int e = active[1 + slot];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = blockIdx.x * 4 + wave;
    if (n >= N) return;
    const int r0 = offsets[e], r1 = offsets[e + 1];
    const size_t wrows = PASS == 0 ? 2 * (size_t)N : (size_t)N;
    const T *We = W + (size_t)e * wrows * K;
    const T *w0 = We + (size_t)n * K;
    const T *w1 = We + (size_t)(PASS == 0 ? n + N : n) * K;
    const int nc = K / VN;
    for (int rb = r0; rb < r1; rb += MR) {
        const int nr = min(MR, r1 - rb);
        const T *xr[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const int i = rb + min(m, nr - 1);
            xr[m] = PASS == 0 ? xin + (size_t)(perm[i] / k) * K : xin + (size_t)i * K;
        }
        float a0[MR], a1[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) a0[m] = a1[m] = 0.f;
        for (int c = lane; c < nc; c += 64) {
            float wf0[VN], wf1[VN];
            Vec<T>::expand(ld_stream(w0 + (size_t)c * VN), wf0);
            if (PASS == 0) Vec<T>::expand(ld_stream(w1 + (size_t)c * VN), wf1);
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                if (m < nr) {
                    float xf[VN];
                    Vec<T>::expand(ld16(xr[m] + (size_t)c * VN), xf);
#pragma unroll
                    for (int x = 0; x < VN; ++x) {
                        a0[m] += wf0[x] * xf[x];
                        if (PASS == 0) a1[m] += wf1[x] * xf[x];
                    }
                }
            }
        }
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            if (m < nr) {
                const float s0 = wave_sum(a0[m]);
                const float s1 = PASS == 0 ? wave_sum(a1[m]) : 0.f;
                if (lane == 0) {
                    float v;
                    if (PASS == 0) v = rho<T>(silu_f32(rho<T>(s0))) * rho<T>(s1);
                    else v = s0;
                    out[(size_t)(rb + m) * N + n] = from_f<T>(v);
                }
            }
        }
    }
}

// ------------------------------------------------------------ weighted slot sum
template <typename T>
__global__ void __launch_bounds__(256) moe_combine_kernel(const T *__restrict__ y, const T *__restrict__ w,
                                                          const int32_t *__restrict__ inv, int hid, int k,
                                                          T *__restrict__ out) {
    const int t = blockIdx.x;
    for (int n = threadIdx.x; n < hid; n += blockDim.x) {
        float acc = 0.f;
        for (int s = 0; s < k; ++s) {
            const int r = t * k + s, p = inv[r];
            if ((unsigned)p >= (unsigned)(gridDim.x * k)) continue;  // never for indices the top-k kernel writes
            acc += rho<T>(to_f(y[(size_t)p * hid + n]) * to_f(w[r]));
        }
        out[(size_t)t * hid + n] = from_f<T>(acc);
    }
}

// ------------------------------------------------------------ dispatch
template <typename T>
static hipError_t moe_t(const void *x, int T_, int hid, const void *Wr, int E, int k, int norm, int Ie,
                        const void *Wgu, const void *Wd, int32_t *idx, void *w, void *out, void *ws, hipStream_t s) {
    const int dt = DtOf<T>::value;
    const MoeWs L = moe_layout(T_, hid, E, k, Ie, dt);
    char *base = (char *)ws;
    T *logits = (T *)(base + L.logits);
    int32_t *offsets = (int32_t *)(base + L.offsets), *perm = (int32_t *)(base + L.perm);
    int32_t *inv = (int32_t *)(base + L.inv), *active = (int32_t *)(base + L.active);
    T *mbuf = (T *)(base + L.m), *ybuf = (T *)(base + L.y);
    const int rows = T_ * k;
    hipError_t e = launch_linear(dt, x, T_, hid, Wr, E, EPI_STORE, nullptr, logits, s);
    if (e != hipSuccess) return e;
    moe_topk_kernel<T><<<T_, 64, 0, s>>>(logits, E, k, norm, idx, (T *)w);
    moe_sort_kernel<<<1, 256, 0, s>>>(idx, rows, E, offsets, perm, inv, active);
    const int na_max = rows < E ? rows : E;
    moe_expert_kernel<T, 0><<<dim3((Ie + 3) / 4, na_max), 256, 0, s>>>((const T *)x, (const T *)Wgu, hid, Ie, k,
                                                                       offsets, perm, active, mbuf);
    moe_expert_kernel<T, 1><<<dim3((hid + 3) / 4, na_max), 256, 0, s>>>(mbuf, (const T *)Wd, Ie, hid, k, offsets,
                                                                        perm, active, ybuf);
    moe_combine_kernel<T><<<T_, 256, 0, s>>>(ybuf, (const T *)w, inv, hid, k, (T *)out);
    return hipGetLastError();
}

hipError_t launch_moe(int dt, const void *x, int T, int hid, const void *Wr, int E, int k, int norm, int Ie,
                      const void *Wgu, const void *Wd, int32_t *idx, void *w, void *out, void *ws, hipStream_t s) {
    if (dt == DT_BF16) return moe_t<bf16>(x, T, hid, Wr, E, k, norm, Ie, Wgu, Wd, idx, w, out, ws, s);
    return moe_t<float>(x, T, hid, Wr, E, k, norm, Ie, Wgu, Wd, idx, w, out, ws, s);
}

}  // namespace q3
