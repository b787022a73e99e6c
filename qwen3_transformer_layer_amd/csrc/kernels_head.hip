// kernels_head.hip -- output head and greedy token ("maya2_mlx/backbone.py", Backbone.cb0_logits:
// the head projection in the model dtype, then fp32; "@mlx-bun/inference" qwen3.ts, lmHead or the
// tied embedding used as a linear): logits[t][v] = fp32(rho(hs[t] . W[v])) and argmax[t] = the
// lowest v whose logit is the largest.
//
// One HBM-bound pass over W [V][K] in the GEMV layout of kernels_linear.hip: at most 2048 blocks,
// each wave64 walking rows v = wave id, + grid waves, ..., streaming each with 128-bit
// non-temporal loads (four in flight per lane) for up to 16 rows of hs at once.  The rounded
// logit is written when asked and becomes an order-preserving 64-bit key: the value's bits mapped
// so unsigned order is numeric order (-0 as +0, a NaN below every number), then the complement of
// v, so the largest key is the largest logit at the lowest index.  A wave keeps its best key per
// row in a register; the block's four are reduced in LDS and one 64-bit atomicMax per (block,
// row) goes to one of HS slots of the row (block % HS), so no address takes more than about 32
// atomics; head_final_kernel reduces the slots and turns the key into an index.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace q3 {

__device__ __forceinline__ unsigned long long head_key(float f, int v) {
    uint32_t u = __float_as_uint(f);
    if (f != f) u = 0u;                            // NaN: below every number
    else if (f == 0.f) u = 0x80000000u;            // -0 ranks as +0
    else u = (u >> 31) ? ~u : (u | 0x80000000u);   // negative: reversed; positive: above all negatives
    return ((unsigned long long)u << 32) | (unsigned long long)(0xffffffffu - (uint32_t)v);
}

constexpr int HS = 64;           // key slots per row
constexpr int HEAD_BLOCKS = 2048;  // grid cap

__global__ void head_init_kernel(unsigned long long *__restrict__ keys, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) keys[i] = 0ull;
}

// one wave per row: the maximum of the row's HS slots
__global__ void head_final_kernel(const unsigned long long *__restrict__ keys, int T, int32_t *__restrict__ argmax) {
    const int t = blockIdx.x, lane = threadIdx.x;
    unsigned long long k = keys[(size_t)t * HS + lane];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const unsigned long long q = __shfl_xor(k, o, 64);
        k = q > k ? q : k;
    }
    if (lane == 0) argmax[t] = (int32_t)(0xffffffffu - (uint32_t)(k & 0xffffffffull));
}

template <typename T, int MR>
__global__ void __launch_bounds__(256) head_kernel(const T *__restrict__ x, int M, int K, const T *__restrict__ W,
                                                   int V, float *__restrict__ logits,
                                                   unsigned long long *__restrict__ keys) {
    constexpr int VN = Vec<T>::N;
    constexpr int U = 4;
    __shared__ unsigned long long kb[4][MR];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nc = K / VN;  // 16-byte chunks per row
    unsigned long long best[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) best[m] = 0ull;
    for (int n = blockIdx.x * 4 + wave; n < V; n += gridDim.x * 4) {
        const T *w0 = W + (size_t)n * K;
        float a[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) a[m] = 0.f;
        for (int c0 = lane; c0 < nc; c0 += 64 * U) {
            u32x4 wv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + 64 * u;
                wv[u] = c < nc ? ld_stream(w0 + (size_t)c * VN) : u32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + 64 * u;
                if (c < nc) {
#pragma unroll
                    for (int m = 0; m < MR; ++m)
                        if (m < M) a[m] = dot16<T>(wv[u], ld16(x + (size_t)m * K + (size_t)c * VN), a[m]);
                }
            }
        }
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            if (m < M) {
                const float r = rho<T>(wave_sum(a[m]));
                if (lane == 0) {
                    if (logits) logits[(size_t)m * V + n] = r;
                    const unsigned long long key = head_key(r, n);
                    best[m] = key > best[m] ? key : best[m];
                }
            }
        }
    }
    if (lane == 0)
#pragma unroll
        for (int m = 0; m < MR; ++m) kb[wave][m] = best[m];
    __syncthreads();
    if (keys && threadIdx.x < MR && (int)threadIdx.x < M) {
        unsigned long long b = kb[0][threadIdx.x];
#pragma unroll
        for (int w = 1; w < 4; ++w) b = kb[w][threadIdx.x] > b ? kb[w][threadIdx.x] : b;
        atomicMax(&keys[(size_t)threadIdx.x * HS + blockIdx.x % HS], b);
    }
}

template <typename T>
static void head_rows(const T *x, int M, int K, const T *W, int V, float *logits, unsigned long long *keys,
                      hipStream_t s) {
    const dim3 grid((V + 3) / 4 < HEAD_BLOCKS ? (V + 3) / 4 : HEAD_BLOCKS);
    if (M <= 1) head_kernel<T, 1><<<grid, 256, 0, s>>>(x, M, K, W, V, logits, keys);
    else if (M <= 4) head_kernel<T, 4><<<grid, 256, 0, s>>>(x, M, K, W, V, logits, keys);
    else if (M <= 8) head_kernel<T, 8><<<grid, 256, 0, s>>>(x, M, K, W, V, logits, keys);
    else head_kernel<T, 16><<<grid, 256, 0, s>>>(x, M, K, W, V, logits, keys);
}

hipError_t launch_head(int dt, const void *hs, int T, int K, const void *W, int V, float *logits, int32_t *argmax,
                       unsigned long long *keys, hipStream_t s) {
    if (argmax) head_init_kernel<<<(T * HS + 255) / 256, 256, 0, s>>>(keys, T * HS);
    const size_t es = dt == DT_BF16 ? 2 : 4;
    for (int t0 = 0; t0 < T; t0 += 16) {
        const int M = T - t0 < 16 ? T - t0 : 16;
        const char *x = (const char *)hs + (size_t)t0 * K * es;
        float *lg = logits ? logits + (size_t)t0 * V : nullptr;
        unsigned long long *kk = argmax ? keys + (size_t)t0 * HS : nullptr;
        if (dt == DT_BF16) head_rows<bf16>((const bf16 *)x, M, K, (const bf16 *)W, V, lg, kk, s);
        else head_rows<float>((const float *)x, M, K, (const float *)W, V, lg, kk, s);
    }
    if (argmax) head_final_kernel<<<T, 64, 0, s>>>(keys, T, argmax);
    return hipGetLastError();
}

// ---- the same head for callers that cannot allocate: the greedy-token keys live in one
// file-scope device array instead of a workspace.  Each device holds its own copy of the array
// until the process ends; its device address is looked up once per device (the array's name in
// host code is a host-side stand-in, never a device address) and kept.  Every call on a device
// shares that device's array: head_init_kernel clears the keys each call, and calls that
// overlap on one device race on them.
static __device__ __align__(256) unsigned long long scratch[HEAD_STATIC_MAX_T * HS];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
unsigned long long *scratch_ptr[MAX_DEVICES];  // per device; null until looked up
}  // namespace

hipError_t head_static_scratch(unsigned long long **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        scratch_ptr[dev] = (unsigned long long *)p;
    }
    *out = scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_head_static(int dt, const void *hs, int T, int K, const void *W, int V, float *logits,
                              int32_t *argmax, hipStream_t s) {
    if (T < 1 || T > HEAD_STATIC_MAX_T) return hipErrorInvalidValue;
    unsigned long long *keys = nullptr;
    if (argmax) {
        const hipError_t e = head_static_scratch(&keys);
        if (e != hipSuccess) return e;
    }
    return launch_head(dt, hs, T, K, W, V, logits, argmax, keys, s);
}

}  // namespace q3
