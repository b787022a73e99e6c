// kernels_linear.hip -- projections y = x . W^T with fused epilogues.
//
// The four projections of a layer ("maya2_mlx/backbone.py", forward: Q.mm with
// the fused q|k|v rows, o_proj, fused gate|up rows, down) all take x [M][K] and a
// row-major weight [rows][K].  Epilogues apply the page's rounding points:
// STORE rounds the product once; RESID adds the rounded product to the residual
// and rounds once more (h = h + o_proj(attn)); SWIGLU takes gate row n and up
// row N + n together and rounds silu (computed in fp32) once, then the product
// with up once.
//
//  - gemv_kernel: M <= 16 (decode).  HBM-bound: each wave64 owns one output
//    column (a gate/up pair for SWIGLU) and streams its weight row with
//    128-bit non-temporal loads, 4 loads in flight per lane; x is read through
//    the L1/L2 caches; one wave reduction per output.
//  - M > 16 in bf16: the MFMA GEMM of kernels_gemm.hip.
//  - gemv_mfma_kernel: 2 <= M <= 16 in bf16 (several seats' decode steps): v_mfma_f32_16x16x32_bf16
//    on 16 weight rows x the M activation rows (padded to 16), so every 16-byte weight load
//    pairs with one activation load (the plain GEMV re-reads all M activation chunks per weight
//    chunk).  Block = 8 waves on the same 16 outputs (32 weight rows for SWIGLU), each a K/8
//    slice with 8 loads in flight per lane; the 8 partial tiles are summed in LDS in wave order.
//  - gemv8_mfma_kernel: the same on 8 outputs per block, where 16-output blocks would leave CUs
//    idle (2048 outputs: o_proj, down) or need a partial second round (gate|up).
//  - gemm_f32_kernel: M > 16 in fp32 (strict mode), LDS-tiled FMA.
#include "common.h"
#include "kernels.h"

namespace q3 {

template <typename T> __device__ __forceinline__ float epi_value(int epi, float a, float b, const T *res, size_t idx) {
    if (epi == EPI_SWIGLU) {
        const float g = rho<T>(a), u = rho<T>(b);
        return rho<T>(silu_f32(g)) * u;
    }
    if (epi == EPI_RESID) return to_f(res[idx]) + rho<T>(a);
    return a;
}

// ------------------------------------------------------------ GEMV (M <= 16)
template <typename T, int EPI, int MR>
__global__ void __launch_bounds__(256) gemv_kernel(const T *__restrict__ x, int M, int K, const T *__restrict__ W,
                                                   int N, const T *__restrict__ res, T *__restrict__ out) {
    constexpr int VN = Vec<T>::N;
    constexpr int U = 4;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = blockIdx.x * 4 + wave;
    if (n >= N) return;
    const T *w0 = W + (size_t)n * K;
    const T *w1 = W + (size_t)(EPI == EPI_SWIGLU ? n + N : n) * K;
    float a0[MR], a1[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) a0[m] = a1[m] = 0.f;
    const int nc = K / VN;  // 16-byte chunks per row
    int c = lane;
    for (; c + 64 * (U - 1) < nc; c += 64 * U) {
        u32x4 wv0[U], wv1[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            wv0[u] = ld_stream(w0 + (size_t)(c + 64 * u) * VN);
            if (EPI == EPI_SWIGLU) wv1[u] = ld_stream(w1 + (size_t)(c + 64 * u) * VN);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                if (m < M) {
                    const u32x4 xv = ld16(x + (size_t)m * K + (size_t)(c + 64 * u) * VN);
                    a0[m] = dot16<T>(wv0[u], xv, a0[m]);
                    if (EPI == EPI_SWIGLU) a1[m] = dot16<T>(wv1[u], xv, a1[m]);
                }
            }
        }
    }
    for (; c < nc; c += 64) {
        const u32x4 wt0 = ld_stream(w0 + (size_t)c * VN);
        const u32x4 wt1 = EPI == EPI_SWIGLU ? ld_stream(w1 + (size_t)c * VN) : wt0;
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            if (m < M) {
                const u32x4 xv = ld16(x + (size_t)m * K + (size_t)c * VN);
                a0[m] = dot16<T>(wt0, xv, a0[m]);
                if (EPI == EPI_SWIGLU) a1[m] = dot16<T>(wt1, xv, a1[m]);
            }
        }
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        if (m < M) {
            const float s0 = wave_sum(a0[m]);
            const float s1 = EPI == EPI_SWIGLU ? wave_sum(a1[m]) : 0.f;
            if (lane == 0) {
                const size_t idx = (size_t)m * N + n;
                out[idx] = from_f<T>(epi_value<T>(EPI, s0, s1, res, idx));
            }
        }
    }
}

// ------------------------------------------------------------ GEMV with RMSNorm prologue (M == 1)
// The decode projections that follow a norm (q|k|v after the input norm with the deferred
// residual add; gate|up after the post-attention norm) normalise the row once per block
// into LDS and stream the weights as gemv_kernel does.
template <typename T, int EPI>
__global__ void __launch_bounds__(256) gemv_norm_kernel(const T *__restrict__ h_in, const T *__restrict__ res,
                                                        const T *__restrict__ nw, float eps, T *__restrict__ h_out,
                                                        int K, const T *__restrict__ W, int N, T *__restrict__ out) {
    constexpr int VN = Vec<T>::N;
    constexpr int U = 4;
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    T *ys = (T *)smem_raw;
    __shared__ float red[8];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = blockIdx.x * 4 + wave;
    const bool active = n < N;
    const T *w0 = W + (size_t)(active ? n : 0) * K;
    const T *w1 = W + (size_t)(active ? (EPI == EPI_SWIGLU ? n + N : n) : 0) * K;
    const int nc = K / VN;
    // the first U chunks of the weight row(s) are in flight while the block normalises
    u32x4 wv0[U], wv1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = lane + 64 * u;
        const bool ok = active && c < nc;
        wv0[u] = ok ? ld_stream(w0 + (size_t)c * VN) : u32x4{0, 0, 0, 0};
        if (EPI == EPI_SWIGLU) wv1[u] = ok ? ld_stream(w1 + (size_t)c * VN) : u32x4{0, 0, 0, 0};
    }
    norm_prologue<T>(h_in, res, nw, eps, h_out, K, ys, red);
    if (!active) return;
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = lane + 64 * u;
        if (c < nc) {
            const u32x4 xv = *(const u32x4 *)&ys[c * VN];
            a0 = dot16<T>(wv0[u], xv, a0);
            if (EPI == EPI_SWIGLU) a1 = dot16<T>(wv1[u], xv, a1);
        }
    }
    int c = lane + 64 * U;
    for (; c + 64 * (U - 1) < nc; c += 64 * U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            wv0[u] = ld_stream(w0 + (size_t)(c + 64 * u) * VN);
            if (EPI == EPI_SWIGLU) wv1[u] = ld_stream(w1 + (size_t)(c + 64 * u) * VN);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const u32x4 xv = *(const u32x4 *)&ys[(c + 64 * u) * VN];
            a0 = dot16<T>(wv0[u], xv, a0);
            if (EPI == EPI_SWIGLU) a1 = dot16<T>(wv1[u], xv, a1);
        }
    }
    for (; c < nc; c += 64) {
        const u32x4 xv = *(const u32x4 *)&ys[c * VN];
        a0 = dot16<T>(ld_stream(w0 + (size_t)c * VN), xv, a0);
        if (EPI == EPI_SWIGLU) a1 = dot16<T>(ld_stream(w1 + (size_t)c * VN), xv, a1);
    }
    const float s0 = wave_sum(a0);
    const float s1 = EPI == EPI_SWIGLU ? wave_sum(a1) : 0.f;
    if (lane == 0) out[n] = from_f<T>(epi_value<T>(EPI, s0, s1, (const T *)nullptr, n));
}

template <typename T>
static void launch_gemv_norm_t(int epi, const void *h_in, const void *res, const void *nw, float eps, void *h_out,
                               int K, const void *W, int N, void *out, hipStream_t s) {
    const dim3 grid((N + 3) / 4);
    const size_t lds = (size_t)K * sizeof(T);
    const T *hi = (const T *)h_in, *rr = (const T *)res, *ww = (const T *)nw, *WW = (const T *)W;
    if (epi == EPI_SWIGLU)
        gemv_norm_kernel<T, EPI_SWIGLU><<<grid, 256, lds, s>>>(hi, rr, ww, eps, (T *)h_out, K, WW, N, (T *)out);
    else
        gemv_norm_kernel<T, EPI_STORE><<<grid, 256, lds, s>>>(hi, rr, ww, eps, (T *)h_out, K, WW, N, (T *)out);
}

hipError_t launch_linear_norm(int dt, const void *h_in, const void *res, const void *nw, float eps, void *h_out,
                              int K, const void *W, int N, int epi, void *out, hipStream_t s) {
    if (epi == EPI_RESID) return hipErrorInvalidValue;
    if (dt == DT_BF16) launch_gemv_norm_t<bf16>(epi, h_in, res, nw, eps, h_out, K, W, N, out, s);
    else launch_gemv_norm_t<float>(epi, h_in, res, nw, eps, h_out, K, W, N, out, s);
    return hipGetLastError();
}

// ------------------------------------------------------------ skinny MFMA GEMV (2 <= M <= 16, bf16)
// MFMA 16x16x32: lane i supplies A[i % 16][8 (i / 16) .. + 8] (activation row i % 16) and
// B[8 (i / 16) .. + 8][i % 16] (weight row n0 + i % 16); accumulator j of lane i is
// C[4 (i / 16) + j][i % 16].  K % 256 == 0.
template <int EPI>
__global__ void __launch_bounds__(512) gemv_mfma_kernel(const bf16 *__restrict__ x, int M, int K,
                                                        const bf16 *__restrict__ W, int N, const bf16 *__restrict__ res,
                                                        bf16 *__restrict__ out) {
    constexpr int NWV = 8, U = 8;
    constexpr int NT = EPI == EPI_SWIGLU ? 2 : 1;  // gate and up tiles
    __shared__ f32x4 part[NWV - 1][NT][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n0 = blockIdx.x * 16, r = lane & 15, h = lane >> 4;
    const bf16 *xr = x + (size_t)min(r, M - 1) * K + 8 * h;
    const bf16 *wr[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) wr[t] = W + (size_t)(t * N + min(n0 + r, N - 1)) * K + 8 * h;
    const int ks = K / NWV, k0 = wave * ks;  // this wave's K slice, a multiple of 32
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kb = k0; kb < k0 + ks; kb += 32 * U) {
        u32x4 wv[NT][U], xv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = kb + 32 * u;
            const bool ok = k < k0 + ks;
#pragma unroll
            for (int t = 0; t < NT; ++t) wv[t][u] = ok ? ld_stream(wr[t] + k) : u32x4{0, 0, 0, 0};
            xv[u] = ok ? ld16(xr + k) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bf16x8 a = __builtin_bit_cast(bf16x8, xv[u]);
#pragma unroll
            for (int t = 0; t < NT; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, wv[t][u]), acc[t], 0, 0, 0);
        }
    }
    if (wave > 0)
#pragma unroll
        for (int t = 0; t < NT; ++t) part[wave - 1][t][lane] = acc[t];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < NWV - 1; ++w)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] += part[w][t][lane];
    const int n = n0 + r;
    if (n >= N) return;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int m = 4 * h + j;
        if (m >= M) continue;
        const size_t idx = (size_t)m * N + n;
        out[idx] = from_f<bf16>(epi_value<bf16>(EPI, acc[0][j], NT > 1 ? acc[NT - 1][j] : 0.f, res, idx));
    }
}

// ------------------------------------------------------------ skinny MFMA GEMV, 8 outputs per block
// The same MFMA and wave layout on 8 outputs per block, for the shapes where 16-output blocks
// leave CUs idle or need a second round: 2048 outputs give 256 blocks, gate|up's 6144 give 768 (three
// resident per CU).  The B operand's 16 columns hold, for SWIGLU, the 8 gate rows then the 8 up rows
// of the same outputs (the up value of column r is column r + 8, lane ^ 8); otherwise the 8 rows
// twice, and the duplicate columns are not stored.  Each lane issues all U weight and activation
// loads of its K slice at once (K = NWV * 32 * U).  Same products and summation order as
// gemv_mfma_kernel with 8 waves.
template <int EPI, int NWV, int U>
__global__ void __launch_bounds__(64 * NWV) gemv8_mfma_kernel(const bf16 *__restrict__ x, int M, int K,
                                                             const bf16 *__restrict__ W, int N, const bf16 *res,
                                                             bf16 *out) {
    __shared__ f32x4 part[NWV - 1][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n0 = blockIdx.x * 8, r = lane & 15, h = lane >> 4;
    const int wrow = EPI == EPI_SWIGLU ? (r < 8 ? min(n0 + r, N - 1) : N + min(n0 + r - 8, N - 1))
                                       : min(n0 + (r & 7), N - 1);
    const bf16 *xr = x + (size_t)min(r, M - 1) * K + 8 * h;
    const bf16 *wr = W + (size_t)wrow * K + 8 * h;
    const int k0 = wave * 32 * U;
    u32x4 wv[U], xv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        wv[u] = ld_stream(wr + k0 + 32 * u);
        xv[u] = ld16(xr + k0 + 32 * u);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load issued before the first MFMA waits for one
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < U; ++u)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xv[u]), __builtin_bit_cast(bf16x8, wv[u]),
                                                      acc, 0, 0, 0);
    if (wave > 0) part[wave - 1][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < NWV - 1; ++w) acc += part[w][lane];
    // accumulator j of lane i: activation row 4 (i / 16) + j, column i % 16
    float up[4] = {0.f, 0.f, 0.f, 0.f};
    if (EPI == EPI_SWIGLU)
#pragma unroll
        for (int j = 0; j < 4; ++j) up[j] = __shfl_xor(acc[j], 8);
    const int n = n0 + r;
    if (r >= 8 || n >= N) return;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int m = 4 * h + j;
        if (m >= M) continue;
        const size_t idx = (size_t)m * N + n;
        out[idx] = from_f<bf16>(epi_value<bf16>(EPI, acc[j], up[j], res, idx));
    }
}

// ------------------------------------------------------------ fp32 tiled GEMM (strict mode)
template <int EPI>
__global__ void __launch_bounds__(256) gemm_f32_kernel(const float *__restrict__ A, int M, int K,
                                                       const float *__restrict__ B, int N,
                                                       const float *__restrict__ res, float *__restrict__ out) {
    // 64 x 64 output tile (SWIGLU: 64 x 32 outputs from 32 gate + 32 up rows), K step 16.
    __shared__ float As[16][64 + 1];
    __shared__ float Bs[16][64 + 1];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int m0 = blockIdx.y * 64, nb = blockIdx.x;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += 16) {
        for (int i = tid; i < 64 * 16; i += 256) {
            const int r = i / 16, kk = i % 16;
            const int gm = m0 + r, gk = k0 + kk;
            As[kk][r] = (gm < M && gk < K) ? A[(size_t)gm * K + gk] : 0.f;
            int wr;
            if (EPI == EPI_SWIGLU) wr = r < 32 ? nb * 32 + r : N + nb * 32 + (r - 32);
            else wr = nb * 64 + r;
            const bool ok = (EPI == EPI_SWIGLU ? (nb * 32 + (r & 31)) < N : wr < N) && gk < K;
            Bs[kk][r] = ok ? B[(size_t)wr * K + gk] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
        }
        __syncthreads();
    }
    if (EPI == EPI_SWIGLU) {
        // columns tx*4+j < 32 are gate, >= 32 up: exchange through LDS
        __shared__ float Cs[64][64 + 1];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) Cs[ty * 4 + i][tx * 4 + j] = acc[i][j];
        __syncthreads();
        for (int e = tid; e < 64 * 32; e += 256) {
            const int r = e / 32, cc = e % 32;
            const int row = m0 + r, col = nb * 32 + cc;
            if (row < M && col < N) {
                const size_t idx = (size_t)row * N + col;
                out[idx] = epi_value<float>(EPI, Cs[r][cc], Cs[r][32 + cc], res, idx);
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = m0 + ty * 4 + i, col = nb * 64 + tx * 4 + j;
            if (row < M && col < N) {
                const size_t idx = (size_t)row * N + col;
                out[idx] = epi_value<float>(EPI, acc[i][j], 0.f, res, idx);
            }
        }
}

// ------------------------------------------------------------ dispatch
template <typename T, int EPI>
static void launch_gemv_t(const void *x, int M, int K, const void *W, int N, const void *res, void *out,
                          hipStream_t s) {
    const dim3 grid((N + 3) / 4);
    const T *xx = (const T *)x, *ww = (const T *)W, *rr = (const T *)res;
    T *oo = (T *)out;
    if (M <= 1) gemv_kernel<T, EPI, 1><<<grid, 256, 0, s>>>(xx, M, K, ww, N, rr, oo);
    else if (M <= 2) gemv_kernel<T, EPI, 2><<<grid, 256, 0, s>>>(xx, M, K, ww, N, rr, oo);
    else if (M <= 4) gemv_kernel<T, EPI, 4><<<grid, 256, 0, s>>>(xx, M, K, ww, N, rr, oo);
    else if (M <= 8) gemv_kernel<T, EPI, 8><<<grid, 256, 0, s>>>(xx, M, K, ww, N, rr, oo);
    else gemv_kernel<T, EPI, 16><<<grid, 256, 0, s>>>(xx, M, K, ww, N, rr, oo);
}

template <typename T>
static void launch_gemv(int epi, const void *x, int M, int K, const void *W, int N, const void *res, void *out,
                        hipStream_t s) {
    if (epi == EPI_SWIGLU) launch_gemv_t<T, EPI_SWIGLU>(x, M, K, W, N, res, out, s);
    else if (epi == EPI_RESID) launch_gemv_t<T, EPI_RESID>(x, M, K, W, N, res, out, s);
    else launch_gemv_t<T, EPI_STORE>(x, M, K, W, N, res, out, s);
}

hipError_t launch_linear(int dt, const void *x, int M, int K, const void *W, int N, int epi, const void *res,
                         void *out, hipStream_t s) {
    if (M <= 16 && M >= 2 && dt == DT_BF16 && K % 256 == 0) {
        const dim3 grid((N + 15) / 16);
        const bf16 *a = (const bf16 *)x, *b = (const bf16 *)W, *r = (const bf16 *)res;
        bf16 *o = (bf16 *)out;
        // 8 outputs per block where 16 would give fewer than 256 blocks or a partial second round
        // (gate|up); K 2048 / 4096 / 6144 (all loads of a K slice in flight at once)
        const bool eight = epi == EPI_SWIGLU ? N % 256 != 0 || (N / 16) % 256 != 0 : (N + 15) / 16 < 256;
        if (eight && (K == 2048 || K == 4096 || K == 6144)) {
            const dim3 g8((N + 7) / 8);
            if (epi == EPI_SWIGLU) {
                if (K == 2048) gemv8_mfma_kernel<EPI_SWIGLU, 8, 8><<<g8, 512, 0, s>>>(a, M, K, b, N, r, o);
                else if (K == 4096) gemv8_mfma_kernel<EPI_SWIGLU, 8, 16><<<g8, 512, 0, s>>>(a, M, K, b, N, r, o);
                else gemv8_mfma_kernel<EPI_SWIGLU, 8, 24><<<g8, 512, 0, s>>>(a, M, K, b, N, r, o);
            } else if (epi == EPI_RESID) {
                if (K == 2048) gemv8_mfma_kernel<EPI_RESID, 8, 8><<<g8, 512, 0, s>>>(a, M, K, b, N, r, o);
                else if (K == 4096) gemv8_mfma_kernel<EPI_RESID, 8, 16><<<g8, 512, 0, s>>>(a, M, K, b, N, r, o);
                else gemv8_mfma_kernel<EPI_RESID, 8, 24><<<g8, 512, 0, s>>>(a, M, K, b, N, r, o);
            } else {
                if (K == 2048) gemv8_mfma_kernel<EPI_STORE, 8, 8><<<g8, 512, 0, s>>>(a, M, K, b, N, r, o);
                else if (K == 4096) gemv8_mfma_kernel<EPI_STORE, 8, 16><<<g8, 512, 0, s>>>(a, M, K, b, N, r, o);
                else gemv8_mfma_kernel<EPI_STORE, 8, 24><<<g8, 512, 0, s>>>(a, M, K, b, N, r, o);
            }
            return hipGetLastError();
        }
        if (epi == EPI_SWIGLU) gemv_mfma_kernel<EPI_SWIGLU><<<grid, 512, 0, s>>>(a, M, K, b, N, r, o);
        else if (epi == EPI_RESID) gemv_mfma_kernel<EPI_RESID><<<grid, 512, 0, s>>>(a, M, K, b, N, r, o);
        else gemv_mfma_kernel<EPI_STORE><<<grid, 512, 0, s>>>(a, M, K, b, N, r, o);
        return hipGetLastError();
    }
    if (M <= 16) {
        if (dt == DT_BF16) launch_gemv<bf16>(epi, x, M, K, W, N, res, out, s);
        else launch_gemv<float>(epi, x, M, K, W, N, res, out, s);
        return hipGetLastError();
    }
    if (dt == DT_BF16) {
        if (!gemm_dma_ok(M, K, N)) return hipErrorInvalidValue;
        return launch_gemm_dma(x, M, K, W, N, epi, res, out, s);
    }
    const dim3 grid(epi == EPI_SWIGLU ? (N + 31) / 32 : (N + 63) / 64, (M + 63) / 64);
    const float *a = (const float *)x, *b = (const float *)W, *r = (const float *)res;
    float *o = (float *)out;
    if (epi == EPI_SWIGLU) gemm_f32_kernel<EPI_SWIGLU><<<grid, 256, 0, s>>>(a, M, K, b, N, r, o);
    else if (epi == EPI_RESID) gemm_f32_kernel<EPI_RESID><<<grid, 256, 0, s>>>(a, M, K, b, N, r, o);
    else gemm_f32_kernel<EPI_STORE><<<grid, 256, 0, s>>>(a, M, K, b, N, r, o);
    return hipGetLastError();
}

}  // namespace q3
