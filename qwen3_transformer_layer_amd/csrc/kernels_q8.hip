// kernels_q8.hip -- projections with 8-bit affine group-quantised weights.
//
// Format (the quantised fused rows of "maya2_mlx/backbone.py" fuse_proj; groups
// of 64 along the input axis): w[n][k] = s[n][g] * q[n][k] + b[n][g], g = k / 64,
// q an unsigned 8-bit code, s and b bf16.  The dequantised weight is used in
// fp32 and never rounded: for each group the kernels form sum_k x_k q_k and
// sum_k x_k and fold them as s * (x . q) + b * sum(x), the same sum regrouped.
//
//  - gemv_q8_kernel (M <= 16): each wave64 owns one output column; a lane reads
//    16 codes (one 128-bit load) and the matching 16 bf16 activations, so a
//    group's 64 codes are 4 lanes; weight bytes per column are K * (1 + 4/64).
//    All code, scale and bias loads of a lane (up to 8 chunks: K <= 8192) are
//    issued before any arithmetic (and, with the norm prologue, before the norm).
//  - M > 16: the MFMA GEMM of kernels_gemm.hip when K % 128 == 0 and the scale and bias
//    arrays are 4-byte aligned; otherwise gemm_q8_kernel: the bf16 MFMA GEMM tiling with K
//    step = one group
//    (64).  Codes are integers 0..255 and exact in bf16, so each group's MFMA
//    partial sum is exact products summed in fp32; it is folded into the
//    running accumulator with the column's scale and bias and the row's
//    activation sum over the group.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace q3 {

static __device__ __forceinline__ float epi_q8(int epi, float a, float b, const bf16 *res, size_t idx) {
    if (epi == EPI_SWIGLU) return rho<bf16>(silu_f32(rho<bf16>(a))) * rho<bf16>(b);
    if (epi == EPI_RESID) return to_f(res[idx]) + rho<bf16>(a);
    return a;
}

// Every code, scale and bias load of the lane's chunks (c = lane + 64 u, u < QU) is issued
// before any arithmetic, so a wave keeps its whole row in flight; K <= 64 * 16 * QU, QU = 2, 4
// or 8 picked from K (registers for unused chunks would lower the occupancy).
constexpr int QU_MAX = 8;

template <int QU> struct Q8Row {
    u32x4 q[QU];
    float s[QU], b[QU];
};

template <int QU>
__device__ __forceinline__ void q8_row_load(Q8Row<QU> &r, const uint8_t *codes, const bf16 *scale, const bf16 *bias,
                                            int row, int K, int ng, bool ok, int lane) {
    const uint8_t *c0 = codes + (size_t)row * K;
#pragma unroll
    for (int u = 0; u < QU; ++u) {
        const int c = lane + 64 * u;
        const bool v = ok && c < K / 16;
        r.q[u] = v ? ld_stream(c0 + (size_t)c * 16) : u32x4{0, 0, 0, 0};
        r.s[u] = v ? to_f(scale[(size_t)row * ng + (c >> 2)]) : 0.f;
        r.b[u] = v ? to_f(bias[(size_t)row * ng + (c >> 2)]) : 0.f;
    }
}

template <int EPI, int MR, int QU>
__global__ void __launch_bounds__(256) gemv_q8_kernel(const bf16 *__restrict__ x, int M, int K,
                                                      const uint8_t *__restrict__ codes,
                                                      const bf16 *__restrict__ scale, const bf16 *__restrict__ bias,
                                                      int N, const bf16 *__restrict__ res, bf16 *__restrict__ out) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = blockIdx.x * 4 + wave;
    if (n >= N) return;
    const int ng = K / 64, nch = K / 16;
    const int n1 = EPI == EPI_SWIGLU ? n + N : n;
    Q8Row<QU> r0, r1;
    q8_row_load(r0, codes, scale, bias, n, K, ng, true, lane);
    if (EPI == EPI_SWIGLU) q8_row_load(r1, codes, scale, bias, n1, K, ng, true, lane);
    float a0[MR], a1[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) a0[m] = a1[m] = 0.f;
#pragma unroll
    for (int u = 0; u < QU; ++u) {
        const int c = lane + 64 * u;
        if (c < nch) {
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                if (m < M) {
                    float xf[16];
                    const bf16 *xp = x + (size_t)m * K + (size_t)c * 16;
                    Vec<bf16>::expand(ld16(xp), xf);
                    Vec<bf16>::expand(ld16(xp + 8), xf + 8);
                    float xs = 0.f;
#pragma unroll
                    for (int i = 0; i < 16; ++i) xs += xf[i];
                    a0[m] += r0.s[u] * dot16_q8(r0.q[u], xf) + r0.b[u] * xs;
                    if (EPI == EPI_SWIGLU) a1[m] += r1.s[u] * dot16_q8(r1.q[u], xf) + r1.b[u] * xs;
                }
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
                out[idx] = from_f<bf16>(epi_q8(EPI, s0, s1, res, idx));
            }
        }
    }
}

// M == 1 with the RMSNorm prologue (norm_prologue): activations come from LDS.
template <int EPI, int QU>
__global__ void __launch_bounds__(256) gemv_q8_norm_kernel(const bf16 *__restrict__ h_in, const bf16 *__restrict__ res,
                                                           const bf16 *__restrict__ nw, float eps,
                                                           bf16 *__restrict__ h_out, int K,
                                                           const uint8_t *__restrict__ codes,
                                                           const bf16 *__restrict__ scale,
                                                           const bf16 *__restrict__ bias, int N,
                                                           bf16 *__restrict__ out) {
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    bf16 *ys = (bf16 *)smem_raw;
    __shared__ float red[8];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = blockIdx.x * 4 + wave;
    const bool active = n < N;
    const int ng = K / 64, nch = K / 16;
    const int n1 = EPI == EPI_SWIGLU ? n + N : n;
    Q8Row<QU> r0, r1;  // the whole row in flight during the norm
    q8_row_load(r0, codes, scale, bias, active ? n : 0, K, ng, active, lane);
    if (EPI == EPI_SWIGLU) q8_row_load(r1, codes, scale, bias, active ? n1 : 0, K, ng, active, lane);
    norm_prologue<bf16>(h_in, res, nw, eps, h_out, K, ys, red);
    if (!active) return;
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int u = 0; u < QU; ++u) {
        const int c = lane + 64 * u;
        if (c < nch) {
            float xf[16];
            Vec<bf16>::expand(*(const u32x4 *)&ys[c * 16], xf);
            Vec<bf16>::expand(*(const u32x4 *)&ys[c * 16 + 8], xf + 8);
            float xs = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) xs += xf[i];
            a0 += r0.s[u] * dot16_q8(r0.q[u], xf) + r0.b[u] * xs;
            if (EPI == EPI_SWIGLU) a1 += r1.s[u] * dot16_q8(r1.q[u], xf) + r1.b[u] * xs;
        }
    }
    const float s0 = wave_sum(a0);
    const float s1 = EPI == EPI_SWIGLU ? wave_sum(a1) : 0.f;
    if (lane == 0) out[n] = from_f<bf16>(epi_q8(EPI, s0, s1, nullptr, n));
}

hipError_t launch_linear_q8_norm(const void *h_in, const void *res, const void *nw, float eps, void *h_out, int K,
                                 const uint8_t *codes, const void *scale, const void *bias, int group, int N,
                                 int epi, void *out, hipStream_t s) {
    if (group != 64 || epi == EPI_RESID || K > 64 * 16 * QU_MAX) return hipErrorInvalidValue;
    const dim3 grid((N + 3) / 4);
    const size_t lds = (size_t)K * sizeof(bf16);
    const bf16 *hi = (const bf16 *)h_in, *rr = (const bf16 *)res, *ww = (const bf16 *)nw;
    const bf16 *sc = (const bf16 *)scale, *bi = (const bf16 *)bias;
    auto go = [&](auto epi_c, auto qu_c) {
        gemv_q8_norm_kernel<decltype(epi_c)::value, decltype(qu_c)::value><<<grid, 256, lds, s>>>(
            hi, rr, ww, eps, (bf16 *)h_out, K, codes, sc, bi, N, (bf16 *)out);
    };
    using I = std::integral_constant<int, EPI_STORE>;
    using G = std::integral_constant<int, EPI_SWIGLU>;
    using U2 = std::integral_constant<int, 2>;
    using U4 = std::integral_constant<int, 4>;
    using U8 = std::integral_constant<int, 8>;
    if (epi == EPI_SWIGLU) {
        if (K <= 2048) go(G{}, U2{});
        else if (K <= 4096) go(G{}, U4{});
        else go(G{}, U8{});
    } else {
        if (K <= 2048) go(I{}, U2{});
        else if (K <= 4096) go(I{}, U4{});
        else go(I{}, U8{});
    }
    return hipGetLastError();
}

namespace gq8 {
constexpr int BM = 128, BN = 128, BK = 64, LDA = BK + 8, LDB = BK + 16;  // pitches: A in bf16, B in bytes
}

template <int EPI> __device__ __forceinline__ int q8_b_row(int nb, int r, int N) {
    if (EPI == EPI_SWIGLU) return r < 64 ? nb * 64 + r : N + nb * 64 + (r - 64);
    return nb * gq8::BN + r;
}

static __device__ __forceinline__ bf16x8 codes_to_bf16x8(uint2 c) {
    bf16x8 r;
    uint32_t *rw = (uint32_t *)&r;
    const uint32_t w[2] = {c.x, c.y};
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const uint32_t lo = __float_as_uint((float)((w[i] >> (16 * b)) & 0xffu)) >> 16;
            const uint32_t hi = __float_as_uint((float)((w[i] >> (16 * b + 8)) & 0xffu)) >> 16;
            rw[2 * i + b] = lo | (hi << 16);
        }
    return r;
}

template <int EPI>
__global__ void __launch_bounds__(256) gemm_q8_kernel(const bf16 *__restrict__ A, int M, int K,
                                                      const uint8_t *__restrict__ codes,
                                                      const bf16 *__restrict__ scale, const bf16 *__restrict__ bias,
                                                      int N, const bf16 *__restrict__ res, bf16 *__restrict__ out) {
    using namespace gq8;
    __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDA];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[BN * LDB];
    __shared__ float Xs[BM];          // sum of the group's activations per row
    __shared__ float Ss[BN], Bb[BN];  // scale and bias of the group per B-tile row
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * BM, nb = blockIdx.x;
    const int ng = K / 64;
    int brow[2];
    if (EPI == EPI_SWIGLU) {
        brow[0] = wn * 32;
        brow[1] = 64 + wn * 32;
    } else {
        brow[0] = wn * 64;
        brow[1] = wn * 64 + 32;
    }
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    for (int g = 0; g < ng; ++g) {
        const int k0 = g * 64;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // A: 128 rows x 64 bf16 = 1024 chunks of 16 B
            const int cidx = tid + i * 256, row = cidx >> 3, col = (cidx & 7) * 8;
            const int gm = m0 + row;
            *(u32x4 *)&As[row * LDA + col] = gm < M ? ld16(A + (size_t)gm * K + k0 + col) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {  // B: 128 rows x 64 codes = 512 chunks of 16 B
            const int cidx = tid + i * 256, row = cidx >> 2, col = (cidx & 3) * 16;
            const bool bval = EPI == EPI_SWIGLU ? nb * 64 + (row & 63) < N : nb * BN + row < N;
            *(u32x4 *)&Bs[row * LDB + col] =
                bval ? ld_stream(codes + (size_t)q8_b_row<EPI>(nb, row, N) * K + k0 + col) : u32x4{0, 0, 0, 0};
        }
        if (tid < BN) {
            const bool bval = EPI == EPI_SWIGLU ? nb * 64 + (tid & 63) < N : nb * BN + tid < N;
            const int wr = q8_b_row<EPI>(nb, tid, N);
            Ss[tid] = bval ? to_f(scale[(size_t)wr * ng + g]) : 0.f;
            Bb[tid] = bval ? to_f(bias[(size_t)wr * ng + g]) : 0.f;
        }
        __syncthreads();
        if (tid < BM) {
            float xs = 0.f;
            for (int c = 0; c < 64; ++c) xs += to_f(bf16{As[tid * LDA + c]});
            Xs[tid] = xs;
        }
        f32x16 part[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) part[i][j][v] = 0.f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            bf16x8 af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *(const bf16x8 *)&As[(wm * 64 + i * 32 + (lane & 31)) * LDA + kk * 16 + (lane >> 5) * 8];
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bfr[j] = codes_to_bf16x8(*(const uint2 *)&Bs[(brow[j] + (lane & 31)) * LDB + kk * 16 + (lane >> 5) * 8]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], part[i][j], 0, 0, 0);
        }
        __syncthreads();  // Xs ready
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float sc = Ss[brow[j] + (lane & 31)], bi = Bb[brow[j] + (lane & 31)];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                    acc[i][j][v] += sc * part[i][j][v] + bi * Xs[r];
                }
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int row = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (row >= M) continue;
            if (EPI == EPI_SWIGLU) {
                const int col = nb * 64 + wn * 32 + (lane & 31);
                if (col >= N) continue;
                const size_t idx = (size_t)row * N + col;
                out[idx] = from_f<bf16>(epi_q8(EPI, acc[i][0][v], acc[i][1][v], res, idx));
            } else {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int col = nb * BN + brow[j] + (lane & 31);
                    if (col >= N) continue;
                    const size_t idx = (size_t)row * N + col;
                    out[idx] = from_f<bf16>(epi_q8(EPI, acc[i][j][v], 0.f, res, idx));
                }
            }
        }
    }
}

template <int EPI>
static void gemv_q8_dispatch(const void *x, int M, int K, const uint8_t *codes, const void *scale, const void *bias,
                             int N, const void *res, void *out, hipStream_t s) {
    const dim3 grid((N + 3) / 4);
    const bf16 *xx = (const bf16 *)x, *sc = (const bf16 *)scale, *bi = (const bf16 *)bias, *rr = (const bf16 *)res;
    bf16 *oo = (bf16 *)out;
    auto go = [&](auto mr_c) {
        constexpr int MR = decltype(mr_c)::value;
        if (K <= 2048) gemv_q8_kernel<EPI, MR, 2><<<grid, 256, 0, s>>>(xx, M, K, codes, sc, bi, N, rr, oo);
        else if (K <= 4096) gemv_q8_kernel<EPI, MR, 4><<<grid, 256, 0, s>>>(xx, M, K, codes, sc, bi, N, rr, oo);
        else gemv_q8_kernel<EPI, MR, 8><<<grid, 256, 0, s>>>(xx, M, K, codes, sc, bi, N, rr, oo);
    };
    if (M <= 1) go(std::integral_constant<int, 1>{});
    else if (M <= 4) go(std::integral_constant<int, 4>{});
    else if (M <= 8) go(std::integral_constant<int, 8>{});
    else go(std::integral_constant<int, 16>{});
}

hipError_t launch_linear_q8(const void *x, int M, int K, const uint8_t *codes, const void *scale, const void *bias,
                            int group, int N, int epi, const void *res, void *out, hipStream_t s) {
    if (group != 64) return hipErrorInvalidValue;
    if (M <= 16) {
        if (K > 64 * 16 * QU_MAX) return hipErrorInvalidValue;
        if (epi == EPI_SWIGLU) gemv_q8_dispatch<EPI_SWIGLU>(x, M, K, codes, scale, bias, N, res, out, s);
        else if (epi == EPI_RESID) gemv_q8_dispatch<EPI_RESID>(x, M, K, codes, scale, bias, N, res, out, s);
        else gemv_q8_dispatch<EPI_STORE>(x, M, K, codes, scale, bias, N, res, out, s);
        return hipGetLastError();
    }
    if (gemm_q8_dma_ok(M, K, N, scale, bias))
        return launch_gemm_q8_dma(x, M, K, codes, scale, bias, N, epi, res, out, s);
    const dim3 grid(epi == EPI_SWIGLU ? (N + 63) / 64 : (N + gq8::BN - 1) / gq8::BN, (M + gq8::BM - 1) / gq8::BM);
    const bf16 *a = (const bf16 *)x, *sc = (const bf16 *)scale, *bi = (const bf16 *)bias, *r = (const bf16 *)res;
    bf16 *o = (bf16 *)out;
    if (epi == EPI_SWIGLU) gemm_q8_kernel<EPI_SWIGLU><<<grid, 256, 0, s>>>(a, M, K, codes, sc, bi, N, r, o);
    else if (epi == EPI_RESID) gemm_q8_kernel<EPI_RESID><<<grid, 256, 0, s>>>(a, M, K, codes, sc, bi, N, r, o);
    else gemm_q8_kernel<EPI_STORE><<<grid, 256, 0, s>>>(a, M, K, codes, sc, bi, N, r, o);
    return hipGetLastError();
}

}  // namespace q3
