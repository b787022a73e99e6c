// kernels_gemm.hip -- the bf16 projections of prefill (M > 16 rows): y = x . W^T with the
// fused epilogues of kernels_linear.hip ("maya2_mlx/backbone.py", forward: the fused q|k|v
// rows, o_proj + residual, fused gate|up rows + SwiGLU, down; the rounding points are those
// of epi_value there).
//
// Design for gfx950:
//  - v_mfma_f32_32x32x16_bf16; block tile 128 rows x BN weight rows (BN = 256 or 128),
//    4 waves in a 2 x 2 layout, each wave 64 rows x BN/2 weight rows (2 x BN/64 MFMA tiles).
//    For SWIGLU a tile holds BN/2 gate rows and the BN/2 up rows of the same outputs, and a
//    wave holds the gate and up accumulators of the same output columns.
//  - K steps of 64 flow through a 3-stage LDS pipeline filled by direct-to-LDS copies
//    (global_load_lds_dwordx4, 1 KB per instruction): two stages are in flight while the
//    third is consumed, with no register staging.  One barrier per K step.
//  - LDS rows are 128 B (64 bf16) with the 16-byte chunks XOR-swizzled by the row index, so
//    a fragment read (32 rows, one chunk each) hits distinct banks.  The copy's lane ->
//    address mapping writes that layout directly: lane l of a copy fetches row l/8, chunk
//    (l%8) ^ (row%8).
//  - Rows past M and weight rows past N are clamped to the last valid row on load and
//    skipped on store.  K must be a multiple of 64.
#include "common.h"
#include "kernels.h"

namespace q3 {
namespace g2 {

constexpr int BM = 128, BK = 64, STAGES = 3;
constexpr int ROWB = BK * 2;  // bytes per LDS row

template <int BN> struct Geo {
    static constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB, STAGE = A_BYTES + B_BYTES;
    static constexpr int COPIES = STAGE / 1024;  // 1 KB copies per stage
    static constexpr int PER_WAVE = COPIES / 4;
    static constexpr int NT = BN / 64;           // MFMA tiles per wave along the weight rows
    static_assert(COPIES % 4 == 0, "copies split evenly over the 4 waves");
};

// Weight row held by tile-local row r of weight block nb.
template <int EPI, int BN> __device__ __forceinline__ int w_row(int nb, int r, int N) {
    if (EPI == EPI_SWIGLU) {
        constexpr int H = BN / 2;
        const int n = nb * H + (r < H ? r : r - H);
        return (r < H ? 0 : N) + min(n, N - 1);
    }
    return min(nb * BN + r, N - 1);
}

// Swizzled byte offset of (row, 16-byte chunk c) inside an operand tile.
__device__ __forceinline__ int swz(int row, int c) { return row * ROWB + ((c ^ (row & 7)) << 4); }

}  // namespace g2

template <int EPI, int BN>
__global__ void __launch_bounds__(256) gemm_bf16_dma_kernel(const bf16 *__restrict__ A, int M, int K,
                                                            const bf16 *__restrict__ W, int N,
                                                            const bf16 *__restrict__ res, bf16 *__restrict__ out) {
    using namespace g2;
    using G = Geo<BN>;
    extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * BM, nb = blockIdx.x;
    const int nk = K / BK;
    const unsigned lds0 = (unsigned)(uintptr_t)smem;

    // this wave's copies of one stage: copy d covers 8 tile rows (A rows for d < 16)
    auto issue = [&](int kt) {
        const int st = kt % STAGES, k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < G::PER_WAVE; ++i) {
            const int d = wave + 4 * i;
            const int r = (d & 15) * 8 + (lane >> 3);  // row inside its operand tile (d < 16: A)
            const int c = (lane & 7) ^ (r & 7);
            const bf16 *src;
            unsigned dst;
            if (d < 16) {
                src = A + (size_t)min(m0 + r, M - 1) * K + k0 + c * 8;
                dst = lds0 + st * G::STAGE + d * 1024;
            } else {
                const int rb = (d - 16) * 8 + (lane >> 3);
                const int cb = (lane & 7) ^ (rb & 7);
                src = W + (size_t)w_row<EPI, BN>(nb, rb, N) * K + k0 + cb * 8;
                dst = lds0 + st * G::STAGE + G::A_BYTES + (d - 16) * 1024;
            }
            dma16(src, __builtin_amdgcn_readfirstlane(dst));
        }
    };

    f32x16 acc[2][G::NT];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < G::NT; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // tile-local weight rows of this wave's MFMA tiles
    int brow[G::NT];
#pragma unroll
    for (int j = 0; j < G::NT; ++j) {
        if (EPI == EPI_SWIGLU) {
            constexpr int HJ = G::NT / 2;  // gate tiles, then the matching up tiles
            brow[j] = (j < HJ ? 0 : BN / 2) + wn * (BN / 4) + 32 * (j % HJ);
        } else {
            brow[j] = wn * (BN / 2) + 32 * j;
        }
    }

    issue(0);
    if (nk > 1) issue(1);
    for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) wait_vm<G::PER_WAVE>();  // this wave's copies of stage kt have landed
        else wait_vm<0>();
        __syncthreads();  // everyone's copies landed; everyone finished stage kt-1
        if (kt + 2 < nk) issue(kt + 2);
        const unsigned char *As = smem + (kt % STAGES) * G::STAGE;
        const unsigned char *Bs = As + G::A_BYTES;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int c = 2 * kk + (lane >> 5);
            bf16x8 af[2], bfr[G::NT];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = wm * 64 + i * 32 + (lane & 31);
                af[i] = *(const bf16x8 *)(As + swz(r, c));
            }
#pragma unroll
            for (int j = 0; j < G::NT; ++j) {
                const int r = brow[j] + (lane & 31);
                bfr[j] = *(const bf16x8 *)(Bs + swz(r, c));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < G::NT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    }

    // epilogue: accumulator v of a 32x32 tile sits at row 8*(v/4) + 4*(lane/32) + v%4, column lane%32
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int row = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (row >= M) continue;
            if (EPI == EPI_SWIGLU) {
                constexpr int HJ = G::NT / 2;
#pragma unroll
                for (int j = 0; j < HJ; ++j) {
                    const int col = nb * (BN / 2) + wn * (BN / 4) + 32 * j + (lane & 31);
                    if (col >= N) continue;
                    const size_t idx = (size_t)row * N + col;
                    const float g = rho<bf16>(acc[i][j][v]), u = rho<bf16>(acc[i][j + HJ][v]);
                    out[idx] = from_f<bf16>(rho<bf16>(silu_f32(g)) * u);
                }
            } else {
#pragma unroll
                for (int j = 0; j < G::NT; ++j) {
                    const int col = nb * BN + brow[j] + (lane & 31);
                    if (col >= N) continue;
                    const size_t idx = (size_t)row * N + col;
                    const float a = acc[i][j][v];
                    out[idx] = from_f<bf16>(EPI == EPI_RESID ? to_f(res[idx]) + rho<bf16>(a) : a);
                }
            }
        }
    }
}

namespace {
template <int EPI, int BN>
hipError_t launch_g2(const bf16 *x, int M, int K, const bf16 *W, int N, const bf16 *res, bf16 *out, hipStream_t s) {
    using G = g2::Geo<BN>;
    const int cols = EPI == EPI_SWIGLU ? BN / 2 : BN;
    const dim3 grid((N + cols - 1) / cols, (M + g2::BM - 1) / g2::BM);
    const size_t lds = (size_t)g2::STAGES * G::STAGE;
    static bool attr = false;  // the kernel needs more than the default 64 KB of dynamic LDS
    if (!attr) {
        const hipError_t e = hipFuncSetAttribute((const void *)gemm_bf16_dma_kernel<EPI, BN>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr = true;
    }
    gemm_bf16_dma_kernel<EPI, BN><<<grid, 256, lds, s>>>(x, M, K, W, N, res, out);
    return hipGetLastError();
}
}  // namespace

bool gemm_dma_ok(int M, int K, int N) { return M > 16 && K % g2::BK == 0 && K > 0 && N > 0; }

hipError_t launch_gemm_dma(const void *x, int M, int K, const void *W, int N, int epi, const void *res, void *out,
                           hipStream_t s) {
    const bf16 *a = (const bf16 *)x, *w = (const bf16 *)W, *r = (const bf16 *)res;
    bf16 *o = (bf16 *)out;
    // 128 x 256 tiles when they still fill the 256 CUs, else 128 x 128
    const int mblocks = (M + g2::BM - 1) / g2::BM;
    const bool wide = (long)mblocks * ((epi == EPI_SWIGLU ? N / 128 : N / 256)) >= 256;
    if (epi == EPI_SWIGLU) return wide ? launch_g2<EPI_SWIGLU, 256>(a, M, K, w, N, r, o, s)
                                       : launch_g2<EPI_SWIGLU, 128>(a, M, K, w, N, r, o, s);
    if (epi == EPI_RESID) return wide ? launch_g2<EPI_RESID, 256>(a, M, K, w, N, r, o, s)
                                      : launch_g2<EPI_RESID, 128>(a, M, K, w, N, r, o, s);
    return wide ? launch_g2<EPI_STORE, 256>(a, M, K, w, N, r, o, s) : launch_g2<EPI_STORE, 128>(a, M, K, w, N, r, o, s);
}

}  // namespace q3
