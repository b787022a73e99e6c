// kernels_gemm.hip -- the MFMA projections of prefill (M > 16 rows): y = x . W^T with the
// fused epilogues of kernels_linear.hip ("maya2_mlx/backbone.py", forward: the fused q|k|v
// rows, o_proj + residual, fused gate|up rows + SwiGLU, down; the rounding points are those
// of epi_value there), for bf16 weights and for 8-bit affine group-quantised weights (codes
// q, bf16 scale s and bias b per 64 along K; w = s * q + b used in fp32, never rounded).
//
// Design for gfx950:
//  - v_mfma_f32_32x32x16_bf16 on block tiles of BM rows x BN weight rows, WM x WN waves, each
//    wave (BM/WM) x (BN/WN).  For SWIGLU a tile holds BN/2 gate rows and the BN/2 up rows of
//    the same outputs, and a wave holds the gate and up accumulators of the same columns.
//  - K steps of 64 flow through an ST-stage LDS ring filled by direct-to-LDS copies
//    (global_load_lds_dwordx4, 1 KB per instruction; no register staging): ST-1 stages are in
//    flight while one is consumed, one barrier per K step.
//  - LDS rows are 128 B (64 bf16; 64 B for 64 codes) with the 16-byte chunks XOR-swizzled by
//    the row (chunk ^ ((row >> 1) & 7) for 128-B rows, chunk ^ ((row >> 2) & 3) for 64-B rows),
//    so 16 lanes reading 16 consecutive rows at one chunk hit distinct banks.  A copy's lane
//    -> address map writes that layout directly.
//  - Tile shapes, the largest that still gives >= 192 tiles: 128 x 256 with 8 waves for gate|up
//    (T >= 512; 131 -> 121 us at T = 2048 against 256 x 128), 256 x 128 with 8 waves (q|k|v
//    at T = 2048), 128 x 128 with 8 waves (o_proj and down at T = 2048), else
//    128 x 64 (64 x 128 for SWIGLU, whose waves hold gate/up pairs) with 4 waves.  The
//    128 x 128 and 128 x 64 store/residual tiles split each K step between two groups of
//    64 x 64 waves (K groups, see Cfg), so a wave does twice the MFMAs per fragment read of a
//    32 x 64 wave and the block still has 8 (4) waves: o_proj at T = 2048 27.8 -> 26.8 us,
//    down 67.4 -> 61.8; at T = 512 down 44.3 -> 36.8, o_proj 18.4 -> 17.6.  Measured
//    against one 128 x 256 / 4-wave tiling at T = 2048: gate|up 148 -> 125 us, q|k|v 48 -> 40,
//    o_proj 40 -> 31; at T = 512 o_proj 54 -> 20 and down 101 -> 38.  8-bit weights: the
//    per-group fold (2 FMAs per accumulator element) costs about as many cycles as the group's
//    MFMAs, so 8 waves per CU let one wave's fold overlap another's MFMAs: 128 x 256 with 8
//    waves when it gives >= 192 tiles, then 128 x 128 (SwiGLU) or 64 x 128 with 8 waves, else
//    64 x 64 with 2 K groups of 4 waves.  Against the 4-wave 128 x 128 / 64 x 128 tilings
//    at T = 512: gate|up 96 -> 67 us, down 77 -> 60, o_proj 32 -> 24, q|k|v 32 -> 28.  A
//    stage's copies are padded with dummies to a multiple of the wave count (a wave's copies of
//    one round may then be of different kinds).
//  - 8-bit weights (one K step = one group): the codes (64 B per row) are copied to LDS like
//    the bf16 operand; the scale and bias words of the group arrive by 4-byte direct copies
//    (the aligned word holding groups 2i and 2i+1).  K is interleaved per lane so one 16-byte
//    read yields the codes of two MFMA steps; codes 0..255 are exact in bf16 (converted
//    through fp32).  Per group the MFMAs form P = x . q, and one more MFMA against a ones
//    operand forms S = sum of x over the group in the same register layout; the group then
//    folds as acc += s * P + b * S (the same sum regrouped, all fp32).
//  - EPI_QKV (bf16, 256 x 128 tiles: one head of 128 columns per tile): the q|k|v projection
//    with the per-head q/k RMSNorm, RoPE and the K/V cache write in the epilogue (qkv_epilogue).
//  - Rows past M and weight rows past N are clamped to the last valid row on load and
//    skipped on store.  K must be a multiple of 64 (of 128 for 8-bit weights).
#include "common.h"
#include "kernels.h"

namespace q3 {
namespace g2 {

// KG > 1: KG groups of WM x WN waves share each K step, group g taking its k-slices
// [g * 4 / KG, (g + 1) * 4 / KG) of the step's four 16-wide slices; group 0 adds the others'
// accumulators (through LDS, in group order) after the K loop and runs the epilogue.
template <int BM_, int BN_, int ST_, int WM_, int WN_, bool Q8_, int KG_ = 1> struct Cfg {
    static constexpr int BM = BM_, BN = BN_, ST = ST_, WM = WM_, WN = WN_, KG = KG_;
    static constexpr bool Q8 = Q8_;
    static constexpr int BK = 64, NWG = WM * WN, NW = NWG * KG, NTH = 64 * NW;
    static constexpr int RBA = 128, RBB = Q8 ? 64 : 128;  // LDS row bytes of A and of the weights
    static constexpr int A_BYTES = BM * RBA, B_BYTES = BN * RBB, SB_BYTES = Q8 ? BN * 8 : 0;
    static constexpr int STAGE = A_BYTES + B_BYTES + SB_BYTES;
    static constexpr int ACOP = A_BYTES / 1024, NBIG = (A_BYTES + B_BYTES) / 1024, NSMALL = SB_BYTES / 256;
    // copies per stage, padded to a multiple of the wave count with 4-byte dummy copies into a
    // junk LDS word (every wave then issues the same number of copies per stage, which its
    // vector-memory waits count on)
    static constexpr int OPS = (NBIG + NSMALL + NW - 1) / NW * NW, PAD = OPS - NBIG - NSMALL;
    static constexpr int PW = OPS / NW, APW = ACOP / NW, BPW = NBIG / NW;
    static constexpr int JUNK = PAD ? 256 : 0, LDS = ST * STAGE + JUNK;
    static constexpr int WTM = BM / WM, WTN = BN / WN, NI = WTM / 32, NT = WTN / 32;
    // bf16 tilings give every wave the same copies in every round; 8-bit ones may mix kinds in a
    // round (the kind is then chosen per copy), and their padding copies read the scale array
    static constexpr bool EVEN = ACOP % NW == 0 && NBIG % NW == 0;
    static_assert(EVEN || Q8, "bf16 row copies split evenly over the waves");
    static_assert(PAD == 0 || Q8, "only the scale/bias copies are padded");
    static_assert(NI >= 1 && NT >= 1, "wave tile at least 32 x 32");
    static_assert(KG == 1 || (4 % KG == 0 && (Q8 || (NI == 2 && NT == 2))), "K groups: bf16 64 x 64 wave tiles");
    static_assert(KG == 1 || (KG - 1) * NWG * 64 * NI * NT * 16 * 4 <= ST * STAGE, "group partials fit in the stages");
};

__device__ __forceinline__ int offA(int row, int c) { return row * 128 + ((c ^ ((row >> 1) & 7)) << 4); }
template <bool Q8> __device__ __forceinline__ int offB(int row, int c) {
    if (Q8) return row * 64 + ((c ^ ((row >> 2) & 3)) << 4);
    return offA(row, c);
}

// Weight row held by tile-local row r of weight block nb.
template <int EPI, int BN> __device__ __forceinline__ int w_row(int nb, int r, int N) {
    if (EPI == EPI_SWIGLU) {
        constexpr int H = BN / 2;
        const int n = nb * H + (r < H ? r : r - H);
        return (r < H ? 0 : N) + min(n, N - 1);
    }
    return min(nb * BN + r, N - 1);
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 4-byte direct-to-LDS copy: lane l's word lands at lds + 4 l.
__device__ __forceinline__ void dma4(const void *g, unsigned lds) {
    __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds)
                     : "memory", "m0");
}
#pragma clang diagnostic pop

}  // namespace g2

// The q|k|v epilogue of "maya2_mlx/backbone.py" (forward: the fused projection, per-head
// q/k RMSNorm with its two roundings, RoPE in fp32 on the table values with one rounding, the
// cache write), for a tile of BN = 128 = head_dim columns, i.e. one head: tile nb is q head nb
// (nb < H), k head nb - H, or v head nb - H - KV.  Each row's 128 columns sit in the two
// waves wn = 0, 1 of the same wm (64 each), so the row's sum of squares and each RoPE pair
// (c, c + 64) are completed through LDS with the partner wave.  With a bias (page 2's Qwen2
// switch) every value is rho(rho(x W^T) + b) first.
// The RoPE table words, norm weights and bias this lane needs, loaded before the K loop so the
// epilogue does not wait a memory round trip for them.
template <class C> struct QkvPre {
    static constexpr int RW = C::WTM;
    u32x4 cw[RW / 8], sw[RW / 8];
    float nw[C::NT], b[C::NT];
};
template <class C>
__device__ __forceinline__ void qkv_prefetch(QkvPre<C> &pre, const QkvEpi &qe, int M, int m0, int nb, int wm, int wn,
                                             int lane) {
    constexpr int RW = C::WTM;
    const int H = qe.H, KV = qe.KV;
    const bool isq = nb < H, isv = nb >= H + KV;
    const bf16 *bias = (const bf16 *)qe.bias;
    const bf16 *nw = isv ? nullptr : (const bf16 *)(isq ? qe.q_norm : qe.k_norm);
#pragma unroll
    for (int j = 0; j < C::NT; ++j) {
        const int col = wn * 64 + j * 32 + (lane & 31);
        pre.b[j] = bias ? to_f(bias[(size_t)nb * 128 + col]) : 0.f;
        pre.nw[j] = nw ? to_f(nw[col]) : 0.f;
    }
    if (isv) return;
    const bf16 *cs = (const bf16 *)qe.cos_t, *sn = (const bf16 *)qe.sin_t;
    const int c = wn * 64 + (lane & 7) * 8;
#pragma unroll
    for (int t = 0; t < RW / 8; ++t) {
        const int row = min(m0 + wm * RW + (lane >> 3) + 8 * t, M - 1), p = qe.p0 + row;
        pre.cw[t] = ld16(cs + (size_t)p * 128 + c);
        pre.sw[t] = ld16(sn + (size_t)p * 128 + c);
    }
}

template <class C>
__device__ __forceinline__ void qkv_epilogue(f32x16 (&acc)[C::NI][C::NT], const QkvPre<C> &pre, const QkvEpi &qe,
                                             unsigned char *smem, int M, int m0, int nb, int wm, int wn, int wave,
                                             int lane) {
    static_assert(C::BN == 128 && C::WN == 2 && C::NT == 2 && !C::Q8, "one head of 128 columns over two waves");
    constexpr int RW = C::WTM;                  // rows per wave
    constexpr int YP = 68;                      // exchange-buffer row (fp32 words; 16-byte aligned)
    constexpr int Y_BYTES = C::NW * RW * YP * 4, RED = RW * 33;
    static_assert(Y_BYTES + 2 * C::NW * RW * 4 <= C::ST * C::STAGE, "exchange buffers fit in the stages");
    static_assert(C::NW * RED * 4 <= Y_BYTES, "row partials fit under the exchange buffer");
    const int H = qe.H, KV = qe.KV;
    const bool isq = nb < H, isv = nb >= H + KV;
    const bool bias = qe.bias != nullptr;
    auto row_of = [&](int i, int v) { return i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); };  // in the wave
#pragma unroll
    for (int i = 0; i < C::NI; ++i)
#pragma unroll
        for (int j = 0; j < C::NT; ++j) {
            const float b = pre.b[j];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                float a = rho<bf16>(acc[i][j][v]);
                if (bias) a = rho<bf16>(a + b);
                acc[i][j][v] = a;
            }
        }
    __syncthreads();  // every wave is done with the last K step's LDS stage
    float *ybuf = (float *)smem;                   // [NW][RW][YP]; first the row partials [NW][RW][33]
    float *ssb = (float *)(smem + Y_BYTES);        // [NW][RW] half-row sums of squares
    float *rb = ssb + C::NW * RW;                  // [NW][RW] 1 / rms of the wave's rows
    const bool nw = !isv && (isq ? qe.q_norm : qe.k_norm) != nullptr;
    if (nw) {
        float *red = ybuf + wave * RED;
#pragma unroll
        for (int i = 0; i < C::NI; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                red[row_of(i, v) * 33 + (lane & 31)] = acc[i][0][v] * acc[i][0][v] + acc[i][1][v] * acc[i][1][v];
        // a wave's LDS accesses complete in order: lane r now sums row r of its own partials
        if (lane < RW) {
            float ss = 0.f;
#pragma unroll
            for (int t = 0; t < 32; ++t) ss += red[lane * 33 + t];
            ssb[wave * RW + lane] = ss;
        }
        __syncthreads();
        if (lane < RW) {
            const int partner = wm * C::WN + (wn ^ 1);
            const float ss = ssb[wave * RW + lane] + ssb[partner * RW + lane];
            rb[wave * RW + lane] = 1.0f / sqrtf(ss / 128.0f + qe.eps);
        }
        const float *w = pre.nw;
#pragma unroll
        for (int i = 0; i < C::NI; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float r = rb[wave * RW + row_of(i, v)];
#pragma unroll
                for (int j = 0; j < C::NT; ++j) acc[i][j][v] = rho<bf16>(w[j] * rho<bf16>(acc[i][j][v] * r));
            }
        __syncthreads();  // the row partials under the exchange buffer are consumed
    }
    // The wave's values go to LDS in the accumulator layout and come back as 8 consecutive
    // columns of one row per lane, so the RoPE table reads and the stores are 16 bytes wide; the
    // partner wave's region holds the other half (c +- 64) of each RoPE pair.
#pragma unroll
    for (int i = 0; i < C::NI; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v)
#pragma unroll
            for (int j = 0; j < C::NT; ++j) ybuf[(wave * RW + row_of(i, v)) * YP + j * 32 + (lane & 31)] = acc[i][j][v];
    __syncthreads();
    const int partner = wm * C::WN + (wn ^ 1), c8 = (lane & 7) * 8;
    bf16 *dst = isq ? (bf16 *)qe.q_out
                    : (bf16 *)(isv ? qe.vc : qe.kc) + (size_t)(nb - H - (isv ? KV : 0)) * qe.cap * 128;
#pragma unroll
    for (int t = 0; t < RW / 8; ++t) {
        const int rl = (lane >> 3) + 8 * t, row = m0 + wm * RW + rl;
        if (row >= M) continue;
        const int p = qe.p0 + row, c = wn * 64 + c8;
        const f32x4 *yo = (const f32x4 *)&ybuf[(wave * RW + rl) * YP + c8];
        float y[8], o[8];
        *(f32x4 *)&y[0] = yo[0];
        *(f32x4 *)&y[4] = yo[1];
        if (isv) {
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = y[e];
        } else {
            const f32x4 *yq = (const f32x4 *)&ybuf[(partner * RW + rl) * YP + c8];
            float yp[8], cv[8], sv[8];
            *(f32x4 *)&yp[0] = yq[0];
            *(f32x4 *)&yp[4] = yq[1];
            Vec<bf16>::expand(pre.cw[t], cv);
            Vec<bf16>::expand(pre.sw[t], sv);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = wn == 0 ? y[e] * cv[e] - yp[e] * sv[e] : y[e] * cv[e] + yp[e] * sv[e];
        }
        const size_t at = isq ? ((size_t)row * H + nb) * 128 + c : (size_t)p * 128 + c;
        *(u32x4 *)(dst + at) = u32x4{pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]), pack_bf2(o[4], o[5]), pack_bf2(o[6], o[7])};
    }
}

// W: bf16 weight rows, or (Q8) the u8 codes with their scale and bias arrays [rows][K/64].
template <int EPI, class C>
__global__ void __launch_bounds__(C::NTH) gemm_mfma_kernel(const bf16 *__restrict__ A, int M, int K,
                                                          const void *__restrict__ W, const bf16 *__restrict__ scale,
                                                          const bf16 *__restrict__ bias, int N,
                                                          const bf16 *res, bf16 *out,  // out may alias res
                                                          QkvEpi qe) {
    using namespace g2;
    static_assert(EPI != EPI_SWIGLU || C::NT % 2 == 0, "a SWIGLU wave holds gate and up tiles in pairs");
    extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = wave / C::NWG, wq = wave % C::NWG;  // K group; wave within the group
    const int wm = wq / C::WN, wn = wq % C::WN;
    const int m0 = blockIdx.y * C::BM, nb = blockIdx.x;
    static_assert(C::KG == 1 || EPI != EPI_QKV, "the q|k|v epilogue uses every wave");
    const int nk = K / C::BK, ng = K / 64;
    const unsigned lds0 = (unsigned)(uintptr_t)smem;

    // this wave's copies of one stage: op d = i * NW + wave, in the order A, weights, scale|bias
    auto issue = [&](int kt) {
        const int k0 = kt * C::BK;
        const unsigned st = lds0 + (kt % C::ST) * C::STAGE;
#pragma unroll
        for (int i = 0; i < C::PW; ++i) {
            const int d = i * C::NW + wave;
            if (C::EVEN ? i < C::APW : d < C::ACOP) {
                const int r = d * 8 + (lane >> 3), c = (lane & 7) ^ ((r >> 1) & 7);
                dma16(A + (size_t)min(m0 + r, M - 1) * K + k0 + c * 8, __builtin_amdgcn_readfirstlane(st + d * 1024));
            } else if (C::EVEN ? i < C::BPW : d < C::NBIG) {
                const int db = d - C::ACOP;
                if (C::Q8) {
                    const int r = db * 16 + (lane >> 2), c = (lane & 3) ^ ((r >> 2) & 3);
                    const uint8_t *src = (const uint8_t *)W + (size_t)w_row<EPI, C::BN>(nb, r, N) * K + k0 + c * 16;
                    dma16(src, __builtin_amdgcn_readfirstlane(st + d * 1024));
                } else {
                    const int r = db * 8 + (lane >> 3), c = (lane & 7) ^ ((r >> 1) & 7);
                    const bf16 *src = (const bf16 *)W + (size_t)w_row<EPI, C::BN>(nb, r, N) * K + k0 + c * 8;
                    dma16(src, __builtin_amdgcn_readfirstlane(st + d * 1024));
                }
            } else {
                const int sm = d - C::NBIG;  // 256-B word copies: scale, then bias, then padding
                if (C::PAD && sm >= C::NSMALL) {
                    dma4(scale, __builtin_amdgcn_readfirstlane(lds0 + C::ST * C::STAGE));
                } else {
                    const int part = sm % (C::BN / 64), which = sm / (C::BN / 64);
                    const int wr = w_row<EPI, C::BN>(nb, part * 64 + lane, N);
                    const bf16 *arr = which ? bias : scale;
                    dma4(arr + (size_t)wr * ng + (kt & ~1),
                         __builtin_amdgcn_readfirstlane(st + C::A_BYTES + C::B_BYTES + sm * 256));
                }
            }
        }
    };

    f32x16 acc[C::NI][C::NT];
#pragma unroll
    for (int i = 0; i < C::NI; ++i)
#pragma unroll
        for (int j = 0; j < C::NT; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    int brow[C::NT];  // tile-local weight rows of this wave's MFMA tiles
#pragma unroll
    for (int j = 0; j < C::NT; ++j) {
        if (EPI == EPI_SWIGLU) {
            constexpr int HJ = C::NT / 2;  // gate tiles, then the matching up tiles
            brow[j] = (j < HJ ? 0 : C::BN / 2) + wn * (C::WTN / 2) + 32 * (j % HJ);
        } else {
            brow[j] = wn * C::WTN + 32 * j;
        }
    }

    // EPI_RESID (bf16 weights): the residual words of this lane's outputs are loaded before the K
    // loop, so the epilogue does not wait a memory round trip for them (o_proj at T = 2048 33.5 ->
    // 29.5 us, down 69.7 -> 65.3).  Rows and columns are clamped in bounds; out may alias res (each
    // word is read and then written by the same lane).
    QkvPre<C> pre;
    if constexpr (EPI == EPI_QKV) qkv_prefetch<C>(pre, qe, M, m0, nb, wm, wn, lane);
    constexpr bool RPF = EPI == EPI_RESID && !C::Q8;
    uint32_t rv[RPF ? C::NI : 1][RPF ? 16 : 1][RPF ? C::NT : 1];
    if (RPF && kg == 0) {
        const uint16_t *r16 = (const uint16_t *)res;
#pragma unroll
        for (int i = 0; i < C::NI; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = min(m0 + wm * C::WTM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3), M - 1);
#pragma unroll
                for (int j = 0; j < C::NT; ++j) {
                    const int col = min(nb * C::BN + brow[j] + (lane & 31), N - 1);
                    rv[i][v][j] = r16[(size_t)row * N + col];
                }
            }
    }
#pragma unroll
    for (int s = 0; s < C::ST - 1; ++s)
        if (s < nk) issue(s);
    for (int kt = 0; kt < nk; ++kt) {
        constexpr int AHEAD = C::ST - 2;  // stages in flight beyond the one consumed
        const int rem = nk - 1 - kt;
        if (AHEAD >= 2 && rem >= 2) wait_vm<(AHEAD >= 2 ? 2 : 0) * C::PW>();
        else if (AHEAD >= 1 && rem >= 1) wait_vm<(AHEAD >= 1 ? 1 : 0) * C::PW>();
        else wait_vm<0>();
        __syncthreads();  // every wave's copies of stage kt landed; every wave finished kt-1
        if (kt + C::ST - 1 < nk) issue(kt + C::ST - 1);
        const unsigned char *As = smem + (kt % C::ST) * C::STAGE;
        const unsigned char *Bs = As + C::A_BYTES;
        if constexpr (!C::Q8 && C::NI == 2 && C::NT == 2) {
            // 64 x 64 per wave: all fragments of the K step are named up front and the schedule is
            // pinned to the reads of k-slice 0, then one MFMA per read of the later slices, so the
            // reads of slice kk+1 overlap the MFMAs of slice kk (left to itself the compiler reuses
            // one fragment set and waits on every read; gate|up at T = 2048 ~130 -> ~118 us)
            constexpr int NKK = C::BK / 16 / C::KG, RPK = C::NI + C::NT, MPK = C::NI * C::NT;
            bf16x8 af[NKK][C::NI], bfr[NKK][C::NT];
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const int c = 2 * (kg * NKK + kk) + (lane >> 5);
#pragma unroll
                for (int i = 0; i < C::NI; ++i)
                    af[kk][i] = *(const bf16x8 *)(As + offA(wm * C::WTM + i * 32 + (lane & 31), c));
#pragma unroll
                for (int j = 0; j < C::NT; ++j) bfr[kk][j] = *(const bf16x8 *)(Bs + offB<false>(brow[j] + (lane & 31), c));
            }
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
                for (int i = 0; i < C::NI; ++i)
#pragma unroll
                    for (int j = 0; j < C::NT; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk][i], bfr[kk][j], acc[i][j], 0, 0, 0);
            static_assert(MPK == RPK, "one read per MFMA");
            __builtin_amdgcn_sched_group_barrier(0x100, RPK, 0);  // DS reads of slice 0
#pragma unroll
            for (int r = 0; r < (NKK - 1) * RPK; ++r) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one DS read
            }
            __builtin_amdgcn_sched_group_barrier(0x008, MPK, 0);  // MFMAs of the last slice
        } else if (!C::Q8) {
#pragma unroll
            for (int kk = 0; kk < C::BK / 16; ++kk) {
                const int c = 2 * kk + (lane >> 5);
                bf16x8 af[C::NI], bfr[C::NT];
#pragma unroll
                for (int i = 0; i < C::NI; ++i)
                    af[i] = *(const bf16x8 *)(As + offA(wm * C::WTM + i * 32 + (lane & 31), c));
#pragma unroll
                for (int j = 0; j < C::NT; ++j) bfr[j] = *(const bf16x8 *)(Bs + offB<false>(brow[j] + (lane & 31), c));
#pragma unroll
                for (int i = 0; i < C::NI; ++i)
#pragma unroll
                    for (int j = 0; j < C::NT; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
            }
        } else {
            // MFMA step kk = 2p + e, lane half h: k = (2p + h) * 16 + 8 e + 0..7 of the group
            const int h = lane >> 5;
            const f32x16 zero = {};
            const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
            // K groups: group g takes the MFMA steps [g * SPG, (g + 1) * SPG) and folds its own
            // partial sums with the group's scale and bias (the fold is linear, so the groups' sums add)
            constexpr int SPG = 4 / C::KG;
            const int pb = C::KG == 1 ? 0 : (kg * SPG) >> 1;
            f32x16 part[C::NI][C::NT], xs[C::NI];
            u32x4 cw[C::NT];
#pragma unroll
            for (int q = 0; q < SPG; ++q) {
                const int p = pb + (q >> 1), e = SPG >= 2 ? (q & 1) : (kg & 1);
                if (SPG == 1 || (q & 1) == 0) {
#pragma unroll
                    for (int j = 0; j < C::NT; ++j)
                        cw[j] = *(const u32x4 *)(Bs + offB<true>(brow[j] + (lane & 31), 2 * p + h));
                }
                bf16x8 af[C::NI], bfr[C::NT];
#pragma unroll
                for (int i = 0; i < C::NI; ++i)
                    af[i] = *(const bf16x8 *)(As + offA(wm * C::WTM + i * 32 + (lane & 31), 2 * (2 * p + h) + e));
#pragma unroll
                for (int j = 0; j < C::NT; ++j)
                    bfr[j] = e ? codes8(cw[j][2], cw[j][3]) : codes8(cw[j][0], cw[j][1]);
#pragma unroll
                for (int i = 0; i < C::NI; ++i) {
#pragma unroll
                    for (int j = 0; j < C::NT; ++j)
                        part[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], q ? part[i][j] : zero, 0, 0, 0);
                    xs[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], ones, q ? xs[i] : zero, 0, 0, 0);
                }
            }
            const uint32_t *sw = (const uint32_t *)(Bs + C::B_BYTES), *bw = sw + C::BN;
            const int sh = (kt & 1) * 16;
#pragma unroll
            for (int j = 0; j < C::NT; ++j) {
                const int col = brow[j] + (lane & 31);
                const float sc = __uint_as_float((sw[col] >> sh) << 16), bi = __uint_as_float((bw[col] >> sh) << 16);
#pragma unroll
                for (int i = 0; i < C::NI; ++i)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[i][j][v] += sc * part[i][j][v] + bi * xs[i][v];
            }
        }
    }

    if constexpr (EPI == EPI_QKV) {
        qkv_epilogue<C>(acc, pre, qe, smem, M, m0, nb, wm, wn, wave, lane);
        return;
    }
    if constexpr (C::KG > 1) {
        // the groups' partial sums of the same outputs meet in LDS (the stages are free once every
        // wave has passed the last K step): group g > 0 stores, group 0 adds them in group order
        constexpr int E = C::NI * C::NT * 16;
        float *part = (float *)smem;  // [KG - 1][NWG][E][64]
        __syncthreads();
        if (kg > 0) {
            float *d = part + ((size_t)(kg - 1) * C::NWG + wq) * E * 64 + lane;
#pragma unroll
            for (int i = 0; i < C::NI; ++i)
#pragma unroll
                for (int j = 0; j < C::NT; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v) d[((i * C::NT + j) * 16 + v) * 64] = acc[i][j][v];
        }
        __syncthreads();
        if (kg > 0) return;
#pragma unroll
        for (int g = 1; g < C::KG; ++g) {
            const float *d = part + ((size_t)(g - 1) * C::NWG + wq) * E * 64 + lane;
#pragma unroll
            for (int i = 0; i < C::NI; ++i)
#pragma unroll
                for (int j = 0; j < C::NT; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[i][j][v] += d[((i * C::NT + j) * 16 + v) * 64];
        }
    }
    // epilogue: accumulator v of a 32x32 tile sits at row 8*(v/4) + 4*(lane/32) + v%4, column lane%32
#pragma unroll
    for (int i = 0; i < C::NI; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int row = m0 + wm * C::WTM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (row >= M) continue;
            if (EPI == EPI_SWIGLU) {
                constexpr int HJ = C::NT / 2;
#pragma unroll
                for (int j = 0; j < HJ; ++j) {
                    const int col = nb * (C::BN / 2) + wn * (C::WTN / 2) + 32 * j + (lane & 31);
                    if (col >= N) continue;
                    const size_t idx = (size_t)row * N + col;
                    const float g = rho<bf16>(acc[i][j][v]), u = rho<bf16>(acc[i][j + HJ][v]);
                    out[idx] = from_f<bf16>(rho<bf16>(silu_f32(g)) * u);
                }
            } else {
#pragma unroll
                for (int j = 0; j < C::NT; ++j) {
                    const int col = nb * C::BN + brow[j] + (lane & 31);
                    if (col >= N) continue;
                    const size_t idx = (size_t)row * N + col;
                    const float a = acc[i][j][v];
                    float r = 0.f;
                    if constexpr (RPF) r = __uint_as_float(rv[i][v][j] << 16);
                    else if (EPI == EPI_RESID) r = to_f(res[idx]);
                    out[idx] = from_f<bf16>(EPI == EPI_RESID ? r + rho<bf16>(a) : a);
                }
            }
        }
    }
}

namespace {
typedef g2::Cfg<256, 128, 3, 4, 2, false> Wide;    // 8 waves, 64 x 64 per wave, 144 KB LDS
typedef g2::Cfg<128, 256, 3, 2, 4, false> WideN;   // 8 waves, 64 x 64 per wave, 144 KB LDS (gate|up)
typedef g2::Cfg<128, 128, 4, 4, 2, false> Mid;     // 8 waves, 32 x 64 per wave, 128 KB LDS
typedef g2::Cfg<128, 128, 4, 2, 2, false, 2> MidK; // 8 waves: 2 K groups of 4 waves, 64 x 64 per wave, 128 KB LDS
typedef g2::Cfg<128, 64, 4, 2, 1, false, 2> SmallNK;  // 4 waves: 2 K groups of 2 waves, 64 x 64 per wave, 96 KB LDS
typedef g2::Cfg<64, 128, 4, 2, 2, false> SmallM;   // 4 waves, 32 x 64 per wave, 96 KB LDS
typedef g2::Cfg<128, 128, 4, 2, 2, true> Quant;    // 4 waves, 100 KB LDS
typedef g2::Cfg<64, 128, 4, 2, 2, true> QuantS;    // 4 waves, 68 KB LDS
typedef g2::Cfg<128, 256, 3, 2, 4, true> QuantW;   // 8 waves, 64 x 64 per wave, 102 KB LDS
typedef g2::Cfg<64, 128, 4, 2, 4, true> QuantS8;   // 8 waves, 32 x 32 per wave, 68 KB LDS
// 8 waves: 2 K groups of 4, 32 x 32 per wave, 50 KB LDS.  At T = 512 (one tile per CU) the 8-bit
// prefill took 5.33 ms with 4 waves (one group), 5.13 with 2 groups, 5.6 with 4 groups; 2 groups of
// 8 waves for the 64 x 128 tiling (q|k|v) 28 -> 31.5 us, of 4 waves of 32 x 64 28 -> 30.6 us; 2-wave
// groups of 32 x 64 wave tiles for 64 x 64 5.6 ms
// (2 groups) and 6.3 (4), interleaved runs on one box
typedef g2::Cfg<64, 64, 4, 2, 2, true, 2> QuantTK;

// Output tiles of a BM x BN weight-row tiling (a SWIGLU tile covers BN/2 outputs).
template <class C> long tiles(int M, int N, int epi) {
    const long cols = epi == EPI_SWIGLU ? C::BN / 2 : C::BN;
    return (long)((M + C::BM - 1) / C::BM) * ((N + cols - 1) / cols);
}

template <int EPI, class C>
hipError_t launch_c(const bf16 *x, int M, int K, const void *W, const bf16 *sc, const bf16 *bi, int N, const bf16 *res,
                    bf16 *out, hipStream_t s, const QkvEpi &qe = QkvEpi()) {
    const int cols = EPI == EPI_SWIGLU ? C::BN / 2 : C::BN;
    const dim3 grid((N + cols - 1) / cols, (M + C::BM - 1) / C::BM);
    const size_t lds = (size_t)C::LDS;
    static bool attr = false;  // more than the default 64 KB of dynamic LDS
    if (!attr) {
        const hipError_t e = hipFuncSetAttribute((const void *)gemm_mfma_kernel<EPI, C>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr = true;
    }
    gemm_mfma_kernel<EPI, C><<<grid, C::NTH, lds, s>>>(x, M, K, W, sc, bi, N, res, out, qe);
    return hipGetLastError();
}

template <class C>
hipError_t launch_e(int epi, const bf16 *x, int M, int K, const void *W, const bf16 *sc, const bf16 *bi, int N,
                    const bf16 *r, bf16 *o, hipStream_t s) {
    if (epi == EPI_SWIGLU) return launch_c<EPI_SWIGLU, C>(x, M, K, W, sc, bi, N, r, o, s);
    if (epi == EPI_RESID) return launch_c<EPI_RESID, C>(x, M, K, W, sc, bi, N, r, o, s);
    return launch_c<EPI_STORE, C>(x, M, K, W, sc, bi, N, r, o, s);
}
// the store and residual epilogues only (tilings whose waves hold single 32-column tiles)
template <class C>
hipError_t launch_sr(int epi, const bf16 *x, int M, int K, const void *W, const bf16 *sc, const bf16 *bi, int N,
                     const bf16 *r, bf16 *o, hipStream_t s) {
    if (epi == EPI_RESID) return launch_c<EPI_RESID, C>(x, M, K, W, sc, bi, N, r, o, s);
    return launch_c<EPI_STORE, C>(x, M, K, W, sc, bi, N, r, o, s);
}
}  // namespace

bool gemm_dma_ok(int M, int K, int N) { return M > 16 && K % 64 == 0 && K > 0 && N > 0; }

hipError_t launch_gemm_dma(const void *x, int M, int K, const void *W, int N, int epi, const void *res, void *out,
                           hipStream_t s) {
    const bf16 *a = (const bf16 *)x, *r = (const bf16 *)res;
    bf16 *o = (bf16 *)out;
    if (epi == EPI_SWIGLU && tiles<WideN>(M, N, epi) >= 192)
        return launch_c<EPI_SWIGLU, WideN>(a, M, K, W, nullptr, nullptr, N, r, o, s);
    if (tiles<Wide>(M, N, epi) >= 192) return launch_e<Wide>(epi, a, M, K, W, nullptr, nullptr, N, r, o, s);
    if (epi == EPI_SWIGLU) {
        if (tiles<Mid>(M, N, epi) >= 192) return launch_c<EPI_SWIGLU, Mid>(a, M, K, W, nullptr, nullptr, N, r, o, s);
        return launch_c<EPI_SWIGLU, SmallM>(a, M, K, W, nullptr, nullptr, N, r, o, s);
    }
    if (tiles<MidK>(M, N, epi) >= 192) return launch_sr<MidK>(epi, a, M, K, W, nullptr, nullptr, N, r, o, s);
    return launch_sr<SmallNK>(epi, a, M, K, W, nullptr, nullptr, N, r, o, s);
}

bool gemm_qkv_fused_ok(int M, int K, int H, int KV, int D) {
    return D == 128 && gemm_dma_ok(M, K, (H + 2 * KV) * D) && tiles<Wide>(M, (H + 2 * KV) * D, EPI_STORE) >= 192;
}

hipError_t launch_gemm_qkv_fused(const void *x, int M, int K, const void *W, const QkvEpi &qe, hipStream_t s) {
    const int N = (qe.H + 2 * qe.KV) * 128;
    return launch_c<EPI_QKV, Wide>((const bf16 *)x, M, K, W, nullptr, nullptr, N, nullptr, nullptr, s, qe);
}

bool gemm_q8_dma_ok(int M, int K, int N, const void *scale, const void *bias) {
    return M > 16 && K % 128 == 0 && K > 0 && N > 0 && ((uintptr_t)scale & 3) == 0 && ((uintptr_t)bias & 3) == 0;
}

hipError_t launch_gemm_q8_dma(const void *x, int M, int K, const uint8_t *codes, const void *scale, const void *bias,
                              int N, int epi, const void *res, void *out, hipStream_t s) {
    const bf16 *a = (const bf16 *)x, *sc = (const bf16 *)scale, *bi = (const bf16 *)bias, *r = (const bf16 *)res;
    bf16 *o = (bf16 *)out;
    if (epi == EPI_SWIGLU) {
        if (tiles<QuantW>(M, N, epi) >= 192) return launch_c<EPI_SWIGLU, QuantW>(a, M, K, codes, sc, bi, N, r, o, s);
        if (tiles<Quant>(M, N, epi) >= 192) return launch_c<EPI_SWIGLU, Quant>(a, M, K, codes, sc, bi, N, r, o, s);
        return launch_c<EPI_SWIGLU, QuantS>(a, M, K, codes, sc, bi, N, r, o, s);
    }
    if (tiles<QuantW>(M, N, epi) >= 192) return launch_sr<QuantW>(epi, a, M, K, codes, sc, bi, N, r, o, s);
    if (tiles<QuantS8>(M, N, epi) >= 192) return launch_sr<QuantS8>(epi, a, M, K, codes, sc, bi, N, r, o, s);
    return launch_sr<QuantTK>(epi, a, M, K, codes, sc, bi, N, r, o, s);
}

}  // namespace q3
