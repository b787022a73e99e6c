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
//  2. moe_topk_kernel: one wave per token does softmax, k selection rounds (a DPP
//     maximum, then ballots in expert order for the lowest index holding it) and
//     the renormalisation;
//  3. moe_sort_kernel: stable counting sort of the T*k (token, slot) rows by
//     expert in one block (LDS counts, a wave scan, then each chunk of 256 rows
//     ranked against the rows before it), giving per-expert row ranges, the
//     sorted-to-row permutation, its inverse and the list of experts that received
//     rows;
//  4. moe_expert_kernel: grid (wave group, active expert); each wave streams
//     weight rows of its expert (the gate/up pair of one output in the first
//     pass, four output rows in the second) once per group of 8 routed rows, so
//     every hit expert's weights are read from HBM once for up to 8 tokens;
//  5. moe_combine_kernel: out[t] = rho(sum_s rho(y[t,s] * w[t,s])), slot order,
//     one thread per output element.
// One token (T == 1, the decode step) takes three launches instead: the router projection
// (with the post-attention RMSNorm in its prologue when the caller passes the norm weight),
// moe_gu1_kernel (every block repeats the softmax/top-k of its token from the logits and
// streams the gate|up rows of its slot's expert) and moe_down1_kernel (down rows of every
// slot for four outputs per block, then the weighted slot sum in slot order).
// 8-bit weights (bf16 model; the quantised gate Linear and QuantizedSwitchLinear experts of
// qwen3-moe.ts): the router goes through the 8-bit projection kernels and
// moe_expert_q8_kernel replaces step 4 with the same work mapping, a lane taking 16 codes
// per weight row per step and folding each group as s * (x . q) + b * sum(x) in fp32
// (kernels_q8.hip's format: groups of 64 along the input axis).
#include <math.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "moe_route.h"

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
// (select_topk and softmax_inplace: moe_route.h)
// The token's E logits as fp32, v[i] for expert lane + 64 i (-inf past E), then their softmax.
template <typename T, int EPL>
__device__ __forceinline__ void load_logits(const T *l, int E, int lane, float (&v)[EPL]) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E ? to_f(l[e]) : -INFINITY;
    }
}
template <typename T, int EPL>
__device__ __forceinline__ void softmax_probs(const T *l, int E, int lane, float (&v)[EPL]) {
    load_logits<T, EPL>(l, E, lane, v);
    softmax_inplace<T, EPL>(E, lane, v);
}

template <typename T>
__device__ __forceinline__ void write_routing(int t, int k, int norm, const float *psel, const int *isel,
                                              int32_t *__restrict__ idx, T *__restrict__ wout) {
    float den = 0.f;
    for (int s = 0; s < k; ++s) den += psel[s];
    const float denr = rho<T>(den);
    for (int s = 0; s < k; ++s) {
        idx[(size_t)t * k + s] = isel[s];
        wout[(size_t)t * k + s] = from_f<T>(norm ? psel[s] / denr : psel[s]);
    }
}

template <typename T>
__global__ void __launch_bounds__(64) moe_topk_kernel(const T *__restrict__ logits, int E, int k, int norm,
                                                      int32_t *__restrict__ idx, T *__restrict__ wout) {
    constexpr int EPL = 4;  // experts per lane (E <= 256)
    const int t = blockIdx.x, lane = threadIdx.x;
    float v[EPL];
    softmax_probs<T, EPL>(logits + (size_t)t * E, E, lane, v);
    float psel[16];
    int isel[16];
    select_topk<EPL>(v, E, k, lane, psel, isel);
    if (lane == 0) write_routing<T>(t, k, norm, psel, isel, idx, wout);
}

// ------------------------------------------------------------ stable counting sort by expert
// One block of 256 threads, E <= 256.  Rows keep their order within an expert.
__global__ void __launch_bounds__(256) moe_sort_kernel(const int32_t *__restrict__ idx, int rows, int E,
                                                       int32_t *__restrict__ offsets, int32_t *__restrict__ perm,
                                                       int32_t *__restrict__ inv, int32_t *__restrict__ active) {
    __shared__ int cnt[256], run[256], ch[256];
    const int tid = threadIdx.x;
    cnt[tid] = 0;
    __syncthreads();
    for (int r = tid; r < rows; r += 256) atomicAdd(&cnt[idx[r]], 1);
    __syncthreads();
    if (tid < 64) {  // exclusive scans of the counts and of the hit flags, four experts per lane
        int c[4], f[4], sc = 0, sf = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = 4 * tid + q;
            c[q] = e < E ? cnt[e] : 0;
            f[q] = c[q] > 0;
            sc += c[q];
            sf += f[q];
        }
        int ic = sc, jf = sf;  // inclusive prefix over lanes
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int uc = __shfl_up(ic, o, 64), uf = __shfl_up(jf, o, 64);
            if (tid >= o) {
                ic += uc;
                jf += uf;
            }
        }
        int pc = ic - sc, pf = jf - sf;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = 4 * tid + q;
            if (e < E) {
                run[e] = pc;
                offsets[e] = pc;
                if (f[q]) active[1 + pf] = e;
            }
            pc += c[q];
            pf += f[q];
        }
        if (tid == 63) {
            offsets[E] = ic;
            active[0] = jf;
        }
    }
    __syncthreads();
    for (int base = 0; base < rows; base += 256) {
        const int r = base + tid;
        const int e = r < rows ? idx[r] : -1;
        ch[tid] = e;
        __syncthreads();
        int pos = 0;
        if (r < rows) {
            int rank = 0;
            for (int j = 0; j < tid; ++j) rank += ch[j] == e;
            pos = run[e] + rank;
            perm[pos] = r;
            inv[r] = pos;
        }
        __syncthreads();  // every row of the chunk has read run[]
        if (r < rows) atomicAdd(&run[e], 1);
        __syncthreads();
    }
}

// ------------------------------------------------------------ grouped expert projections
// PASS 0: m[i] = swiglu(x[row(i)] . Wgu_e^T)  (Wgu_e [2*Ie][hid], output Ie columns)
// PASS 1: y[i] = rho(m[i] . Wd_e^T)           (Wd_e [hid][Ie], output hid columns)
// i runs over the sorted rows of expert e; row(i) = perm[i] / k for PASS 0.  A wave streams
// NR weight rows together: the gate and up rows of one output (PASS 0), or four outputs
// (PASS 1, whose rows are short: Ie values).
template <typename T, int PASS>
__global__ void __launch_bounds__(256) moe_expert_kernel(const T *__restrict__ xin, const T *__restrict__ W,
                                                         int K, int N, int k, const int32_t *__restrict__ offsets,
                                                         const int32_t *__restrict__ perm,
                                                         const int32_t *__restrict__ active, T *__restrict__ out) {
    constexpr int VN = Vec<T>::N;
    constexpr int MR = 8;
    constexpr int NR = PASS == 0 ? 2 : 4;
    const int slot = blockIdx.y;
    if (slot >= active[0]) return;
    const int e = active[1 + slot];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n0 = PASS == 0 ? blockIdx.x * 4 + wave : (blockIdx.x * 4 + wave) * NR;
    if (n0 >= N) return;
    const int r0 = offsets[e], r1 = offsets[e + 1];
    const size_t wrows = PASS == 0 ? 2 * (size_t)N : (size_t)N;
    const T *We = W + (size_t)e * wrows * K;
    const T *wr[NR];
#pragma unroll
    for (int q = 0; q < NR; ++q) wr[q] = We + (size_t)(PASS == 0 ? n0 + q * N : min(n0 + q, N - 1)) * K;
    const int nc = K / VN;
    for (int rb = r0; rb < r1; rb += MR) {
        const int nr = min(MR, r1 - rb);
        const T *xr[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const int i = rb + min(m, nr - 1);
            xr[m] = PASS == 0 ? xin + (size_t)(perm[i] / k) * K : xin + (size_t)i * K;
        }
        float a[NR][MR];
#pragma unroll
        for (int q = 0; q < NR; ++q)
#pragma unroll
            for (int m = 0; m < MR; ++m) a[q][m] = 0.f;
        for (int c = lane; c < nc; c += 64) {
            u32x4 wv[NR];
#pragma unroll
            for (int q = 0; q < NR; ++q) wv[q] = ld_stream(wr[q] + (size_t)c * VN);
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                if (m < nr) {
                    const u32x4 xv = ld16(xr[m] + (size_t)c * VN);
#pragma unroll
                    for (int q = 0; q < NR; ++q) a[q][m] = dot16<T>(wv[q], xv, a[q][m]);
                }
            }
        }
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            if (m < nr) {
                if (PASS == 0) {
                    const float s0 = wave_sum(a[0][m]), s1 = wave_sum(a[1][m]);
                    if (lane == 0) out[(size_t)(rb + m) * N + n0] = from_f<T>(rho<T>(silu_f32(rho<T>(s0))) * rho<T>(s1));
                } else {
#pragma unroll
                    for (int q = 0; q < NR; ++q) {
                        const float sq = wave_sum(a[q][m]);
                        if (lane == 0 && n0 + q < N) out[(size_t)(rb + m) * N + n0 + q] = from_f<T>(sq);
                    }
                }
            }
        }
    }
}

// The 8-bit form of moe_expert_kernel (bf16 activations): codes [E][rows][K] u8, scale and
// bias [E][rows][K/64] bf16; chunk c of a row is codes 16c..16c+15, in group c / 4.
template <int PASS>
__global__ void __launch_bounds__(256) moe_expert_q8_kernel(const bf16 *__restrict__ xin,
                                                            const uint8_t *__restrict__ codes,
                                                            const bf16 *__restrict__ scale,
                                                            const bf16 *__restrict__ bias, int K, int N, int k,
                                                            const int32_t *__restrict__ offsets,
                                                            const int32_t *__restrict__ perm,
                                                            const int32_t *__restrict__ active, bf16 *__restrict__ out) {
    constexpr int MR = 8;
    constexpr int NR = PASS == 0 ? 2 : 4;
    const int slot = blockIdx.y;
    if (slot >= active[0]) return;
    const int e = active[1 + slot];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n0 = PASS == 0 ? blockIdx.x * 4 + wave : (blockIdx.x * 4 + wave) * NR;
    if (n0 >= N) return;
    const int r0 = offsets[e], r1 = offsets[e + 1];
    const size_t wrows = PASS == 0 ? 2 * (size_t)N : (size_t)N;
    const int ng = K / 64, nc = K / 16;
    size_t row[NR];
#pragma unroll
    for (int q = 0; q < NR; ++q) row[q] = (size_t)e * wrows + (PASS == 0 ? n0 + q * N : min(n0 + q, N - 1));
    for (int rb = r0; rb < r1; rb += MR) {
        const int nr = min(MR, r1 - rb);
        const bf16 *xr[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const int i = rb + min(m, nr - 1);
            xr[m] = PASS == 0 ? xin + (size_t)(perm[i] / k) * K : xin + (size_t)i * K;
        }
        float a[NR][MR];
#pragma unroll
        for (int q = 0; q < NR; ++q)
#pragma unroll
            for (int m = 0; m < MR; ++m) a[q][m] = 0.f;
        for (int c = lane; c < nc; c += 64) {
            u32x4 cw[NR];
            float sc[NR], bi[NR];
#pragma unroll
            for (int q = 0; q < NR; ++q) {
                cw[q] = ld_stream(codes + row[q] * K + (size_t)c * 16);
                sc[q] = to_f(scale[row[q] * ng + (c >> 2)]);
                bi[q] = to_f(bias[row[q] * ng + (c >> 2)]);
            }
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                if (m < nr) {
                    float xf[16];
                    const bf16 *xp = xr[m] + (size_t)c * 16;
                    Vec<bf16>::expand(ld16(xp), xf);
                    Vec<bf16>::expand(ld16(xp + 8), xf + 8);
                    float xs = 0.f;
#pragma unroll
                    for (int i = 0; i < 16; ++i) xs += xf[i];
#pragma unroll
                    for (int q = 0; q < NR; ++q) a[q][m] += sc[q] * dot16_q8(cw[q], xf) + bi[q] * xs;
                }
            }
        }
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            if (m < nr) {
                if (PASS == 0) {
                    const float s0 = wave_sum(a[0][m]), s1 = wave_sum(a[1][m]);
                    if (lane == 0)
                        out[(size_t)(rb + m) * N + n0] = from_f<bf16>(rho<bf16>(silu_f32(rho<bf16>(s0))) * rho<bf16>(s1));
                } else {
#pragma unroll
                    for (int q = 0; q < NR; ++q) {
                        const float sq = wave_sum(a[q][m]);
                        if (lane == 0 && n0 + q < N) out[(size_t)(rb + m) * N + n0 + q] = from_f<bf16>(sq);
                    }
                }
            }
        }
    }
}

// MFMA form of moe_expert_kernel for bf16 when K % 256 == 0 (v_mfma_f32_16x16x32_bf16, as in
// kernels_linear.hip's gemv_mfma_kernel): block (16 outputs, active expert) with 8 waves, each
// a K/8 slice; A = up to 16 routed rows of the expert (lane i: row i % 16, k 8 (i / 16) ..),
// B = 16 weight rows (the gate and the up rows in PASS 0), so each weight chunk is loaded once
// per group of 16 rows and meets all of them in one MFMA.  The 8 partial tiles are summed in
// LDS in wave order; wave 0 applies the epilogue of the scalar kernel.
template <int PASS>
__global__ void __launch_bounds__(512) moe_expert_mfma_kernel(const bf16 *__restrict__ xin, const bf16 *__restrict__ W,
                                                              int K, int N, int k, const int32_t *__restrict__ offsets,
                                                              const int32_t *__restrict__ perm,
                                                              const int32_t *__restrict__ active,
                                                              bf16 *__restrict__ out) {
    constexpr int NWV = 8, U = 8;
    constexpr int NT = PASS == 0 ? 2 : 1;  // gate and up tiles
    __shared__ f32x4 part[NWV - 1][NT][64];
    const int slot = blockIdx.y;
    if (slot >= active[0]) return;  // uniform over the block
    const int e = active[1 + slot];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n0 = blockIdx.x * 16, r = lane & 15, h = lane >> 4;
    const int r0 = offsets[e], r1 = offsets[e + 1];
    const size_t wrows = PASS == 0 ? 2 * (size_t)N : (size_t)N;
    const bf16 *wr[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) wr[t] = W + ((size_t)e * wrows + (size_t)t * N + min(n0 + r, N - 1)) * K + 8 * h;
    const int ks = K / NWV, k0 = wave * ks;  // this wave's K slice, a multiple of 32
    for (int rb = r0; rb < r1; rb += 16) {
        const int i = rb + min(r, r1 - 1 - rb);  // rows past the expert's last repeat it (not stored)
        const bf16 *xr = (PASS == 0 ? xin + (size_t)(perm[i] / k) * K : xin + (size_t)i * K) + 8 * h;
        f32x4 acc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int kb = k0; kb < k0 + ks; kb += 32 * U) {
            u32x4 wv[NT][U], xv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int kk = kb + 32 * u;
                const bool ok = kk < k0 + ks;
#pragma unroll
                for (int t = 0; t < NT; ++t) wv[t][u] = ok ? ld_stream(wr[t] + kk) : u32x4{0, 0, 0, 0};
                xv[u] = ok ? ld16(xr + kk) : u32x4{0, 0, 0, 0};
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
        if (wave == 0 && n0 + r < N) {
#pragma unroll
            for (int w = 0; w < NWV - 1; ++w)
#pragma unroll
                for (int t = 0; t < NT; ++t) acc[t] += part[w][t][lane];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = rb + 4 * h + j;  // C element j of lane: row 4 (lane / 16) + j, output lane % 16
                if (row >= r1) continue;
                const float v = PASS == 0 ? rho<bf16>(silu_f32(rho<bf16>(acc[0][j]))) * rho<bf16>(acc[NT - 1][j])
                                          : acc[0][j];
                out[(size_t)row * N + n0 + r] = from_f<bf16>(v);
            }
        }
        __syncthreads();  // part[] is rewritten by the next group
    }
}

// The 8-bit form (K % 256 == 0; 4 waves, each a K/4 slice of whole groups of 64).  A group is
// two MFMA steps; lane (r, h) takes codes 16 h .. 16 h + 15 of the group (one 16-byte load),
// the first 8 in the first step and the rest in the second, and the activations of the same
// k: the steps cover k = 16 h + 0..7 and 16 h + 8..15, all 64 between them.  Codes are exact
// in bf16.  Per group P = x . q (gate and up tiles) and S = sum of x (an MFMA against ones, in
// the same register layout) fold as acc += s P + b S with the scale and bias of the lane's
// weight row, all fp32.
template <int PASS>
__global__ void __launch_bounds__(256) moe_expert_q8_mfma_kernel(const bf16 *__restrict__ xin,
                                                                 const uint8_t *__restrict__ codes,
                                                                 const bf16 *__restrict__ scale,
                                                                 const bf16 *__restrict__ bias, int K, int N, int k,
                                                                 const int32_t *__restrict__ offsets,
                                                                 const int32_t *__restrict__ perm,
                                                                 const int32_t *__restrict__ active,
                                                                 bf16 *__restrict__ out) {
    constexpr int NWV = 4, U = 4;  // groups in flight per lane
    constexpr int NT = PASS == 0 ? 2 : 1;
    __shared__ f32x4 part[NWV - 1][NT][64];
    const int slot = blockIdx.y;
    if (slot >= active[0]) return;  // uniform over the block
    const int e = active[1 + slot];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n0 = blockIdx.x * 16, r = lane & 15, h = lane >> 4;
    const int r0 = offsets[e], r1 = offsets[e + 1];
    const size_t wrows = PASS == 0 ? 2 * (size_t)N : (size_t)N;
    const int ng = K / 64;
    size_t wrow[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) wrow[t] = (size_t)e * wrows + (size_t)t * N + min(n0 + r, N - 1);
    const int gs = ng / NWV, g0 = wave * gs;  // this wave's groups
    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    for (int rb = r0; rb < r1; rb += 16) {
        const int i = rb + min(r, r1 - 1 - rb);
        const bf16 *xr = (PASS == 0 ? xin + (size_t)(perm[i] / k) * K : xin + (size_t)i * K) + 16 * h;
        f32x4 acc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = zero;
        for (int gb = g0; gb < g0 + gs; gb += U) {
            u32x4 cv[NT][U], xa[U], xb[U];
            float sv[NT][U], bv[NT][U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int g = gb + u;
                const bool ok = g < g0 + gs;
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    cv[t][u] = ok ? ld_stream(codes + wrow[t] * K + (size_t)g * 64 + 16 * h) : u32x4{0, 0, 0, 0};
                    sv[t][u] = ok ? to_f(scale[wrow[t] * ng + g]) : 0.f;
                    bv[t][u] = ok ? to_f(bias[wrow[t] * ng + g]) : 0.f;
                }
                xa[u] = ok ? ld16(xr + (size_t)g * 64) : u32x4{0, 0, 0, 0};
                xb[u] = ok ? ld16(xr + (size_t)g * 64 + 8) : u32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bf16x8 a0 = __builtin_bit_cast(bf16x8, xa[u]), a1 = __builtin_bit_cast(bf16x8, xb[u]);
                f32x4 S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, ones, zero, 0, 0, 0);
                S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, ones, S, 0, 0, 0);
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    f32x4 P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, codes8(cv[t][u][0], cv[t][u][1]), zero, 0, 0, 0);
                    P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, codes8(cv[t][u][2], cv[t][u][3]), P, 0, 0, 0);
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[t][j] += sv[t][u] * P[j] + bv[t][u] * S[j];
                }
            }
        }
        if (wave > 0)
#pragma unroll
            for (int t = 0; t < NT; ++t) part[wave - 1][t][lane] = acc[t];
        __syncthreads();
        if (wave == 0 && n0 + r < N) {
#pragma unroll
            for (int w = 0; w < NWV - 1; ++w)
#pragma unroll
                for (int t = 0; t < NT; ++t) acc[t] += part[w][t][lane];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = rb + 4 * h + j;
                if (row >= r1) continue;
                const float v = PASS == 0 ? rho<bf16>(silu_f32(rho<bf16>(acc[0][j]))) * rho<bf16>(acc[NT - 1][j])
                                          : acc[0][j];
                out[(size_t)row * N + n0 + r] = from_f<bf16>(v);
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------ one token (T == 1)
// acc[q] += W_q . x over K inputs: NR weight rows in storage type T, U 16-byte chunks per lane
// in flight per row before any arithmetic; x in LDS or global memory.
template <typename T, int NR, int U>
__device__ __forceinline__ void rows_dot(const T *const (&w)[NR], const T *x, int K, int lane, float (&acc)[NR]) {
    constexpr int VN = Vec<T>::N;
    const int nc = K / VN;
    for (int c0 = 0; c0 < nc; c0 += 64 * U) {
        u32x4 wv[U][NR];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + lane + 64 * u;
#pragma unroll
            for (int q = 0; q < NR; ++q) wv[u][q] = c < nc ? ld_stream(w[q] + (size_t)c * VN) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + lane + 64 * u;
            if (c < nc) {
                const u32x4 xv = ld16(x + (size_t)c * VN);
#pragma unroll
                for (int q = 0; q < NR; ++q) acc[q] = dot16<T>(wv[u][q], xv, acc[q]);
            }
        }
    }
}

// The 8-bit form: rows of u8 codes with bf16 scale and bias per 64 codes; chunk c is codes
// 16c..16c+15 in group c / 4; x bf16.
template <int NR, int U>
__device__ __forceinline__ void rows_dot_q8(const uint8_t *const (&w)[NR], const bf16 *const (&sc)[NR],
                                            const bf16 *const (&bi)[NR], const bf16 *x, int K, int lane,
                                            float (&acc)[NR]) {
    const int nc = K / 16;
    for (int c0 = 0; c0 < nc; c0 += 64 * U) {
        u32x4 wv[U][NR];
        float sv[U][NR], bv[U][NR];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + lane + 64 * u;
#pragma unroll
            for (int q = 0; q < NR; ++q) {
                const bool ok = c < nc;
                wv[u][q] = ok ? ld_stream(w[q] + (size_t)c * 16) : u32x4{0, 0, 0, 0};
                sv[u][q] = ok ? to_f(sc[q][c >> 2]) : 0.f;
                bv[u][q] = ok ? to_f(bi[q][c >> 2]) : 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + lane + 64 * u;
            if (c < nc) {
                float xf[16];
                Vec<bf16>::expand(ld16(x + (size_t)c * 16), xf);
                Vec<bf16>::expand(ld16(x + (size_t)c * 16 + 8), xf + 8);
                float xs = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i) xs += xf[i];
#pragma unroll
                for (int q = 0; q < NR; ++q) acc[q] += sv[u][q] * dot16_q8(wv[u][q], xf) + bv[u][q] * xs;
            }
        }
    }
}

// grid (ceil(Ie / 4), k), 256 threads, hid * sizeof(T) bytes of dynamic LDS.  x: the hidden
// row, normalised here with nw (RMSNorm, eps) or, with nw == NULL, already normalised.
// Every block ranks the E logits with the code of moe_topk_kernel, so all blocks agree;
// block (0, 0) writes idx / wsel.  m [k][Ie] in slot order.
template <typename T, bool Q8>
__global__ void __launch_bounds__(256) moe_gu1_kernel(const T *__restrict__ x, const T *__restrict__ nw, float eps,
                                                      const T *__restrict__ logits, int E, int k, int norm,
                                                      const void *__restrict__ Wgu, const bf16 *__restrict__ Ws,
                                                      const bf16 *__restrict__ Wb, int hid, int Ie,
                                                      int32_t *__restrict__ idx, T *__restrict__ wsel,
                                                      T *__restrict__ m) {
    constexpr int VN = Vec<T>::N;
    constexpr int EPL = 4;
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    T *ys = (T *)smem_raw;
    __shared__ float red[8];
    __shared__ int sel;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, s = blockIdx.y;
    float v[EPL];
    if (wave == 0) load_logits<T, EPL>(logits, E, lane, v);  // in flight during the norm
    if (nw) {
        norm_prologue<T>(x, nullptr, nw, eps, nullptr, hid, ys, red);
    } else {
        for (int c = threadIdx.x; c < hid / VN; c += blockDim.x) *(u32x4 *)&ys[c * VN] = ld16(x + (size_t)c * VN);
        __syncthreads();
    }
    if (wave == 0) {
        softmax_inplace<T, EPL>(E, lane, v);
        float psel[16];
        int isel[16];
        select_topk<EPL>(v, E, k, lane, psel, isel);
        if (lane == 0) {
            int e = 0;
#pragma unroll
            for (int q = 0; q < 16; ++q)
                if (q == s) e = isel[q];
            sel = e;
            if (blockIdx.x == 0 && s == 0) write_routing<T>(0, k, norm, psel, isel, idx, wsel);
        }
    }
    __syncthreads();
    const int e = sel, n = blockIdx.x * 4 + wave;
    if (n >= Ie) return;
    const size_t g = (size_t)e * 2 * Ie + n, u = g + Ie;  // gate and up rows
    float acc[2] = {0.f, 0.f};
    if constexpr (Q8) {
        const int ng = hid / 64;
        const uint8_t *W8 = (const uint8_t *)Wgu;
        const uint8_t *const w[2] = {W8 + g * hid, W8 + u * hid};
        const bf16 *const sc[2] = {Ws + g * ng, Ws + u * ng}, *const bi[2] = {Wb + g * ng, Wb + u * ng};
        rows_dot_q8<2, 2>(w, sc, bi, (const bf16 *)ys, hid, lane, acc);
    } else {
        const T *WT = (const T *)Wgu;
        const T *const w[2] = {WT + g * hid, WT + u * hid};
        rows_dot<T, 2, 4>(w, ys, hid, lane, acc);
    }
    const float s0 = wave_sum(acc[0]), s1 = wave_sum(acc[1]);
    if (lane == 0) m[(size_t)s * Ie + n] = from_f<T>(rho<T>(silu_f32(rho<T>(s0))) * rho<T>(s1));
}

// grid hid / 4, 512 threads: wave w takes slots w, w + 8 (k <= 16) and computes outputs
// 4x..4x+3 of its slot's expert from m[s]; part[s][q] = rho(rho(y) * w_s); the block sums the
// slots in slot order, as moe_combine_kernel does.
template <typename T, bool Q8>
__global__ void __launch_bounds__(512) moe_down1_kernel(const T *__restrict__ m, const void *__restrict__ Wd,
                                                        const bf16 *__restrict__ Ws, const bf16 *__restrict__ Wb,
                                                        int Ie, int hid, int E, int k,
                                                        const int32_t *__restrict__ idx, const T *__restrict__ wsel,
                                                        T *__restrict__ out) {
    constexpr int NO = 4;
    __shared__ float part[16][NO];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n0 = blockIdx.x * NO;
    for (int s = wave; s < k; s += 8) {
        const int e = idx[s];
        float acc[NO] = {0.f, 0.f, 0.f, 0.f};
        if ((unsigned)e < (unsigned)E) {  // always: the routing names valid experts
            const size_t r0 = (size_t)e * hid + n0;
            if constexpr (Q8) {
                const int ng = Ie / 64;
                const uint8_t *W8 = (const uint8_t *)Wd;
                const uint8_t *const w[NO] = {W8 + r0 * Ie, W8 + (r0 + 1) * Ie, W8 + (r0 + 2) * Ie, W8 + (r0 + 3) * Ie};
                const bf16 *const sc[NO] = {Ws + r0 * ng, Ws + (r0 + 1) * ng, Ws + (r0 + 2) * ng, Ws + (r0 + 3) * ng};
                const bf16 *const bi[NO] = {Wb + r0 * ng, Wb + (r0 + 1) * ng, Wb + (r0 + 2) * ng, Wb + (r0 + 3) * ng};
                rows_dot_q8<NO, 1>(w, sc, bi, (const bf16 *)m + (size_t)s * Ie, Ie, lane, acc);
            } else {
                const T *WT = (const T *)Wd;
                const T *const w[NO] = {WT + r0 * Ie, WT + (r0 + 1) * Ie, WT + (r0 + 2) * Ie, WT + (r0 + 3) * Ie};
                rows_dot<T, NO, 2>(w, m + (size_t)s * Ie, Ie, lane, acc);
            }
        }
        const float ws = to_f(wsel[s]);
#pragma unroll
        for (int q = 0; q < NO; ++q) {
            const float y = wave_sum(acc[q]);
            if (lane == 0) part[s][q] = rho<T>(rho<T>(y) * ws);
        }
    }
    __syncthreads();
    if (threadIdx.x < NO) {
        float a = 0.f;
        for (int s = 0; s < k; ++s) a += part[s][threadIdx.x];
        out[n0 + threadIdx.x] = from_f<T>(a);
    }
}

// ------------------------------------------------------------ weighted slot sum
// grid (hid / 256, T): one thread per output element; the token's k sorted positions and
// weights are loaded first, so the k row reads are in flight together.
template <typename T>
__global__ void __launch_bounds__(256) moe_combine_kernel(const T *__restrict__ y, const T *__restrict__ w,
                                                          const int32_t *__restrict__ inv, int hid, int k, int rows,
                                                          T *__restrict__ out) {
    const int t = blockIdx.y, n = blockIdx.x * 256 + threadIdx.x;
    int p[16];
    float ws[16];
#pragma unroll
    for (int s = 0; s < 16; ++s)
        if (s < k) {
            p[s] = inv[t * k + s];
            ws[s] = to_f(w[t * k + s]);
        }
    if (n >= hid) return;
    float acc = 0.f;
#pragma unroll
    for (int s = 0; s < 16; ++s)
        if (s < k && (unsigned)p[s] < (unsigned)rows)  // always, for positions the sort writes
            acc += rho<T>(to_f(y[(size_t)p[s] * hid + n]) * ws[s]);
    out[(size_t)t * hid + n] = from_f<T>(acc);
}

// ------------------------------------------------------------ dispatch
// One token: router projection (norm prologue when nw), moe_gu1_kernel, moe_down1_kernel.
template <typename T>
static hipError_t moe1_t(const void *x, const void *nw, float eps, int hid, const MoeWeights &W, int E, int k,
                         int norm, int Ie, int32_t *idx, void *w, void *out, void *ws, hipStream_t s) {
    const int dt = DtOf<T>::value;
    const MoeWs L = moe_layout(1, hid, E, k, Ie, dt);
    char *base = (char *)ws;
    T *logits = (T *)(base + L.logits), *mbuf = (T *)(base + L.m);
    if (W.q8 && !std::is_same<T, bf16>::value) return hipErrorInvalidValue;
    hipError_t e;
    if (W.q8)
        e = nw ? launch_linear_q8_norm(x, nullptr, nw, eps, nullptr, hid, (const uint8_t *)W.router, W.router_s,
                                       W.router_b, 64, E, EPI_STORE, logits, s)
               : launch_linear_q8(x, 1, hid, (const uint8_t *)W.router, W.router_s, W.router_b, 64, E, EPI_STORE,
                                  nullptr, logits, s);
    else
        e = nw ? launch_linear_norm(dt, x, nullptr, nw, eps, nullptr, hid, W.router, E, EPI_STORE, logits, s)
               : launch_linear(dt, x, 1, hid, W.router, E, EPI_STORE, nullptr, logits, s);
    if (e != hipSuccess) return e;
    const dim3 g1((Ie + 3) / 4, k);
    const size_t lds = (size_t)hid * sizeof(T);
    const bf16 *gs = (const bf16 *)W.gate_up_s, *gb = (const bf16 *)W.gate_up_b;
    const bf16 *ds = (const bf16 *)W.down_s, *db = (const bf16 *)W.down_b;
    if (W.q8) {
        if constexpr (std::is_same<T, bf16>::value) {
            moe_gu1_kernel<T, true><<<g1, 256, lds, s>>>((const T *)x, (const T *)nw, eps, logits, E, k, norm,
                                                         W.gate_up, gs, gb, hid, Ie, idx, (T *)w, mbuf);
            moe_down1_kernel<T, true><<<hid / 4, 512, 0, s>>>(mbuf, W.down, ds, db, Ie, hid, E, k, idx, (const T *)w,
                                                              (T *)out);
        } else {
            return hipErrorInvalidValue;  // 8-bit weights come with the bf16 model dtype only
        }
    } else {
        moe_gu1_kernel<T, false><<<g1, 256, lds, s>>>((const T *)x, (const T *)nw, eps, logits, E, k, norm,
                                                      W.gate_up, gs, gb, hid, Ie, idx, (T *)w, mbuf);
        moe_down1_kernel<T, false><<<hid / 4, 512, 0, s>>>(mbuf, W.down, ds, db, Ie, hid, E, k, idx, (const T *)w,
                                                           (T *)out);
    }
    return hipGetLastError();
}

template <typename T>
static hipError_t moe_t(const void *x, int T_, int hid, const MoeWeights &W, int E, int k, int norm, int Ie,
                        int32_t *idx, void *w, void *out, void *ws, hipStream_t s) {
    const int dt = DtOf<T>::value;
    const MoeWs L = moe_layout(T_, hid, E, k, Ie, dt);
    char *base = (char *)ws;
    T *logits = (T *)(base + L.logits);
    int32_t *offsets = (int32_t *)(base + L.offsets), *perm = (int32_t *)(base + L.perm);
    int32_t *inv = (int32_t *)(base + L.inv), *active = (int32_t *)(base + L.active);
    T *mbuf = (T *)(base + L.m), *ybuf = (T *)(base + L.y);
    const int rows = T_ * k;
    if (T_ == 1) return moe1_t<T>(x, nullptr, 0.f, hid, W, E, k, norm, Ie, idx, w, out, ws, s);
    hipError_t e = W.q8 ? launch_linear_q8(x, T_, hid, (const uint8_t *)W.router, W.router_s, W.router_b, 64, E,
                                           EPI_STORE, nullptr, logits, s)
                        : launch_linear(dt, x, T_, hid, W.router, E, EPI_STORE, nullptr, logits, s);
    if (e != hipSuccess) return e;
    moe_topk_kernel<T><<<T_, 64, 0, s>>>(logits, E, k, norm, idx, (T *)w);
    moe_sort_kernel<<<1, 256, 0, s>>>(idx, rows, E, offsets, perm, inv, active);
    const int na_max = rows < E ? rows : E;
    const dim3 g0((Ie + 3) / 4, na_max), g1((hid + 15) / 16, na_max);
    if constexpr (std::is_same<T, bf16>::value) {
        if (W.q8 && hid % 256 == 0 && Ie % 256 == 0) {
            moe_expert_q8_mfma_kernel<0><<<dim3((Ie + 15) / 16, na_max), 256, 0, s>>>(
                (const bf16 *)x, (const uint8_t *)W.gate_up, (const bf16 *)W.gate_up_s, (const bf16 *)W.gate_up_b, hid,
                Ie, k, offsets, perm, active, mbuf);
            moe_expert_q8_mfma_kernel<1><<<dim3((hid + 15) / 16, na_max), 256, 0, s>>>(
                mbuf, (const uint8_t *)W.down, (const bf16 *)W.down_s, (const bf16 *)W.down_b, Ie, hid, k, offsets,
                perm, active, ybuf);
        } else if (W.q8) {
            moe_expert_q8_kernel<0><<<g0, 256, 0, s>>>((const bf16 *)x, (const uint8_t *)W.gate_up,
                                                       (const bf16 *)W.gate_up_s, (const bf16 *)W.gate_up_b, hid, Ie,
                                                       k, offsets, perm, active, mbuf);
            moe_expert_q8_kernel<1><<<g1, 256, 0, s>>>(mbuf, (const uint8_t *)W.down, (const bf16 *)W.down_s,
                                                       (const bf16 *)W.down_b, Ie, hid, k, offsets, perm, active,
                                                       ybuf);
        }
    }
    if (!W.q8) {
        bool mfma = false;
        if constexpr (std::is_same<T, bf16>::value) {
            if (hid % 256 == 0 && Ie % 256 == 0) {
                mfma = true;
                moe_expert_mfma_kernel<0><<<dim3((Ie + 15) / 16, na_max), 512, 0, s>>>(
                    (const bf16 *)x, (const bf16 *)W.gate_up, hid, Ie, k, offsets, perm, active, mbuf);
                moe_expert_mfma_kernel<1><<<dim3((hid + 15) / 16, na_max), 512, 0, s>>>(
                    mbuf, (const bf16 *)W.down, Ie, hid, k, offsets, perm, active, ybuf);
            }
        }
        if (!mfma) {
            moe_expert_kernel<T, 0><<<g0, 256, 0, s>>>((const T *)x, (const T *)W.gate_up, hid, Ie, k, offsets, perm,
                                                       active, mbuf);
            moe_expert_kernel<T, 1><<<g1, 256, 0, s>>>(mbuf, (const T *)W.down, Ie, hid, k, offsets, perm, active,
                                                       ybuf);
        }
    }
    moe_combine_kernel<T><<<dim3((hid + 255) / 256, T_), 256, 0, s>>>(ybuf, (const T *)w, inv, hid, k, rows, (T *)out);
    return hipGetLastError();
}

hipError_t launch_moe_norm1(int dt, const void *h, const void *nw, float eps, int hid, const MoeWeights &W, int E,
                            int k, int norm, int Ie, int32_t *idx, void *w, void *out, void *ws, hipStream_t s) {
    if (dt == DT_BF16) return moe1_t<bf16>(h, nw, eps, hid, W, E, k, norm, Ie, idx, w, out, ws, s);
    if (W.q8) return hipErrorInvalidValue;
    return moe1_t<float>(h, nw, eps, hid, W, E, k, norm, Ie, idx, w, out, ws, s);
}

hipError_t launch_moe(int dt, const void *x, int T, int hid, const MoeWeights &W, int E, int k, int norm, int Ie,
                      int32_t *idx, void *w, void *out, void *ws, hipStream_t s) {
    if (dt == DT_BF16) return moe_t<bf16>(x, T, hid, W, E, k, norm, Ie, idx, w, out, ws, s);
    if (W.q8) return hipErrorInvalidValue;  // 8-bit weights come with the bf16 model dtype only
    return moe_t<float>(x, T, hid, W, E, k, norm, Ie, idx, w, out, ws, s);
}

}  // namespace q3
