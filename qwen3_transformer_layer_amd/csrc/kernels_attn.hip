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
//  - attn_prefill_fa_kernel (T > 1, bf16, head_dim 128): causal flash attention on
//    v_mfma_f32_32x32x16_bf16.  Block = 32 queries x the G heads of one kv head, NP waves
//    per head (4 for G <= 2, else 2), each taking one 32-key part of every (32 NP)-key tile;
//    K/V tiles arrive by direct-to-LDS copies in a 2-stage ring.  S^T = K Q^T leaves each lane
//    one query and 32 of the tile's keys, which is exactly the P^T operand layout of
//    O^T += V^T P^T once the keys of each 16-key MFMA step are taken in the order
//    {4h..4h+3, 8+4h..8+4h+3} (h = lane / 32); V^T comes from the LDS transpose read.  The
//    grid is 1-D with kv head b % KV (one kv head per XCD when KV = 8); a block takes the
//    heaviest and the lightest remaining query tile together when that still gives one block
//    per CU, else one tile, heaviest first.
//  - attn_prefill_mfma_kernel (T > 1, bf16, head_dim 64): causal flash attention on MFMA.
//    Computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (q and k are bf16
//    values, so the products are exact and the sums fp32), an online fp32
//    softmax, and O^T += V^T P^T where the fp32 P is split into bf16 hi + lo
//    parts so the probability weights keep ~16 bits instead of bf16's 8.
//  - attn_rowwise_kernel (T > 1, fp32 strict mode): one wave per (query, head),
//    online softmax over key blocks of 64.
#include <climits>
#include <math.h>

#include "attn_core.h"
#include "common.h"
#include "kernels.h"

namespace q3 {

// First key a query at position p sees: 0 (causal) or the start of a sliding window of w
// positions ("rlx_flow/blocks/qwen3_decoder.rs", Qwen3DecoderSpec mask SlidingWindow(w)).
static inline int window_lo(int p, int window) { return window > 0 && p - window + 1 > 0 ? p - window + 1 : 0; }

static inline int decode_chunk(int nkeys, int KV) {  // keys per split of a T == 1 step
    int c = (nkeys * KV + 511) / 512;
    c = (c + 31) / 32 * 32;
    if (c < 32) c = 32;
    if (c > 1024) c = 1024;
    return c;
}

// split partials of one seat (fp32 words): H heads x up to cap / 32 splits x (max, sum, D values)
static size_t seat_part_words(int H, int D, int cap) { return (size_t)H * ((cap + 31) / 32) * (D + 2); }

size_t attention_workspace(int T, int H, int KV, int D, int cap) {
    (void)KV;
    const int seats = T < DECODE_MAXB ? (T < 1 ? 1 : T) : DECODE_MAXB;
    return (size_t)seats * seat_part_words(H, D, cap) * sizeof(float);
}

// ------------------------------------------------------------ split-K decode
template <typename T, int D, int G>
__device__ __forceinline__ void decode_core(const float *qs, const T *__restrict__ Kg, const T *__restrict__ Vg,
                                            const u32x4 *kp, const u32x4 *vp, int j0, int j1, int jspec,
                                            const float *kspec, const float *vspec, float scale, float *sc, int chunk,
                                            float *red, float *mrow, float *lrow, float *__restrict__ part,
                                            int nsplit, int g, int s) {
    decode_core_lds<T, D, G, 4>(qs, Kg, Vg, kp, vp, j0, j1, jspec, kspec, vspec, scale, sc, chunk, red, mrow, lrow);
    for (int idx = threadIdx.x; idx < G * D; idx += 256) {
        const int i = idx / D, d = idx % D;
        part[((size_t)(g * G + i) * nsplit + s) * (D + 2) + 2 + d] = decode_core_reduce<D, G, 4>(red, i, d);
    }
    if (threadIdx.x < G) {
        float *pp = part + ((size_t)(g * G + threadIdx.x) * nsplit + s) * (D + 2);
        pp[0] = mrow[threadIdx.x];
        pp[1] = lrow[threadIdx.x];
    }
}

// q [H][D] already normalised and rotated; the cache already holds position nkeys - 1.
template <typename T, int D, int G>
__global__ void __launch_bounds__(256) attn_decode_kernel(const T *__restrict__ q, const T *__restrict__ Kc,
                                                          const T *__restrict__ Vc, int cap, int lo, int nkeys,
                                                          int chunk, float scale, float *__restrict__ part,
                                                          int nsplit) {
    extern __shared__ float smem[];
    float *sc = smem;                  // [G][chunk]
    float *red = smem + G * chunk;     // [4][G][D]
    __shared__ float qs[G * D];
    __shared__ float mrow[G], lrow[G];
    const int s = blockIdx.x, g = blockIdx.y;
    const int j0 = lo + s * chunk, j1 = min(nkeys, j0 + chunk);
    const T *Kg = Kc + (size_t)g * cap * D, *Vg = Vc + (size_t)g * cap * D;
    u32x4 kp[DEC_PF], vp[DEC_PF];
    decode_prefetch<T, D>(Kg, Vg, j0, j1, kp, vp);
    for (int i = threadIdx.x; i < G * D; i += 256) qs[i] = to_f(q[(size_t)g * G * D + i]);
    __syncthreads();
    decode_core<T, D, G>(qs, Kg, Vg, kp, vp, j0, j1, -1, nullptr, nullptr, scale, sc, chunk, red, mrow, lrow, part,
                         nsplit, g, s);
}

// Fused decode step at position p = nkeys - 1: per-head RMSNorm of the group's q heads and
// (in the split holding p) of k, RoPE at p, and the cache write of k and v at p, then the
// split's attention over keys lo + s chunk ..  qkv: [(H+2KV)D] for the one token.  With a
// bias [(H+2KV)D] each q/k/v element is first rho(x + b); with q_norm == k_norm == NULL the
// per-head norm is skipped (page 2's qk_norm / attention_bias switches).
template <typename T, int D, int G>
__device__ __forceinline__ void decode_fused_block(const T *__restrict__ qkv, int H, int KV, const T *__restrict__ q_norm,
                                                   const T *__restrict__ k_norm, const T *__restrict__ bias, float eps,
                                                   const T *__restrict__ cos_t, const T *__restrict__ sin_t,
                                                   T *__restrict__ Kc, T *__restrict__ Vc, int cap, int lo, int nkeys,
                                                   int chunk, float scale, float *__restrict__ part, int nsplit, int s,
                                                   int g) {
    extern __shared__ float smem[];
    float *sc = smem;
    float *red = smem + G * chunk;
    __shared__ float qs[G * D];
    __shared__ float kvs[2 * D];
    __shared__ float mrow[G], lrow[G];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j0 = lo + s * chunk, j1 = min(nkeys, j0 + chunk);
    const int p = nkeys - 1;
    const bool has_p = j1 == nkeys;
    T *Kg = Kc + (size_t)g * cap * D, *Vg = Vc + (size_t)g * cap * D;
    u32x4 kp[DEC_PF], vp[DEC_PF];
    decode_prefetch<T, D>(Kg, Vg, j0, j1, kp, vp);  // entry p, if loaded here, is replaced by kvs below
    constexpr int half = D / 2;
    const int nheads = G + (has_p ? 1 : 0);
    for (int hh = wave; hh < nheads; hh += 4) {
        const bool is_q = hh < G;
        const size_t ro = (size_t)(is_q ? g * G + hh : H + g) * D;
        const T *row = qkv + ro;
        const T *wn = is_q ? q_norm : k_norm;
        const bool on = lane < half;
        float x1 = 0.f, x2 = 0.f;
        if (on) {
            x1 = to_f(row[lane]);
            x2 = to_f(row[lane + half]);
            if (bias) {
                x1 = rho<T>(x1 + to_f(bias[ro + lane]));
                x2 = rho<T>(x2 + to_f(bias[ro + lane + half]));
            }
        }
        const float r = 1.0f / sqrtf(wave_sum(x1 * x1 + x2 * x2) / (float)D + eps);
        if (on) {
            const float n1 = wn ? rho<T>(to_f(wn[lane]) * rho<T>(x1 * r)) : x1;
            const float n2 = wn ? rho<T>(to_f(wn[lane + half]) * rho<T>(x2 * r)) : x2;
            const float c1 = to_f(cos_t[(size_t)p * D + lane]), s1 = to_f(sin_t[(size_t)p * D + lane]);
            const float c2 = to_f(cos_t[(size_t)p * D + lane + half]), s2 = to_f(sin_t[(size_t)p * D + lane + half]);
            const float o1 = rho<T>(n1 * c1 - n2 * s1), o2 = rho<T>(n2 * c2 + n1 * s2);
            if (is_q) {
                qs[hh * D + lane] = o1;
                qs[hh * D + lane + half] = o2;
            } else {
                kvs[lane] = o1;
                kvs[lane + half] = o2;
                T *kd = Kg + (size_t)p * D;
                kd[lane] = from_f<T>(o1);
                kd[lane + half] = from_f<T>(o2);
                const T *vrow = qkv + (size_t)(H + KV + g) * D;
                T *vd = Vg + (size_t)p * D;
                T v1 = vrow[lane], v2 = vrow[lane + half];
                if (bias) {
                    v1 = from_f<T>(to_f(v1) + to_f(bias[(size_t)(H + KV + g) * D + lane]));
                    v2 = from_f<T>(to_f(v2) + to_f(bias[(size_t)(H + KV + g) * D + lane + half]));
                }
                vd[lane] = v1;
                vd[lane + half] = v2;
                kvs[D + lane] = to_f(v1);
                kvs[D + lane + half] = to_f(v2);
            }
        }
    }
    __syncthreads();
    decode_core<T, D, G>(qs, Kg, Vg, kp, vp, j0, j1, has_p ? p : -1, kvs, kvs + D, scale, sc, chunk, red, mrow, lrow,
                         part, nsplit, g, s);
}

template <typename T, int D, int G>
__global__ void __launch_bounds__(256) attn_decode_fused_kernel(
    const T *__restrict__ qkv, int H, int KV, const T *__restrict__ q_norm, const T *__restrict__ k_norm,
    const T *__restrict__ bias, float eps, const T *__restrict__ cos_t, const T *__restrict__ sin_t,
    T *__restrict__ Kc, T *__restrict__ Vc, int cap, int lo, int nkeys, int chunk, float scale,
    float *__restrict__ part, int nsplit) {
    decode_fused_block<T, D, G>(qkv, H, KV, q_norm, k_norm, bias, eps, cos_t, sin_t, Kc, Vc, cap, lo, nkeys, chunk,
                                scale, part, nsplit, blockIdx.x, blockIdx.y);
}

// Several seats at once (blockIdx.z = seat b): seat b's q|k|v row, cache, position and split
// come from the by-value batch; its partials go to part + b * part_stride.
template <typename T, int D, int G>
__global__ void __launch_bounds__(256) attn_decode_fused_batch_kernel(
    const T *__restrict__ qkv, int nqkv, int H, int KV, const T *__restrict__ q_norm, const T *__restrict__ k_norm,
    const T *__restrict__ bias, float eps, const T *__restrict__ cos_t, const T *__restrict__ sin_t, DecodeBatch bt,
    int cap, float scale, float *__restrict__ part, size_t part_stride) {
    const int b = blockIdx.z;
    if ((int)blockIdx.x >= bt.nsplit[b]) return;  // uniform over the block
    decode_fused_block<T, D, G>(qkv + (size_t)b * nqkv, H, KV, q_norm, k_norm, bias, eps, cos_t, sin_t,
                                (T *)bt.kc[b], (T *)bt.vc[b], cap, bt.lo[b], bt.p[b] + 1, bt.chunk[b], scale,
                                part + (size_t)b * part_stride, bt.nsplit[b], blockIdx.x, blockIdx.y);
}

// Merge the splits of one head: out = rho(sum_s o_s e^(m_s - M) / sum_s l_s e^(m_s - M)).
// Thread t owns 32 consecutive values of split t / (D/32) in each pass of 256/(D/32)
// splits, so every load of a pass is issued at once.
template <typename T, int D>
__device__ __forceinline__ void combine_block(const float *__restrict__ part, int nsplit, T *__restrict__ out, int h) {
    constexpr int TPS = D / 32;        // threads per split
    constexpr int SPP = 256 / TPS;     // splits per pass
    __shared__ float red[4];
    __shared__ float accs[SPP][D + 1];
    __shared__ float lsum[SPP];
    const int tid = threadIdx.x;
    const int sl = tid / TPS, d0 = (tid % TPS) * 32;
    const float *ph = part + (size_t)h * nsplit * (D + 2);
    float M = -INFINITY;
    for (int s = sl; s < nsplit; s += SPP) M = fmaxf(M, ph[(size_t)s * (D + 2)]);
    M = wave_max(M);
    if ((tid & 63) == 0) red[tid >> 6] = M;
    __syncthreads();
    M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float acc[32], L = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) acc[e] = 0.f;
    for (int s = sl; s < nsplit; s += SPP) {
        const float *pp = ph + (size_t)s * (D + 2);
        const float f = __expf(pp[0] - M);
        L += pp[1] * f;
#pragma unroll
        for (int e = 0; e < 32; ++e) acc[e] += pp[2 + d0 + e] * f;
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) accs[sl][d0 + e] = acc[e];
    if (d0 == 0) lsum[sl] = L;
    __syncthreads();
    if (tid < D) {
        float a = 0.f, l = 0.f;
        for (int k = 0; k < SPP; ++k) {
            a += accs[k][tid];
            l += lsum[k];
        }
        out[(size_t)h * D + tid] = from_f<T>(a / l);
    }
}

template <typename T, int D>
__global__ void __launch_bounds__(256) attn_combine_kernel(const float *__restrict__ part, int nsplit,
                                                           T *__restrict__ out) {
    combine_block<T, D>(part, nsplit, out, blockIdx.x);
}

// grid (H, seats): seat b's partials at part + b * part_stride, output row b of out [B][H*D]
template <typename T, int D>
__global__ void __launch_bounds__(256) attn_combine_batch_kernel(const float *__restrict__ part, size_t part_stride,
                                                                 DecodeBatch bt, int H, T *__restrict__ out) {
    const int b = blockIdx.y;
    combine_block<T, D>(part + (size_t)b * part_stride, bt.nsplit[b], out + (size_t)b * H * D, blockIdx.x);
}

// ------------------------------------------------------------ fp32 / fallback row-wise kernel
template <typename T>
__global__ void __launch_bounds__(64) attn_rowwise_kernel(const T *__restrict__ q, const T *__restrict__ Kc,
                                                          const T *__restrict__ Vc, int H, int KV, int D, int cap,
                                                          int p0, int window, float scale, T *__restrict__ out) {
    __shared__ float qs[128];
    __shared__ float es[64];
    const int t = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
    const int g = h / (H / KV), p = p0 + t;
    const T *Kg = Kc + (size_t)g * cap * D;
    const T *Vg = Vc + (size_t)g * cap * D;
    for (int d = lane; d < D; d += 64) qs[d] = to_f(q[((size_t)t * H + h) * D + d]);
    __syncthreads();
    float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
    const int lo = window > 0 && p - window + 1 > 0 ? p - window + 1 : 0;  // the first chunk holds key lo
    for (int jb = lo & ~63; jb <= p; jb += 64) {
        const int j = jb + lane;
        float sj = -INFINITY;
        if (j >= lo && j <= p) {
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
// Block: QB queries of all G query heads of one kv head (so every K/V tile read serves G
// heads); wave w owns 16 queries of one head.  K/V tiles of 64 keys are double-buffered in
// LDS (next tile's global loads in registers while the current tile is computed).
//   S^T (keys x queries) = K Q^T with v_mfma_f32_16x16x32_bf16: lane l holds query l%16 and
//   keys 4*(l/16) + a of each 16-key sub-tile, so its softmax statistics are per query;
//   O^T (d x queries) += V^T P^T: the V^T operand comes straight from the row-major V tile
//   with the gfx950 LDS transpose read (ds_read_b64_tr_b16): in each 16-lane group, source
//   lane s points at V[k + s/4][d + 4*(s%4)], and lane r receives V[k + v][d + r], v = 0..3;
//   P (fp32) enters as bf16 hi + bf16 lo.  Scores are kept in base 2 (log2 e folded into
//   the scale) and exponentiated with v_exp_f32.
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ s16x4 lds_tr_b64(const uint16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p);
}

template <int D, int G>
__global__ void __launch_bounds__(64 * (G >= 8 ? 8 : 4)) attn_prefill_mfma_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ Kc, const bf16 *__restrict__ Vc, int T, int H, int KV,
    int cap, int p0, int window, float scale_log2, bf16 *__restrict__ out) {
    constexpr int QB = G >= 4 ? 16 : 64 / G;   // queries per block
    constexpr int QG = QB / 16;                // 16-query groups per head
    constexpr int NW = G * QG;                 // waves
    constexpr int NT = 64 * NW;
    constexpr int P = D + 8;                   // LDS row pitch (elements)
    constexpr int CH = 64 * (D / 8);           // 16-byte chunks per 64-key tile
    constexpr int CPT = (CH + NT - 1) / NT;    // chunks per thread per operand
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][64 * P];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][64 * P];
    const int ntiles = (T + QB - 1) / QB;
    const int qt = ntiles - 1 - blockIdx.x;  // latest (heaviest) query tiles first
    const int g = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = g * G + wave / QG;
    const int t0 = qt * QB, wq0 = t0 + (wave % QG) * 16;
    const int col = lane & 15, quad = lane >> 4;
    const int tq = wq0 + col;
    const int qpos = p0 + min(tq, T - 1);
    const int kmax = p0 + min(t0 + QB - 1, T - 1);
    const int wlast = p0 + min(wq0 + 15, T - 1);  // last query position of this wave
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

    u32x4 rk[CPT], rv[CPT];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * NT;
            const int r = c / (D / 8), d8 = (c % (D / 8)) * 8;
            const bool ok = c < CH && k0 + r <= kmax;
            rk[i] = ok ? ld16(Kg + (size_t)(k0 + r) * D + d8) : u32x4{0, 0, 0, 0};
            rv[i] = ok ? ld16(Vg + (size_t)(k0 + r) * D + d8) : u32x4{0, 0, 0, 0};
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + i * NT;
            if (c < CH) {
                const int r = c / (D / 8), d8 = (c % (D / 8)) * 8;
                *(u32x4 *)&Ks[buf][r * P + d8] = rk[i];
                *(u32x4 *)&Vs[buf][r * P + d8] = rv[i];
            }
        }
    };

    const int nkt = kmax / 64 + 1;
    // sliding window: keys below the block's first window start are never visible
    const int kt0 = window > 0 && p0 + t0 - window + 1 > 0 ? (p0 + t0 - window + 1) / 64 : 0;
    const int wlo = window > 0 ? p0 + wq0 - window + 1 : 0;          // the wave's lowest window start
    const int qlo = window > 0 ? qpos - window + 1 : INT_MIN;         // this lane's query
    gload(kt0 * 64);
    sstore(0);
    __syncthreads();
    for (int kt = kt0; kt < nkt; ++kt) {
        const int k0 = kt * 64, buf = (kt - kt0) & 1;
        if (kt + 1 < nkt) gload(k0 + 64);
        if (k0 <= wlast && k0 + 63 >= wlo) {
            const uint16_t *Kt = Ks[buf], *Vt = Vs[buf];
            f32x4 sacc[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks) {
                    const bf16x8 kf = *(const bf16x8 *)&Kt[(kb * 16 + col) * P + ks * 32 + quad * 8];
                    sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], sacc[kb], 0, 0, 0);
                }
            }
            const bool need_mask = k0 + 63 > p0 + wq0 || (window > 0 && k0 < wlast - window + 1);
            float tmax = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    float sv = sacc[kb][a] * scale_log2;
                    const int key = k0 + kb * 16 + quad * 4 + a;
                    if (need_mask && (key > qpos || key < qlo)) sv = -INFINITY;
                    sacc[kb][a] = sv;
                    tmax = fmaxf(tmax, sv);
                }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            // a query whose window has not started yet has no visible key: its p stay 0
            const float m_new = fmaxf(m_run, tmax);
            const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
            const float m_sub = m_new == -INFINITY ? 0.0f : m_new;
            float psum = 0.f;
            bf16x8 phi[2], plo[2];
#pragma unroll
            for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const float pv = __builtin_amdgcn_exp2f(sacc[2 * kc + hf][a] - m_sub);
                        psum += pv;
                        const __bf16 hb = (__bf16)pv;
                        phi[kc][hf * 4 + a] = hb;
                        plo[kc][hf * 4 + a] = (__bf16)(pv - (float)hb);
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
                    const uint16_t *src = &Vt[(kc * 32 + quad * 4 + (col >> 2)) * P + dt * 16 + 4 * (col & 3)];
                    const s16x4 lo4 = lds_tr_b64(src);
                    const s16x4 hi4 = lds_tr_b64(src + 16 * P);
                    bf16x8 vf;
                    short *vs = (short *)&vf;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        vs[e] = lo4[e];
                        vs[4 + e] = hi4[e];
                    }
                    acc_o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, phi[kc], acc_o[dt], 0, 0, 0);
                    acc_o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, plo[kc], acc_o[dt], 0, 0, 0);
                }
            }
        }
        if (kt + 1 < nkt) sstore(buf ^ 1);
        __syncthreads();
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

// The values of lanes l and l ^ 32 in every lane, as (value of the lower lane, value of the upper
// lane): one v_permlane32_swap instead of an LDS permute.
__device__ __forceinline__ f32x2 halves32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// ------------------------------------------------------------ bf16 causal flash prefill, head_dim 128
// Block: 32 queries x the G heads of one kv head; NP waves per head (NP = 4 for G <= 2, else
// 2), wave part w takes keys 32 w .. 32 w + 31 of every (32 NP)-key tile, so a block holds
// 2 waves per SIMD on its own and one wave's softmax arithmetic overlaps another's MFMAs.
// (With two key halves and two blocks per CU, a CU whose light block finished ran its heavy
// block at one wave per SIMD, latency-bound: 4 parts, 60 -> 52 us at T = 2048.)  Each wave
// keeps its own running maximum, sum and O; at the end the parts exchange them through LDS and
// each part merges (log-sum-exp scaling) and stores its own quarter (half for NP = 2) of the
// output columns.  The running maximum is raised only
// when a tile's maximum exceeds it by more than 8 (base 2), so probabilities stay <= 2^8 in
// fp32 and the O rescale is rare; the normalised result is the same softmax.  Query tiles
// are dispatched heaviest (most keys) first, so the blocks that start last are the short
// ones.
// LDS: per stage a K tile and a V tile of 32 NP rows x 256 B.  K rows: 16-byte chunk c at
// slot c ^ (row & 15) (16 lanes reading 16 rows at one chunk hit distinct banks); V rows:
// chunk c at slot c ^ (4 (row & 3)) (a transpose read covers 4 rows x 32 B per 16 lanes:
// distinct banks for 32 lanes).
template <int G>
struct FaGeo {
    static constexpr int NP = G <= 2 ? 4 : 2;  // key parts (waves) per head
    static constexpr int D = 128, RB = 256, KT = 32 * NP, ST = 2, NW = NP * G;
    static constexpr int TILE = KT * RB, STAGE = 2 * TILE;
    static constexpr int COPIES = STAGE / 1024, PW = COPIES / NW, HALF = PW / 2;
    // merge: part w of a head merges output columns [32 w DP, 32 (w + 1) DP) and hands every other
    // part its O of those columns (4 KB per 32 columns, fp32), plus its m and l of the 32 queries
    static constexpr int DP = D / 32 / NP, OSL = D / 32 - DP, OB = 32 * 32 * 4;
    static constexpr int MERGE_O = G * NP * OSL * OB, MERGE = MERGE_O + G * NP * 2 * 32 * 4;
    static constexpr int LDS = ST * STAGE > MERGE ? ST * STAGE : MERGE;
    static_assert(D / 32 % NP == 0, "output column tiles split evenly over the parts");
    static_assert(COPIES % (2 * NW) == 0, "K and V copies split evenly over the waves");
};

// One query tile qt (32 queries) of kv head g: every wave of the block takes part.
template <int G>
__device__ __forceinline__ void fa_query_tile(unsigned char *fa_smem, const bf16 *__restrict__ q,
                                              const bf16 *__restrict__ Kc, const bf16 *__restrict__ Vc, int T, int H,
                                              int cap, int p0, int window, float scale_log2, bf16 *__restrict__ out,
                                              int qt, int g) {
    using F = FaGeo<G>;
    constexpr int D = F::D, RB = F::RB, KT = F::KT;
    constexpr bool HOIST = F::NW <= 8;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hw = wave / F::NP, par = wave % F::NP;
    const int h = g * G + hw, t0 = qt * 32;
    const int qi = lane & 31, hh = lane >> 5;
    const int tq = min(t0 + qi, T - 1), qpos = p0 + tq;
    const int kmax = p0 + min(t0 + 31, T - 1);  // the block's queries see keys 0..kmax
    const int nkt = kmax / KT + 1;
    // sliding window: the block's queries see keys kmin..kmax, query qpos keys qlo..qpos
    const int kmin = window > 0 && p0 + t0 - window + 1 > 0 ? p0 + t0 - window + 1 : 0;
    const int kt0 = kmin / KT;
    const int qlo = window > 0 ? qpos - window + 1 : INT_MIN;
    const bf16 *Kg = Kc + (size_t)g * cap * D, *Vg = Vc + (size_t)g * cap * D;
    const unsigned lds0 = (unsigned)(uintptr_t)fa_smem;

    bf16x8 qf[D / 16];  // Q^T operand: query qi, d = 16 ks + 8 hh + 0..7
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
        qf[ks] = __builtin_bit_cast(bf16x8, ld16(q + ((size_t)tq * H + h) * D + 16 * ks + 8 * hh));

    // copy i < HALF of this wave: K rows; i >= HALF: V rows (4 rows of 256 B per copy)
    auto issue = [&](int kt) {
        const unsigned st = lds0 + (kt % F::ST) * F::STAGE;
        const int slot = lane & 15;
#pragma unroll
        for (int i = 0; i < F::PW; ++i) {
            const bool isv = i >= F::HALF;
            const int dl = (isv ? i - F::HALF : i) * F::NW + wave;
            const int r = dl * 4 + (lane >> 4);
            const int c = isv ? (slot ^ (4 * (r & 3))) : (slot ^ (r & 15));
            const int key = min(kt * KT + r, kmax);  // rows past kmax are masked
            dma16((isv ? Vg : Kg) + (size_t)key * D + c * 8,
                  __builtin_amdgcn_readfirstlane(st + (isv ? F::TILE : 0) + dl * 1024));
        }
    };

    f32x16 o[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[i][v] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const int gi = lane >> 4, sl = lane & 15;  // transpose-read group and source lane

    issue(kt0);
    for (int kt = kt0; kt < nkt; ++kt) {
        wait_vm<0>();
        __syncthreads();  // stage kt landed for every wave; every wave finished kt - 1
        if (kt + 1 < nkt) issue(kt + 1);
        const int kb0 = kt * KT + 32 * par;  // this wave's 32 keys
        if (kb0 > kmax || kb0 + 31 < kmin) continue;  // all masked for every query of the block
        const unsigned char *Ks = fa_smem + (kt % F::ST) * F::STAGE, *Vs = Ks + F::TILE;
        f32x16 sc;
#pragma unroll
        for (int v = 0; v < 16; ++v) sc[v] = 0.f;
        {
            // with 8 waves (256 registers per lane) every K fragment read is issued before the first
            // MFMA (pinned: left to itself the compiler waits on each read right before its MFMA;
            // T = 2048, G = 2: 45.5 -> 42.8 us with the V reads below); 16 waves have half the
            // registers and keep one read per MFMA
            const int r = 32 * par + qi;
            bf16x8 kf[HOIST ? D / 16 : 1];
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                const bf16x8 k = *(const bf16x8 *)(Ks + r * RB + (((2 * ks + hh) ^ (r & 15)) << 4));
                if constexpr (HOIST) kf[ks] = k;
                else sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k, qf[ks], sc, 0, 0, 0);
            }
            if constexpr (HOIST) {
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks) sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], sc, 0, 0, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, D / 16, 0);  // the DS reads
                __builtin_amdgcn_sched_group_barrier(0x008, D / 16, 0);  // then the MFMAs
            }
        }
        // accumulator v of S^T: key kb0 + 8 (v / 4) + 4 hh + v % 4, query qi.  Only tiles that cross
        // the diagonal or the window edge test keys (a uniform branch).
        const bool need_mask = kb0 + 31 > p0 + t0 || (window > 0 && kb0 < kmax - window + 1);
        if (need_mask) {
            int qp = qpos;  // passed through the asm so the test cannot be hoisted out of the branch
            __asm__ volatile("" : "+v"(qp));
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int key = kb0 + 8 * (v >> 2) + 4 * hh + (v & 3);
                if (key > qp || key < qlo) sc[v] = -INFINITY;
            }
        }
        // The scale (> 0) is applied after the maximum (fp32 rounding is monotonic, so the rounded
        // product of the maximum is the maximum of the rounded products) and enters each exponent
        // through one fma.
        float tmax = sc[0];
#pragma unroll
        for (int v = 1; v < 16; ++v) tmax = fmaxf(tmax, sc[v]);
        const f32x2 tm2 = halves32(tmax);
        tmax = fmaxf(tm2[0], tm2[1]) * scale_log2;
        const bool up = tmax > m_run + 8.0f;  // also on the first tile with a visible key
        const float m_use = up ? tmax : m_run;
        const float alpha = up ? __builtin_amdgcn_exp2f(m_run - tmax) : 1.0f;
        if (__ballot(up)) {  // rare: a real branch, not a multiply by 1 on every tile
            float a = alpha;
            __asm__ volatile("" : "+v"(a));
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int v = 0; v < 16; ++v) o[dt][v] *= a;
        }
        m_run = m_use;
        const float nm = m_use == -INFINITY ? 0.f : -m_use;  // no visible key yet: every p is 0
        float psum = 0.f;
        u32x4 hw[2], lw[2];  // P^T operand of 16-key step cc: values 8 cc .. 8 cc + 7, as hi + lo bf16
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[8 * cc + e], scale_log2, nm));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[8 * cc + e + 1], scale_log2, nm));
                psum += p0;
                psum += p1;
                const uint32_t h = pack_bf2(p0, p1);
                hw[cc][e / 2] = h;
                lw[cc][e / 2] = pack_bf2(p0 - __uint_as_float(h << 16), p1 - __uint_as_float(h & 0xffff0000u));
            }
        const bf16x8 phi[2] = {__builtin_bit_cast(bf16x8, hw[0]), __builtin_bit_cast(bf16x8, hw[1])};
        const bf16x8 plo[2] = {__builtin_bit_cast(bf16x8, lw[0]), __builtin_bit_cast(bf16x8, lw[1])};
        const f32x2 ps2 = halves32(psum);
        psum = ps2[0] + ps2[1];
        l_run = l_run * alpha + psum;
        // V^T operand: group gi reads rows 32 par + 16 cc + 4 (gi / 2) (+ 8) and columns
        // 32 dt + 16 (gi % 2) + 0..15; lane r of the group receives 4 keys of column 16 (gi % 2) + r
        // with 8 waves every V^T read is issued before the first P.V MFMA (pinned as the K reads)
        constexpr int NVQ = HOIST ? D / 32 : 1;
        s16x4 vq[NVQ][2][2];
        auto vread = [&](int dt, int cc, s16x4 &lo4, s16x4 &hi4) {
            const int d0 = 32 * dt + 16 * (gi & 1) + 4 * (sl & 3);
            const int r0 = 32 * par + 16 * cc + 4 * (gi >> 1) + (sl >> 2), r1 = r0 + 8;
            lo4 = lds_tr_b64((const uint16_t *)(Vs + r0 * RB + (((d0 >> 3) ^ (4 * (r0 & 3))) << 4) + ((d0 >> 2) & 1) * 8));
            hi4 = lds_tr_b64((const uint16_t *)(Vs + r1 * RB + (((d0 >> 3) ^ (4 * (r1 & 3))) << 4) + ((d0 >> 2) & 1) * 8));
        };
        if constexpr (HOIST) {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) vread(dt, cc, vq[HOIST ? dt : 0][cc][0], vq[HOIST ? dt : 0][cc][1]);
        }
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const int qd = HOIST ? dt : 0;
                if constexpr (!HOIST) vread(dt, cc, vq[0][cc][0], vq[0][cc][1]);
                bf16x8 vf;
                short *vs = (short *)&vf;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    vs[e] = vq[qd][cc][0][e];
                    vs[4 + e] = vq[qd][cc][1][e];
                }
                o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, phi[cc], o[dt], 0, 0, 0);
                o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, plo[cc], o[dt], 0, 0, 0);
            }
        if constexpr (HOIST) {
            __builtin_amdgcn_sched_group_barrier(0x100, 4 * D / 32, 0);  // the DS reads
            __builtin_amdgcn_sched_group_barrier(0x008, 4 * D / 32, 0);  // then the MFMAs
        }
    }
    // merge the key parts of each head: part w combines the (m, l, O) of every part for its own
    // output columns; the sums run over the parts in part order
    __syncthreads();  // every wave is done with the K/V tiles
    // O of (head, source part, column tile dt) at slot dt (dt below the part's own tiles) or dt - DP,
    // as [v / 4][lane][v % 4] (16-byte accesses); then m[32], l[32] of (head, part)
    auto obuf = [&](int w, int dt) {
        const int slot = dt < w * F::DP ? dt : dt - F::DP;
        return (float *)(fa_smem + ((hw * F::NP + w) * F::OSL + slot) * F::OB);
    };
    auto mlbuf = [&](int w) { return (float *)(fa_smem + F::MERGE_O + (hw * F::NP + w) * 2 * 32 * 4); };
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
        if (dt / F::DP == par) continue;  // this part's own columns stay in registers
        float *mb = obuf(par, dt);
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4)
            *(f32x4 *)&mb[(v4 * 64 + lane) * 4] = f32x4{o[dt][4 * v4], o[dt][4 * v4 + 1], o[dt][4 * v4 + 2], o[dt][4 * v4 + 3]};
    }
    if (lane < 32) {
        mlbuf(par)[lane] = m_run;
        mlbuf(par)[32 + lane] = l_run;
    }
    __syncthreads();
    if (t0 + qi < T) {
        float mw[F::NP], lw[F::NP], a[F::NP], m = -INFINITY, lsum = 0.f;
#pragma unroll
        for (int w = 0; w < F::NP; ++w) {
            mw[w] = mlbuf(w)[qi];
            lw[w] = mlbuf(w)[32 + qi];
            m = fmaxf(m, mw[w]);
        }
#pragma unroll
        for (int w = 0; w < F::NP; ++w) {
            a[w] = __builtin_amdgcn_exp2f(mw[w] - m);
            lsum += lw[w] * a[w];
        }
        const float inv = 1.0f / lsum;
        bf16 *dst = out + (size_t)tq * H * D + (size_t)h * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            if (dt / F::DP != par) continue;
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                float r[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) r[e] = 0.f;
#pragma unroll
                for (int w = 0; w < F::NP; ++w) {
                    f32x4 pv;
                    if (w == par) pv = f32x4{o[dt][4 * v4], o[dt][4 * v4 + 1], o[dt][4 * v4 + 2], o[dt][4 * v4 + 3]};
                    else pv = *(const f32x4 *)&obuf(w, dt)[(v4 * 64 + lane) * 4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) r[e] = w ? r[e] + pv[e] * a[w] : pv[e] * a[w];
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) r[e] *= inv;
                uint2 wd;
                wd.x = pack_bf2(r[0], r[1]);
                wd.y = pack_bf2(r[2], r[3]);
                *(uint2 *)&dst[32 * dt + 8 * v4 + 4 * hh] = wd;
            }
        }
    }
}

// paired: block bi takes query tiles ntiles - 1 - bi and bi (their key-tile counts sum to about the
// same for every bi), so one wave of blocks covers the causal triangle evenly; otherwise block bi
// takes tile ntiles - 1 - bi (heaviest first).
template <int G>
__global__ void __launch_bounds__(64 * FaGeo<G>::NW) attn_prefill_fa_kernel(const bf16 *__restrict__ q, const bf16 *__restrict__ Kc,
                                                                  const bf16 *__restrict__ Vc, int T, int H, int KV,
                                                                  int cap, int p0, int window, float scale_log2,
                                                                  int paired, bf16 *__restrict__ out) {
    extern __shared__ __attribute__((aligned(1024))) unsigned char fa_smem[];
    const int ntiles = (T + 31) / 32;
    const int bi = (int)(blockIdx.x / KV), g = blockIdx.x % KV;
    const int qa = ntiles - 1 - bi;
    fa_query_tile<G>(fa_smem, q, Kc, Vc, T, H, cap, p0, window, scale_log2, out, qa, g);
    if (paired && bi < qa) {
        __syncthreads();  // every wave is done with the merge buffers before the next tile's copies land
        fa_query_tile<G>(fa_smem, q, Kc, Vc, T, H, cap, p0, window, scale_log2, out, bi, g);
    }
}

template <int G>
static hipError_t prefill_fa(const bf16 *q, const bf16 *k, const bf16 *v, int T, int H, int KV, int cap, int p0,
                             int window, float sl2, bf16 *out, hipStream_t s) {
    const size_t lds = FaGeo<G>::LDS;
    static bool attr = false;
    if (!attr) {
        const hipError_t e = hipFuncSetAttribute((const void *)attn_prefill_fa_kernel<G>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr = true;
    }
    const int ntiles = (T + 31) / 32;
    // pairs only when they still give at least one block per CU
    const int paired = (ntiles + 1) / 2 * KV >= 256;
    const int nb = paired ? (ntiles + 1) / 2 : ntiles;
    attn_prefill_fa_kernel<G><<<nb * KV, 64 * FaGeo<G>::NW, lds, s>>>(q, k, v, T, H, KV, cap, p0, window, sl2, paired,
                                                                      out);
    return hipGetLastError();
}

// ------------------------------------------------------------ dispatch
template <typename T, int D, int G>
static void decode_launch(bool fused, dim3 grid, size_t lds, hipStream_t s, const void *q, const void *qkv, int H,
                          int KV, const void *qn, const void *kn, const void *bias, float eps, const void *cs,
                          const void *sn, void *kc, void *vc, int cap, int lo, int nkeys, int chunk, float scale,
                          float *ws, int nsplit) {
    if (fused)
        attn_decode_fused_kernel<T, D, G><<<grid, 256, lds, s>>>((const T *)qkv, H, KV, (const T *)qn, (const T *)kn,
                                                                  (const T *)bias, eps, (const T *)cs, (const T *)sn,
                                                                  (T *)kc, (T *)vc, cap, lo, nkeys, chunk, scale, ws,
                                                                  nsplit);
    else
        attn_decode_kernel<T, D, G><<<grid, 256, lds, s>>>((const T *)q, (const T *)kc, (const T *)vc, cap, lo, nkeys,
                                                            chunk, scale, ws, nsplit);
}

template <typename T, int D>
static hipError_t decode_t(bool fused, const void *q, const void *qkv, int H, int KV, const void *qn, const void *kn,
                           const void *bias, float eps, const void *cs, const void *sn, void *kc, void *vc, int cap,
                           int nkeys, int window, void *out, float *ws, hipStream_t s) {
    const int G = H / KV;
    const int lo = window_lo(nkeys - 1, window), nvis = nkeys - lo;  // keys lo..nkeys-1
    const int chunk = decode_chunk(nvis, KV);
    const int nsplit = (nvis + chunk - 1) / chunk;
    const float scale = (float)(1.0 / sqrt((double)D));
    const size_t lds = ((size_t)G * chunk + 4 * (size_t)G * D) * sizeof(float);
    const dim3 grid(nsplit, KV);
#define DECODE_CASE(GG)                                                                                          \
    case GG:                                                                                                     \
        decode_launch<T, D, GG>(fused, grid, lds, s, q, qkv, H, KV, qn, kn, bias, eps, cs, sn, kc, vc, cap, lo,  \
                                nkeys, chunk, scale, ws, nsplit);                                                \
        break;
    switch (G) {
        DECODE_CASE(1) DECODE_CASE(2) DECODE_CASE(4) DECODE_CASE(8)
    default: return hipErrorInvalidValue;
    }
#undef DECODE_CASE
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    attn_combine_kernel<T, D><<<H, 256, 0, s>>>(ws, nsplit, (T *)out);
    return hipGetLastError();
}

hipError_t launch_attention_decode_fused(int dt, const void *qkv, int H, int KV, int D, const void *q_norm,
                                         const void *k_norm, const void *bias, float eps, const void *cos_t,
                                         const void *sin_t, int p0, int cap, int window, void *k_cache,
                                         void *v_cache, void *out, float *ws, hipStream_t s) {
    if ((q_norm == nullptr) != (k_norm == nullptr)) return hipErrorInvalidValue;
    const int nkeys = p0 + 1;
    if (dt == DT_BF16)
        return D == 128 ? decode_t<bf16, 128>(true, nullptr, qkv, H, KV, q_norm, k_norm, bias, eps, cos_t, sin_t,
                                              k_cache, v_cache, cap, nkeys, window, out, ws, s)
                        : decode_t<bf16, 64>(true, nullptr, qkv, H, KV, q_norm, k_norm, bias, eps, cos_t, sin_t,
                                             k_cache, v_cache, cap, nkeys, window, out, ws, s);
    return D == 128 ? decode_t<float, 128>(true, nullptr, qkv, H, KV, q_norm, k_norm, bias, eps, cos_t, sin_t, k_cache,
                                           v_cache, cap, nkeys, window, out, ws, s)
                    : decode_t<float, 64>(true, nullptr, qkv, H, KV, q_norm, k_norm, bias, eps, cos_t, sin_t, k_cache,
                                          v_cache, cap, nkeys, window, out, ws, s);
}

template <typename T, int D, int G>
static void batch_launch(dim3 grid, size_t lds, hipStream_t s, const T *qkv, int nqkv, int H, int KV, const T *qn,
                         const T *kn, const T *bias, float eps, const T *cs, const T *sn, const DecodeBatch &bt,
                         int cap, float scale, float *ws, size_t stride) {
    attn_decode_fused_batch_kernel<T, D, G><<<grid, 256, lds, s>>>(qkv, nqkv, H, KV, qn, kn, bias, eps, cs, sn, bt, cap,
                                                                   scale, ws, stride);
}

template <typename T, int D>
static hipError_t decode_batch_t(const void *qkv, int B, int H, int KV, const void *qn, const void *kn,
                                 const void *bias, float eps, const void *cs, const void *sn, void *const *kc,
                                 void *const *vc, const int *p, int cap, int window, void *out, float *ws,
                                 hipStream_t s) {
    const int G = H / KV;
    DecodeBatch bt{};
    int maxsplit = 0, maxchunk = 0;
    for (int b = 0; b < B; ++b) {
        bt.kc[b] = kc[b];
        bt.vc[b] = vc[b];
        bt.p[b] = p[b];
        bt.lo[b] = window_lo(p[b], window);
        const int nvis = p[b] + 1 - bt.lo[b];
        bt.chunk[b] = decode_chunk(nvis, KV);
        bt.nsplit[b] = (nvis + bt.chunk[b] - 1) / bt.chunk[b];
        maxsplit = bt.nsplit[b] > maxsplit ? bt.nsplit[b] : maxsplit;
        maxchunk = bt.chunk[b] > maxchunk ? bt.chunk[b] : maxchunk;
    }
    const float scale = (float)(1.0 / sqrt((double)D));
    const size_t lds = ((size_t)G * maxchunk + 4 * (size_t)G * D) * sizeof(float);
    const size_t stride = seat_part_words(H, D, cap);
    const int nqkv = (H + 2 * KV) * D;
    const dim3 grid(maxsplit, KV, B);
    const T *q = (const T *)qkv, *qnn = (const T *)qn, *knn = (const T *)kn, *c = (const T *)cs, *sv = (const T *)sn;
    const T *bb = (const T *)bias;
    switch (G) {
    case 1: batch_launch<T, D, 1>(grid, lds, s, q, nqkv, H, KV, qnn, knn, bb, eps, c, sv, bt, cap, scale, ws, stride); break;
    case 2: batch_launch<T, D, 2>(grid, lds, s, q, nqkv, H, KV, qnn, knn, bb, eps, c, sv, bt, cap, scale, ws, stride); break;
    case 4: batch_launch<T, D, 4>(grid, lds, s, q, nqkv, H, KV, qnn, knn, bb, eps, c, sv, bt, cap, scale, ws, stride); break;
    case 8: batch_launch<T, D, 8>(grid, lds, s, q, nqkv, H, KV, qnn, knn, bb, eps, c, sv, bt, cap, scale, ws, stride); break;
    default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    attn_combine_batch_kernel<T, D><<<dim3(H, B), 256, 0, s>>>(ws, stride, bt, H, (T *)out);
    return hipGetLastError();
}

hipError_t launch_attention_decode_batch(int dt, const void *qkv, int B, int H, int KV, int D, const void *q_norm,
                                         const void *k_norm, const void *bias, float eps, const void *cos_t,
                                         const void *sin_t, void *const *k_cache, void *const *v_cache, const int *p,
                                         int cap, int window, void *out, float *ws, hipStream_t s) {
    if (B < 1 || B > DECODE_MAXB) return hipErrorInvalidValue;
    if ((q_norm == nullptr) != (k_norm == nullptr)) return hipErrorInvalidValue;
    if (dt == DT_BF16)
        return D == 128 ? decode_batch_t<bf16, 128>(qkv, B, H, KV, q_norm, k_norm, bias, eps, cos_t, sin_t, k_cache,
                                                    v_cache, p, cap, window, out, ws, s)
                        : decode_batch_t<bf16, 64>(qkv, B, H, KV, q_norm, k_norm, bias, eps, cos_t, sin_t, k_cache,
                                                   v_cache, p, cap, window, out, ws, s);
    return D == 128 ? decode_batch_t<float, 128>(qkv, B, H, KV, q_norm, k_norm, bias, eps, cos_t, sin_t, k_cache,
                                                 v_cache, p, cap, window, out, ws, s)
                    : decode_batch_t<float, 64>(qkv, B, H, KV, q_norm, k_norm, bias, eps, cos_t, sin_t, k_cache,
                                                v_cache, p, cap, window, out, ws, s);
}

hipError_t launch_attention(int dt, const void *q, const void *k_cache, const void *v_cache, int T, int H, int KV,
                            int D, int cap, int p0, int window, void *out, float *ws, size_t ws_bytes, hipStream_t s) {
    (void)ws_bytes;
    const float scale = (float)(1.0 / sqrt((double)D));
    if (T == 1) {
        const int nkeys = p0 + 1;
        void *kc = (void *)k_cache, *vc = (void *)v_cache;
        if (dt == DT_BF16)
            return D == 128 ? decode_t<bf16, 128>(false, q, nullptr, H, KV, nullptr, nullptr, nullptr, 0.f, nullptr,
                                                  nullptr, kc, vc, cap, nkeys, window, out, ws, s)
                            : decode_t<bf16, 64>(false, q, nullptr, H, KV, nullptr, nullptr, nullptr, 0.f, nullptr,
                                                 nullptr, kc, vc, cap, nkeys, window, out, ws, s);
        return D == 128 ? decode_t<float, 128>(false, q, nullptr, H, KV, nullptr, nullptr, nullptr, 0.f, nullptr,
                                               nullptr, kc, vc, cap, nkeys, window, out, ws, s)
                        : decode_t<float, 64>(false, q, nullptr, H, KV, nullptr, nullptr, nullptr, 0.f, nullptr,
                                              nullptr, kc, vc, cap, nkeys, window, out, ws, s);
    }
    if (dt == DT_BF16) {
        const float sl2 = scale * 1.4426950408889634f;
        const bf16 *qq = (const bf16 *)q, *kk = (const bf16 *)k_cache, *vv = (const bf16 *)v_cache;
        bf16 *oo = (bf16 *)out;
        const int G = H / KV;
        if (D == 128) {
            if (G == 1) return prefill_fa<1>(qq, kk, vv, T, H, KV, cap, p0, window, sl2, oo, s);
            if (G == 2) return prefill_fa<2>(qq, kk, vv, T, H, KV, cap, p0, window, sl2, oo, s);
            if (G == 4) return prefill_fa<4>(qq, kk, vv, T, H, KV, cap, p0, window, sl2, oo, s);
            if (G == 8) return prefill_fa<8>(qq, kk, vv, T, H, KV, cap, p0, window, sl2, oo, s);
            return hipErrorInvalidValue;
        }
        const int QB = G >= 4 ? 16 : 64 / G, NT = 64 * (G >= 8 ? 8 : 4);
        const dim3 grid((T + QB - 1) / QB, KV);
#define PREFILL_CASE(DD, GG)                                                                                   \
    if (D == DD && G == GG) {                                                                                  \
        attn_prefill_mfma_kernel<DD, GG><<<grid, NT, 0, s>>>(qq, kk, vv, T, H, KV, cap, p0, window, sl2, oo);  \
        return hipGetLastError();                                                                              \
    }
        PREFILL_CASE(128, 1) PREFILL_CASE(128, 2) PREFILL_CASE(128, 4) PREFILL_CASE(128, 8)
        PREFILL_CASE(64, 1) PREFILL_CASE(64, 2) PREFILL_CASE(64, 4) PREFILL_CASE(64, 8)
#undef PREFILL_CASE
        return hipErrorInvalidValue;
    }
    attn_rowwise_kernel<float><<<dim3(T, H), 64, 0, s>>>((const float *)q, (const float *)k_cache,
                                                          (const float *)v_cache, H, KV, D, cap, p0, window, scale,
                                                          (float *)out);
    return hipGetLastError();
}

}  // namespace q3
