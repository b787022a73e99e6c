// kernels_decode_mk.hip -- the whole T = 1 decode step of a dense bf16 stack as one
// persistent kernel.
//
// What is computed is the layer of "maya2_mlx/backbone.py" (Backbone.forward and its
// docstring's rounding points) for one token at position p, through every layer, then the
// final norm; the kernels of kernels_linear.hip / kernels_attn.hip compute the same values.
//
// Why one kernel.  A decode layer is six dependent steps (q|k|v projection, split-K
// attention, split merge, o_proj + residual, gate|up + SwiGLU, down) whose weight streams are
// 1 - 50 MB each.  As separate kernels every step pays launch, ramp-up and drain (~3-5 us on
// gfx950), which is more than the 1.3 - 2.6 us the small steps need at HBM speed.  Here 256
// blocks of 8 waves (one block per CU, co-resident) run all steps of all layers; each wave
// issues its next steps' weight loads (registers, 128-bit non-temporal) before it waits for
// the current step's inputs, so HBM streams while the exchange completes.
//
// Exchange protocol between blocks (no grid barrier, no cache-maintenance fences): every
// value handed to other blocks is written as one 32-bit word (tag << 16 | bf16 bits) or one
// 64-bit word (tag << 32 | fp32 bits) with an agent-scope relaxed atomic store, which
// writes through the non-coherent per-XCD L2; consumers poll exactly the words they need
// with agent-scope relaxed atomic loads until every tag equals the expected tag.  The tag is
// (call counter * 64 + layer) mod 2^16; the counter lives in device memory and is advanced
// by block 0 at the end of the step, so graph replays of the same launch get fresh tags.
// Every step's outputs go to a buffer that is rewritten only after all blocks have consumed
// them: each full-vector exchange is a point every block passes only after every block has
// finished the preceding steps.  Polls are bounded; a timeout sets bit 1 of the device
// error word (the step's result is then invalid).
#include "attn_core.h"
#include "common.h"
#include "kernels.h"

namespace q3 {
namespace mk {

constexpr int NB = 256;        // blocks
constexpr int NWB = 8;         // waves per block
constexpr int NT = 64 * NWB;   // threads per block
constexpr int NW = NB * NWB;   // waves in the grid
constexpr int D = 128;         // head dimension
constexpr int CHUNK_MAX = 256; // keys per attention split
constexpr int NSPLIT_MAX = 256;
constexpr long SPIN = 1L << 21;  // poll rounds before a waiter gives up (order of a second)

struct DevLayer {
    const bf16 *in_norm, *post_norm, *q_norm, *k_norm, *qkv, *o, *gu, *down;
};

struct Args {
    const DevLayer *layers;
    int n_layers, H, KV, cap, p, nsplit, chunk;
    float eps, scale;
    const bf16 *x, *final_norm, *cos_t, *sin_t;
    bf16 *out, *kc, *vc;
    uint32_t *x_qkv, *x_a, *x_h2, *x_m, *x_pend;
    uint64_t *x_part;
    unsigned *ctr;
    int *err;
};

__device__ __forceinline__ void xstore(uint32_t *p, uint32_t w) {
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void xstore64(uint64_t *p, uint64_t w) {
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t xload(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t xload64(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t tagw(unsigned tag, float v) { return (tag << 16) | f2bf_bits(v); }

// Poll bookkeeping: after SPIN rounds a waiter gives up and sets bit 1 of the error word;
// every 256 rounds it also gives up when another waiter already has, so a step that cannot
// complete (another block never ran) ends the whole grid after about one SPIN period
// instead of one per remaining poll.
__device__ __forceinline__ bool spin_out(long s, int *err) {
    if (s > SPIN) {
        atomicOr(err, 2);
        return true;
    }
    return (s & 255) == 0 && (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 2);
}

// Wait for words src[t], t < n, to carry `tag`; their bf16 payloads go to dst[t] (LDS).
// Thread tid owns t = tid + NT * k; all its loads are in flight together.
template <int NPT>
__device__ __forceinline__ void poll_bf16(const uint32_t *src, int n, unsigned tag, uint16_t *dst, int *err) {
    uint32_t v[NPT];
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
        const int t = threadIdx.x + NT * k;
        v[k] = t < n ? xload(src + t) : (tag << 16);
    }
    long s = 0;
    while (true) {
        bool ok = true;
#pragma unroll
        for (int k = 0; k < NPT; ++k) ok &= (v[k] >> 16) == tag;
        if (ok) break;
        if (spin_out(++s, err)) break;
#pragma unroll
        for (int k = 0; k < NPT; ++k) {
            const int t = threadIdx.x + NT * k;
            if ((v[k] >> 16) != tag) v[k] = xload(src + t);
        }
    }
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
        const int t = threadIdx.x + NT * k;
        if (t < n) dst[t] = (uint16_t)(v[k] & 0xffffu);
    }
}

// Keeps the compiler from moving memory operations (the weight prefetches in particular)
// across step boundaries, which would stretch their register live ranges.
__device__ __forceinline__ void step_fence() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ float bfv(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

// Sum over the block (NT threads); every thread gets the total.
__device__ __forceinline__ float bsum(float v, float *red) {
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < NWB; ++i) t += red[i];
    return t;
}

// ys[i] = rho(w[i] * rho(hs[i] * r)), r = 1/sqrt(mean(hs^2) + eps), i < n (n = NT * NPT).
template <int NPT>
__device__ __forceinline__ void rmsnorm_lds(const float *hs, const bf16 *__restrict__ w, float eps, uint16_t *ys,
                                            float *red) {
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
        const float v = hs[threadIdx.x + NT * k];
        ss += v * v;
    }
    const float r = 1.0f / sqrtf(bsum(ss, red) / (float)(NT * NPT) + eps);
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
        const int i = threadIdx.x + NT * k;
        ys[i] = (uint16_t)f2bf_bits(to_f(w[i]) * rho<bf16>(hs[i] * r));
    }
}

// Weight-row prefetch: row `row` of a [rows][64*8*CH] bf16 matrix, CH 16-byte chunks per lane.
template <int CH>
__device__ __forceinline__ void ld_row(const bf16 *__restrict__ W, size_t row, int K, u32x4 *r) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int c = 0; c < CH; ++c) r[c] = ld_stream(W + row * K + (size_t)(lane + 64 * c) * 8);
}
// Dot of a prefetched row with the LDS activation ys (bf16 bits), summed over the wave.
template <int CH>
__device__ __forceinline__ float dot_row(const u32x4 *r, const uint16_t *ys) {
    const int lane = threadIdx.x & 63;
    float a = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        float w[8], x[8];
        Vec<bf16>::expand(r[c], w);
        Vec<bf16>::expand(*(const u32x4 *)&ys[(lane + 64 * c) * 8], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) a += w[e] * x[e];
    }
    return wave_sum(a);
}

// HCH: 16-byte chunks per lane of a hidden-size row (hidden = 512 * HCH); ICH likewise for
// an intermediate-size row; QR q|k|v rows, UR gate/up pairs per wave; G query heads per kv head.
template <int HCH, int ICH, int G, int QR, int UR>
__global__ void __launch_bounds__(NT) decode_mk_kernel(Args A) {
    constexpr int HID = 512 * HCH, IM = 512 * ICH;
    constexpr int HPT = HID / NT, IPT = IM / NT;  // words per thread of a hidden / intermediate vector
    constexpr int XMAX = HID > IM ? HID : IM;
    __shared__ float hs[HID];                       // this block's copy of the residual stream h
    __shared__ __attribute__((aligned(16))) uint16_t ys[XMAX];  // current projection input (bf16 bits)
    __shared__ __attribute__((aligned(16))) uint16_t qraw[G * D + 2 * D];
    __shared__ float qs[G * D], kvs[2 * D];
    __shared__ float sc[G * CHUNK_MAX];
    __shared__ float red[NWB * G * D];
    __shared__ float mrow[G], lrow[G], rsum[NWB];
    __shared__ float pm[NSPLIT_MAX], pl[NSPLIT_MAX];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, b = blockIdx.x;
    const int gw = b * NWB + wave;
    const int H = A.H, KV = A.KV;
    const int p = A.p, nkeys = p + 1;
    const unsigned tag0 = A.ctr[0] * 64u;
    const int bpg = NB / KV;                 // attention blocks per kv head (= splits)
    const int ag = b / bpg, as = b % bpg;    // this block's (kv head, split)
    const int j0 = as * A.chunk, j1 = min(nkeys, j0 + A.chunk);
    const bool has_p = j0 < nkeys && j1 == nkeys;
    const int dpb = H * D / NB;              // merged attention outputs per block
    const int mh = b / (NB / H), md0 = (b % (NB / H)) * dpb;

    for (int k = 0; k < HPT; ++k) hs[tid + NT * k] = to_f(A.x[tid + NT * k]);

    u32x4 wq[QR][HCH];  // next q|k|v rows (loop-carried across layers)
    {
        const DevLayer L0 = A.layers[0];
#pragma unroll
        for (int r = 0; r < QR; ++r) ld_row<HCH>(L0.qkv, (size_t)gw * QR + r, HID, wq[r]);
    }

    for (int l = 0; l < A.n_layers; ++l) {
        const DevLayer L = A.layers[l];
        const unsigned tag = (tag0 + (unsigned)l) & 0xffffu;
        const unsigned ptag = (tag0 + (unsigned)l - 1u) & 0xffffu;
        bf16 *Kg = A.kc + ((size_t)l * KV + ag) * A.cap * D;
        bf16 *Vg = A.vc + ((size_t)l * KV + ag) * A.cap * D;

        // ---------------- step 1: h = rho(h + pend); y = RMSNorm(h); q|k|v rows
        u32x4 kp[DEC_PF], vp[DEC_PF];
        decode_prefetch<bf16, D, NWB>(Kg, Vg, j0, j1, kp, vp);
        if (l > 0) {
            poll_bf16<HPT>(A.x_pend, HID, ptag, ys, A.err);
            __syncthreads();
            for (int k = 0; k < HPT; ++k) {
                const int i = tid + NT * k;
                hs[i] = rho<bf16>(hs[i] + bfv(ys[i]));
            }
            __syncthreads();
        }
        rmsnorm_lds<HPT>(hs, L.in_norm, A.eps, ys, rsum);
        __syncthreads();
#pragma unroll
        for (int r = 0; r < QR; ++r) {
            const float acc = dot_row<HCH>(wq[r], ys);
            if (lane == 0) xstore(A.x_qkv + (size_t)gw * QR + r, tagw(tag, acc));
        }

        step_fence();
        // ---------------- step 2: per-head q/k norm + RoPE + cache write, split-K attention
        u32x4 wo[HCH];
        ld_row<HCH>(L.o, (size_t)gw, HID, wo);
        poll_bf16<(G * D + NT - 1) / NT>(A.x_qkv + (size_t)ag * G * D, G * D, tag, qraw, A.err);
        if (has_p) {
            poll_bf16<1>(A.x_qkv + (size_t)(H + ag) * D, D, tag, qraw + G * D, A.err);
            poll_bf16<1>(A.x_qkv + (size_t)(H + KV + ag) * D, D, tag, qraw + G * D + D, A.err);
        }
        __syncthreads();
        {
            constexpr int half = D / 2;
            const int nheads = G + (has_p ? 1 : 0);
            for (int hh = wave; hh < nheads; hh += NWB) {
                const bool is_q = hh < G;
                const uint16_t *row = qraw + hh * D;
                const bf16 *wn = is_q ? L.q_norm : L.k_norm;
                const float x1 = bfv(row[lane]), x2 = bfv(row[lane + half]);
                const float r = 1.0f / sqrtf(wave_sum(x1 * x1 + x2 * x2) / (float)D + A.eps);
                const float n1 = rho<bf16>(to_f(wn[lane]) * rho<bf16>(x1 * r));
                const float n2 = rho<bf16>(to_f(wn[lane + half]) * rho<bf16>(x2 * r));
                const float c1 = to_f(A.cos_t[(size_t)p * D + lane]), s1 = to_f(A.sin_t[(size_t)p * D + lane]);
                const float c2 = to_f(A.cos_t[(size_t)p * D + lane + half]);
                const float s2 = to_f(A.sin_t[(size_t)p * D + lane + half]);
                const float o1 = rho<bf16>(n1 * c1 - n2 * s1), o2 = rho<bf16>(n2 * c2 + n1 * s2);
                if (is_q) {
                    qs[hh * D + lane] = o1;
                    qs[hh * D + lane + half] = o2;
                } else {
                    kvs[lane] = o1;
                    kvs[lane + half] = o2;
                    Kg[(size_t)p * D + lane] = from_f<bf16>(o1);
                    Kg[(size_t)p * D + lane + half] = from_f<bf16>(o2);
                    const uint16_t *vr = qraw + (G + 1) * D;
                    Vg[(size_t)p * D + lane] = bf16{vr[lane]};
                    Vg[(size_t)p * D + lane + half] = bf16{vr[lane + half]};
                    kvs[D + lane] = bfv(vr[lane]);
                    kvs[D + lane + half] = bfv(vr[lane + half]);
                }
            }
        }
        __syncthreads();
        if (j0 < nkeys) {
            decode_core_lds<bf16, D, G, NWB>(qs, Kg, Vg, kp, vp, j0, j1, has_p ? p : -1, kvs, kvs + D, A.scale, sc,
                                             A.chunk, red, mrow, lrow);
            for (int idx = tid; idx < G * D; idx += NT) {
                const int i = idx / D, d = idx % D;
                const float v = decode_core_reduce<D, G, NWB>(red, i, d);
                xstore64(A.x_part + ((size_t)(ag * G + i) * A.nsplit + as) * (D + 2) + 2 + d,
                         ((uint64_t)tag << 32) | __float_as_uint(v));
            }
            if (tid < G) {
                uint64_t *pp = A.x_part + ((size_t)(ag * G + tid) * A.nsplit + as) * (D + 2);
                xstore64(pp, ((uint64_t)tag << 32) | __float_as_uint(mrow[tid]));
                xstore64(pp + 1, ((uint64_t)tag << 32) | __float_as_uint(lrow[tid]));
            }
        } else {  // an empty split (fewer keys than splits): max -inf, sum 0
            for (int idx = tid; idx < G * (D + 2); idx += NT) {
                const int i = idx / (D + 2), e = idx % (D + 2);
                const float v = e == 0 ? -INFINITY : 0.f;
                xstore64(A.x_part + ((size_t)(ag * G + i) * A.nsplit + as) * (D + 2) + e,
                         ((uint64_t)tag << 32) | __float_as_uint(v));
            }
        }

        step_fence();
        // ---------------- step 3: merge the splits of (head mh, dims md0 .. md0 + dpb)
        u32x4 wg[UR][HCH], wu[UR][HCH];
#pragma unroll
        for (int r = 0; r < UR; ++r) {
            ld_row<HCH>(L.gu, (size_t)gw * UR + r, HID, wg[r]);
            ld_row<HCH>(L.gu, (size_t)IM + gw * UR + r, HID, wu[r]);
        }
        __syncthreads();  // step 2's reads of red are finished before it becomes the merge buffer
        {
            const int ns = A.nsplit;
            const int nwords = ns * (2 + dpb);
            float *po = red;  // [ns][dpb]
            for (int t = tid; t < nwords; t += NT) {
                const uint64_t *src;
                if (t < 2 * ns) src = A.x_part + ((size_t)mh * ns + t / 2) * (D + 2) + (t % 2);
                else {
                    const int u = t - 2 * ns;
                    src = A.x_part + ((size_t)mh * ns + u / dpb) * (D + 2) + 2 + md0 + u % dpb;
                }
                uint64_t v = xload64(src);
                long sp = 0;
                while ((unsigned)(v >> 32) != tag) {
                    if (spin_out(++sp, A.err)) break;
                    v = xload64(src);
                }
                const float f = __uint_as_float((uint32_t)v);
                if (t < 2 * ns) {
                    if (t % 2 == 0) pm[t / 2] = f;
                    else pl[t / 2] = f;
                } else {
                    po[t - 2 * ns] = f;
                }
            }
            __syncthreads();
            if (tid < dpb) {
                float M = -INFINITY;
                for (int s = 0; s < ns; ++s) M = fmaxf(M, pm[s]);
                float Ls = 0.f, acc = 0.f;
                for (int s = 0; s < ns; ++s) {
                    const float f = __expf(pm[s] - M);
                    Ls += pl[s] * f;
                    acc += po[s * dpb + tid] * f;
                }
                xstore(A.x_a + (size_t)mh * D + md0 + tid, tagw(tag, acc / Ls));
            }
        }

        step_fence();
        // ---------------- step 4: h = rho(h + rho(a . Wo^T)) for this wave's row
        poll_bf16<HPT>(A.x_a, HID, tag, ys, A.err);
        __syncthreads();
        {
            const float acc = dot_row<HCH>(wo, ys);
            if (lane == 0) xstore(A.x_h2 + gw, tagw(tag, hs[gw] + rho<bf16>(acc)));
        }

        step_fence();
        // ---------------- step 5: y2 = RMSNorm(h); gate|up rows + SwiGLU
        __syncthreads();  // every wave has read hs for its residual before it is replaced
        poll_bf16<HPT>(A.x_h2, HID, tag, ys, A.err);
        __syncthreads();
        for (int k = 0; k < HPT; ++k) hs[tid + NT * k] = bfv(ys[tid + NT * k]);
        __syncthreads();
        rmsnorm_lds<HPT>(hs, L.post_norm, A.eps, ys, rsum);
        __syncthreads();
#pragma unroll
        for (int r = 0; r < UR; ++r) {
            const float g = dot_row<HCH>(wg[r], ys);
            const float u = dot_row<HCH>(wu[r], ys);
            if (lane == 0)
                xstore(A.x_m + (size_t)gw * UR + r, tagw(tag, rho<bf16>(silu_f32(rho<bf16>(g))) * rho<bf16>(u)));
        }

        step_fence();
        // ---------------- step 6: pend = rho(m . Wdown^T) for this wave's row
        u32x4 wd[ICH];
        ld_row<ICH>(L.down, (size_t)gw, IM, wd);
        if (l + 1 < A.n_layers) {
            const DevLayer Ln = A.layers[l + 1];
#pragma unroll
            for (int r = 0; r < QR; ++r) ld_row<HCH>(Ln.qkv, (size_t)gw * QR + r, HID, wq[r]);
        }
        __syncthreads();  // ys (y2) fully consumed before it receives m
        poll_bf16<IPT>(A.x_m, IM, tag, ys, A.err);
        __syncthreads();
        {
            const float acc = dot_row<ICH>(wd, ys);
            if (lane == 0) xstore(A.x_pend + gw, tagw(tag, acc));
        }
        __syncthreads();
    }

    // ---------------- out = RMSNorm(rho(h + pend), final_norm) (block 0), then advance the counter
    if (b == 0) {
        const unsigned ltag = (tag0 + (unsigned)A.n_layers - 1u) & 0xffffu;
        poll_bf16<HPT>(A.x_pend, HID, ltag, ys, A.err);
        __syncthreads();
        for (int k = 0; k < HPT; ++k) {
            const int i = tid + NT * k;
            hs[i] = rho<bf16>(hs[i] + bfv(ys[i]));
        }
        __syncthreads();
        rmsnorm_lds<HPT>(hs, A.final_norm, A.eps, ys, rsum);
        __syncthreads();
        for (int k = 0; k < HPT; ++k) {
            const int i = tid + NT * k;
            A.out[i] = bf16{ys[i]};
        }
        if (tid == 0) __hip_atomic_store(A.ctr, tag0 / 64u + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace mk

// ------------------------------------------------------------ host side
size_t decode_mk_workspace(int n_layers, int H, int KV, int hid, int I) {
    const size_t nsplit = mk::NB / (KV > 0 ? KV : 1);
    auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
    const size_t nqkv = (size_t)(H + 2 * KV) * mk::D;
    return al(sizeof(mk::DevLayer) * n_layers) + al(nqkv * 4) + al((size_t)H * mk::D * 4) + al((size_t)hid * 4) +
           al((size_t)I * 4) + al((size_t)hid * 4) + al((size_t)H * nsplit * (mk::D + 2) * 8) + al(256);
}

namespace {
struct MkLayout {
    size_t layers, qkv, a, h2, m, pend, part, ctr;
};
MkLayout mk_layout(int n_layers, int H, int KV, int hid, int I) {
    const size_t nsplit = mk::NB / KV;
    auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
    const size_t nqkv = (size_t)(H + 2 * KV) * mk::D;
    MkLayout L{};
    size_t o = 0;
    L.layers = o; o += al(sizeof(mk::DevLayer) * n_layers);
    L.qkv = o; o += al(nqkv * 4);
    L.a = o; o += al((size_t)H * mk::D * 4);
    L.h2 = o; o += al((size_t)hid * 4);
    L.m = o; o += al((size_t)I * 4);
    L.pend = o; o += al((size_t)hid * 4);
    L.part = o; o += al((size_t)H * nsplit * (mk::D + 2) * 8);
    L.ctr = o;
    return L;
}

template <int HCH, int ICH, int G, int QR, int UR> const void *mk_fn() {
    return (const void *)mk::decode_mk_kernel<HCH, ICH, G, QR, UR>;
}

const void *mk_select(int hid, int I, int G, int nqkv) {
    if (hid == 2048 && I == 6144 && nqkv == 4096 && G == 2) return mk_fn<4, 12, 2, 2, 3>();
    return nullptr;
}
}  // namespace

bool decode_mk_supported(int n_layers, int dt, int n_experts, int quant_bits, int hid, int H, int KV, int D, int I, int cap) {
    if (dt != DT_BF16 || n_experts > 0 || quant_bits != 0 || D != mk::D) return false;
    if (n_layers < 1 || n_layers > 63) return false;  // tags are call * 64 + layer
    if (H % KV || mk::NB % KV || (H * D) != hid || hid != mk::NW || (H * D) % mk::NB) return false;
    const int nsplit = mk::NB / KV;
    if (nsplit > mk::NSPLIT_MAX || (cap + nsplit - 1) / nsplit > mk::CHUNK_MAX) return false;
    if (nsplit * (2 + H * D / mk::NB) > mk::NWB * (H / KV) * mk::D) return false;  // merge buffer fits in LDS
    return mk_select(hid, I, H / KV, (H + 2 * KV) * D) != nullptr;
}

hipError_t decode_mk_init(void *ws, int n_layers, int H, int KV, int hid, int I, const void *layer_ptrs, hipStream_t s) {
    const MkLayout L = mk_layout(n_layers, H, KV, hid, I);
    char *b = (char *)ws;
    hipError_t e = hipMemcpyAsync(b + L.layers, layer_ptrs, sizeof(mk::DevLayer) * n_layers, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return e;
    // exchange words start with tag 0xffff, never the tag of a first call's layer
    e = hipMemsetAsync(b + L.qkv, 0xff, L.ctr - L.qkv, s);
    if (e != hipSuccess) return e;
    e = hipMemsetAsync(b + L.ctr, 0, 256, s);
    if (e != hipSuccess) return e;
    return hipStreamSynchronize(s);  // layer_ptrs is a caller's host array
}

hipError_t launch_decode_mk(void *ws, int n_layers, int H, int KV, int hid, int I, int cap, int p, float eps,
                            const void *x, void *out, const void *final_norm, const void *cos_t, const void *sin_t,
                            void *kc, void *vc, int *err, hipStream_t s) {
    const MkLayout L = mk_layout(n_layers, H, KV, hid, I);
    char *b = (char *)ws;
    const int nsplit = mk::NB / KV;
    mk::Args A;
    A.layers = (const mk::DevLayer *)(b + L.layers);
    A.n_layers = n_layers;
    A.H = H;
    A.KV = KV;
    A.cap = cap;
    A.p = p;
    A.nsplit = nsplit;
    A.chunk = (p + 1 + nsplit - 1) / nsplit;
    A.eps = eps;
    A.scale = (float)(1.0 / sqrt((double)mk::D));
    A.x = (const bf16 *)x;
    A.final_norm = (const bf16 *)final_norm;
    A.cos_t = (const bf16 *)cos_t;
    A.sin_t = (const bf16 *)sin_t;
    A.out = (bf16 *)out;
    A.kc = (bf16 *)kc;
    A.vc = (bf16 *)vc;
    A.x_qkv = (uint32_t *)(b + L.qkv);
    A.x_a = (uint32_t *)(b + L.a);
    A.x_h2 = (uint32_t *)(b + L.h2);
    A.x_m = (uint32_t *)(b + L.m);
    A.x_pend = (uint32_t *)(b + L.pend);
    A.x_part = (uint64_t *)(b + L.part);
    A.ctr = (unsigned *)(b + L.ctr);
    A.err = err;
    const void *fn = mk_select(hid, I, H / KV, (H + 2 * KV) * mk::D);
    if (!fn) return hipErrorInvalidValue;
    void *args[] = {&A};
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(s, &cs);
    if (e != hipSuccess) return e;
    if (cs == hipStreamCaptureStatusNone)
        return hipLaunchCooperativeKernel(fn, dim3(mk::NB), dim3(mk::NT), args, 0, s);
    // graph capture: a plain launch (the grid is one block per CU and fits the device at once)
    return hipLaunchKernel(fn, dim3(mk::NB), dim3(mk::NT), args, 0, s);
}

int decode_mk_max_blocks(int hid, int I, int H, int KV) {
    const void *fn = mk_select(hid, I, H / KV, (H + 2 * KV) * mk::D);
    if (!fn) return 0;
    int per_cu = 0, dev = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, mk::NT, 0) != hipSuccess) return 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
    return per_cu * prop.multiProcessorCount;
}

int decode_mk_blocks() { return mk::NB; }

}  // namespace q3
