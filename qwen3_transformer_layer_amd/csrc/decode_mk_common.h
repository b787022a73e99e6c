// decode_mk_common.h -- device pieces shared by the persistent decode kernels
// (kernels_decode_mk.hip: dense stacks; kernels_decode_moe.hip: Qwen3-MoE stacks).
//
// Block roles, the LDS ring and its handshake, and the exchange protocol between blocks
// are described at the top of kernels_decode_mk.hip; this header holds the constants and
// the helpers both kernels use for them.
#pragma once
#include "common.h"

namespace q3 {
namespace mk {

constexpr int NB = 256;              // blocks, one per CU
constexpr int NC = 8;                // compute waves per block
// Stream waves x chunks in flight per wave.  Before the weight stream carried the non-temporal
// policy, 3 x 3 beat 2 x 4, 3 x 4, 4 x 3 and 4 x 4 on the 1.7B shape (ms per step 0.911 against
// 0.960, 0.939, 0.965, 0.965 on one box) and 3 x 2, 4 x 2 (0.916 against 0.929, 0.947 on
// another).  With it, 4 x 2 edges out 3 x 3 (1.7B 0.703 against 0.707 ms in three interleaved
// pairs on one box, 8-bit even, MoE 1.745 against 1.758), while 2 x 4, 2 x 5 (0.79 to 0.80)
// and 4 x 3 (0.747) lose.
constexpr int NL = 4;                // stream waves per block
constexpr int NCT = 64 * NC;         // compute threads
constexpr int NTH = 64 * (NC + NL);  // threads per block
constexpr int D = 128;               // head dimension
constexpr int HID = 2048;            // hidden size: one chunk is one weight row of HID bf16
constexpr int CHB = HID * 2;         // chunk bytes
constexpr int DL = 2;                // chunks in flight per stream wave while the ring has room
constexpr int KPC = CHB / (D * 2);   // keys per K or V chunk (16)
constexpr int NSPLIT_MAX = 256;
constexpr int MAXL = 63;             // layers (tags are call * 64 + layer)
// Every block reads the whole of each exchanged vector.  Read from one copy, 256 blocks
// would poll the same few KB, which sit in a few memory channels; producers therefore write
// NREP copies, spaced so they fall in different channels, and block b reads copy b % NREP.
// Each copy costs the producers a store per value: on the 1.7B shape 4 copies beat 1, 2, 8
// and 16 (ms per step 1.004, 0.982, 0.977, 0.992, 1.048 for 1, 2, 4, 8, 16 on one box).
constexpr int NREP = 4;
__host__ __device__ constexpr int rep_stride(int words) {  // words between copies
    return ((words * 4 + 4095) / 4096 * 4096 + 1280) / 4;
}
constexpr long SPIN = 1L << 21;      // global poll rounds before a waiter gives up (order of a second)
constexpr long LSPIN = 1L << 22;     // LDS wait rounds before a waiter gives up (order of a second)
static_assert(5 * (DL - 1) <= 63, "vector-memory counter range");
// The thread index behind an empty asm: every call yields a value the compiler cannot prove
// equal to the last one, so per-thread addresses derived from it are recomputed inside the
// layer loop instead of being hoisted out of it and kept live (or spilled) across all steps.
__device__ __forceinline__ int tid_now() {
    int z = 0;
    __asm__ volatile("" : "+s"(z));
    return (int)threadIdx.x + z;
}

// ---------------------------------------------------------------- cross-block exchange
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

// Every wait is bounded.  After SPIN rounds a waiter gives up, sets bit 1 of the error word
// and the block's abort flag (LDS); every 256 rounds it also gives up when the error word or
// the flag shows that another waiter already has, so a step that cannot complete ends the
// whole grid after about one SPIN period instead of one per remaining wait.
__device__ __forceinline__ bool spin_out(long s, int *err, unsigned *abt) {
    if (s > SPIN) {
        atomicOr(err, 2);
        __hip_atomic_store(abt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        return true;
    }
    return (s & 255) == 0 &&
           ((__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 2) ||
            __hip_atomic_load(abt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
}

// Poll pacing.  A block reaches an exchange about when the other blocks do, so a poll round issued
// at once mostly finds words not yet written: the round is wasted, and its loads (one memory
// request per word, from every block) queue ahead of the round that would find the words and of
// the producers' own traffic.  A short pause before the first round (N times 64 clocks) lets that
// round find nearly every word.  Measured on the 1.7B decode step (ms per step, one box): no pause
// 0.893; 16 before the q|k|v, pend, h and SwiGLU polls 0.827, 32 0.794, 64 0.827 (longer pauses
// only add latency); 16 more before the split-partial and merged-output polls 0.791.  Per exchange
// (same box, interleaved runs, 786 us/step with 32 everywhere): 48 before the pend and q|k|v polls
// of the dense kernel 779 us (each alone 782 / 781; 64 at both 787); 20 or 48 before the h or
// SwiGLU polls no better (787-796).
template <int N> __device__ __forceinline__ void poll_pause() { __builtin_amdgcn_s_sleep(N); }
constexpr int PAUSE_VEC = 32;    // before polling a vector every block produces (h, SwiGLU; MoE: all)
constexpr int PAUSE_LONG = 48;   // dense kernel: before the pend and q|k|v polls
constexpr int PAUSE_SPLIT = 16;  // before the split partials and the merged attention output

// Wait for words src[t], t < n, to carry `tag`; their bf16 payloads go to dst[t] (LDS).
// Compute thread tid owns t = tid + NCT * k; all its loads are in flight together.
template <int NPT>
__device__ __forceinline__ void poll_bf16(const uint32_t *src, int n, unsigned tag, uint16_t *dst, int *err,
                                          unsigned *abt, int tid) {
    uint32_t v[NPT];
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
        const int t = tid + NCT * k;
        v[k] = t < n ? xload(src + t) : (tag << 16);
    }
    long s = 0;
    while (true) {
        bool ok = true;
#pragma unroll
        for (int k = 0; k < NPT; ++k) ok &= (v[k] >> 16) == tag;
        if (ok) break;
        if (spin_out(++s, err, abt)) break;
#pragma unroll
        for (int k = 0; k < NPT; ++k) {
            const int t = tid + NCT * k;
            if ((v[k] >> 16) != tag) v[k] = xload(src + t);
        }
    }
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
        const int t = tid + NCT * k;
        if (t < n) dst[t] = (uint16_t)(v[k] & 0xffffu);
    }
}

// The SwiGLU output travels as one 64-bit word per (block, wave): tag << 48 | three bf16
// values, those of the wave's gate|up pairs w, w + NC, w + 2 NC (2048 words instead of 6144,
// four polls per thread instead of twelve).  Word u = block * NC + wave; its values go to
// dst[block * GPB + wave + NC * j].
template <int NPT, int GPB>
__device__ __forceinline__ void poll_m3(const uint64_t *src, int nw, unsigned tag, uint16_t *dst, int *err,
                                        unsigned *abt, int tid) {
    uint64_t v[NPT];
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
        const int t = tid + NCT * k;
        v[k] = t < nw ? xload64(src + t) : ((uint64_t)tag << 48);
    }
    long s = 0;
    while (true) {
        bool ok = true;
#pragma unroll
        for (int k = 0; k < NPT; ++k) ok &= (unsigned)(v[k] >> 48) == tag;
        if (ok) break;
        if (spin_out(++s, err, abt)) break;
#pragma unroll
        for (int k = 0; k < NPT; ++k) {
            const int t = tid + NCT * k;
            if ((unsigned)(v[k] >> 48) != tag) v[k] = xload64(src + t);
        }
    }
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
        const int t = tid + NCT * k;
        if (t < nw) {
            const int bb = t / NC, w = t % NC;
#pragma unroll
            for (int j = 0; j < 3; ++j) dst[bb * GPB + w + NC * j] = (uint16_t)(v[k] >> (16 * j));
        }
    }
}

// ---------------------------------------------------------------- LDS handshakes
__device__ __forceinline__ unsigned lds_acquire(const unsigned *p) {
    return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Wait until the LDS word *p reaches v (>= v).  Bounded like the global polls; on its own
// time-out it raises the block's abort flag (and, where err is given, the error word).
__device__ __forceinline__ void lds_wait_ge(const unsigned *p, unsigned v, unsigned *abt, int *err) {
    long s = 0;
    while (lds_acquire(p) < v) {
        ++s;
        if (s > LSPIN) {
            __hip_atomic_store(abt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            if (err) atomicOr(err, 2);
            return;
        }
        if ((s & 63) == 0 && __hip_atomic_load(abt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) return;
        __builtin_amdgcn_s_sleep(1);
    }
}

// Barrier of the NC compute waves: a monotonic LDS counter; `ep` is the wave's running
// target (NC per barrier passed).
__device__ __forceinline__ void cbar(unsigned *ctr, unsigned &ep, unsigned *abt, int *err, int lane) {
    ep += NC;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (lane == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    lds_wait_ge(ctr, ep, abt, err);
}

// Wait until ring chunk g has landed; returns its slot.
template <int NSL>
__device__ __forceinline__ const unsigned char *chunk_get(const unsigned char *ring, const unsigned *ready,
                                                          unsigned g, unsigned *abt, int *err) {
    const unsigned s = g % NSL, gen = g / NSL;
    lds_wait_ge(ready + s, gen + 1u, abt, err);
    return ring + (size_t)s * CHB;
}
// The wave's reads of chunk g are complete: its slot may be refilled.
template <int NSL> __device__ __forceinline__ void chunk_put(unsigned *done, unsigned g, int lane) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (lane == 0)
        __hip_atomic_fetch_add(done + g % NSL, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ float bfv(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

// A lane's four 16-byte pieces of a 2048-element bf16 vector x in LDS (elements
// (lane + 64 k) * 8 .. + 7, k < 4): loaded once per step, reused for every chunk.
struct X4 {
    u32x4 v[4];
};
__device__ __forceinline__ X4 load_x(const uint16_t *x, int lane) {
    X4 r;
#pragma unroll
    for (int k = 0; k < 4; ++k) r.v[k] = *(const u32x4 *)(x + (lane + 64 * k) * 8);
    return r;
}
// Per-lane partial dot of a 4 KB chunk (2048 bf16 in the same lane interleave) with x, added
// to a; not summed over the wave.  All four LDS reads are issued before the arithmetic, which
// is one v_dot2c_f32_bf16 per pair of elements (bf16 products are exact in fp32; 16 dot
// instructions per lane instead of 32 conversions and 32 FMAs).
__device__ __forceinline__ float dot_chunk(const unsigned char *c, const X4 &x, int lane, float a) {
    u32x4 w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = *(const u32x4 *)(c + k * 1024 + lane * 16);
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // through plain words: a bit cast applied to a vector element directly read element 0
            const uint32_t wq = w[k][q], xq = x.v[k][q];
            a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wq), __builtin_bit_cast(bf16x2, xq), a, false);
        }
    return a;
}

// 8-bit weights: a lane's activations for a row of 2048 codes, elements 16 lane .. + 15
// (first 1 KB of the row's codes) and 1024 + 16 lane .. + 15 (second 1 KB), as bf16 pairs,
// and the fp32 sums of each 16 (the bias term of the group fold).
struct X8 {
    u32x4 v[4];
    float s0, s1;
};
__device__ __forceinline__ X8 load_x8(const uint16_t *x, int lane) {
    X8 r;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        r.v[2 * k] = *(const u32x4 *)(x + 1024 * k + 16 * lane);
        r.v[2 * k + 1] = *(const u32x4 *)(x + 1024 * k + 16 * lane + 8);
    }
    float s[2] = {0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t w = r.v[2 * k + h][q];
                s[k] += bf_lo(w) + bf_hi(w);
            }
    r.s0 = s[0];
    r.s1 = s[1];
    return r;
}
// 16 codes (one 16-byte piece) against 16 activations (two bf16x8): the codes are exact bf16
// values, so each pair is one v_dot2c_f32_bf16 (exact products, fp32 sum).
__device__ __forceinline__ float dot16_codes(u32x4 c, u32x4 xa, u32x4 xb, float a) {
    const bf16x8 c0 = codes8(c[0], c[1]), c1 = codes8(c[2], c[3]);
    const u32x4 w0 = __builtin_bit_cast(u32x4, c0), w1 = __builtin_bit_cast(u32x4, c1);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t wq = w0[q], xq = xa[q];
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wq), __builtin_bit_cast(bf16x2, xq), a, false);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t wq = w1[q], xq = xb[q];
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wq), __builtin_bit_cast(bf16x2, xq), a, false);
    }
    return a;
}
// A lane's part of one row of 2048 codes: pieces p0 (codes 16 lane ..) and p1 (1024 + 16 lane ..)
// of the chunk, with the row's 32 scales at sb[0..31] and biases at sb[32..63]:
// s_g0 (x . q)_0 + b_g0 (sum x)_0 + s_g1 (x . q)_1 + b_g1 (sum x)_1, groups g0 = lane / 4 and
// g1 = 16 + lane / 4.  Not summed over the wave.
__device__ __forceinline__ float dot_q8_row(const unsigned char *c, int p0, int p1, const uint16_t *sb, const X8 &x,
                                            int lane) {
    const u32x4 c0 = *(const u32x4 *)(c + p0 * 1024 + lane * 16), c1 = *(const u32x4 *)(c + p1 * 1024 + lane * 16);
    const int g0 = lane >> 2, g1 = 16 + (lane >> 2);
    const float s0 = bfv(sb[g0]), b0 = bfv(sb[32 + g0]), s1 = bfv(sb[g1]), b1 = bfv(sb[32 + g1]);
    const float P0 = dot16_codes(c0, x.v[0], x.v[1], 0.f), P1 = dot16_codes(c1, x.v[2], x.v[3], 0.f);
    return (s0 * P0 + b0 * x.s0) + (s1 * P1 + b1 * x.s1);
}

// Sum over the compute waves; every compute thread gets the total.  Two alternating
// partial buffers, so one barrier per call suffices.
__device__ __forceinline__ float csum(float v, float (*red)[NC], unsigned &par, unsigned *bar, unsigned &ep,
                                     unsigned *abt, int *err, int tid) {
    v = wave_sum(v);
    float *r = red[par];
    par ^= 1u;
    if ((tid & 63) == 0) r[tid >> 6] = v;
    cbar(bar, ep, abt, err, tid & 63);
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < NC; ++i) t += r[i];
    return t;
}

// Merge of the split-K attention partials of one output dim, from LDS: pm[s], pl[s] are split s's
// max and sum, po[s * dpb + d] its output for dim d (an empty split has max -inf, sum 0).  Thread
// t < LPD dpb takes dim t / LPD and splits t % LPD, + LPD, ...; the LPD lanes of a dim combine by
// xor shuffles, giving a = (sum_s o_s e^(m_s - M)) / (sum_s l_s e^(m_s - M)), M = max_s m_s.
// Returns true on the lane holding a dim's result (t % LPD == 0).  Splitting the serial loop over
// the splits across lanes matters: each step of it is an LDS read's latency.
template <int LPD>
__device__ __forceinline__ bool merge_lds(const float *pm, const float *pl, const float *po, int ns, int dpb, int tid,
                                          float *a) {
    if (tid >= LPD * dpb) return false;
    const int d = tid / LPD, pt = tid % LPD;
    float M = -INFINITY;
    for (int s = pt; s < ns; s += LPD) M = fmaxf(M, pm[s]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY)
        for (int s = pt; s < ns; s += LPD) {
            const float f = __expf(pm[s] - M);
            L += pl[s] * f;
            O += po[s * dpb + d] * f;
        }
    auto comb = [&](float M2, float L2, float O2) {
        const float Mn = fmaxf(M, M2);
        const float f1 = M == -INFINITY ? 0.f : __expf(M - Mn), f2 = M2 == -INFINITY ? 0.f : __expf(M2 - Mn);
        L = L * f1 + L2 * f2;
        O = O * f1 + O2 * f2;
        M = Mn;
    };
    if constexpr (LPD == 8) {
        // DPP lane moves within each group of 8 (VALU, no LDS crossbar round trip): lane i with
        // lane 7 - i, then xor 2, then xor 1 pairs every lane of the group with every other; the
        // combine is symmetric, so all 8 lanes end with the same (M, L, O).  The calling lanes
        // are whole waves.
#pragma unroll
        for (int st = 0; st < 3; ++st) {
            float M2, L2, O2;
            if (st == 0) M2 = Q3_DPP(M, 0x141), L2 = Q3_DPP(L, 0x141), O2 = Q3_DPP(O, 0x141);
            else if (st == 1) M2 = Q3_DPP(M, 0x4e), L2 = Q3_DPP(L, 0x4e), O2 = Q3_DPP(O, 0x4e);
            else M2 = Q3_DPP(M, 0xb1), L2 = Q3_DPP(L, 0xb1), O2 = Q3_DPP(O, 0xb1);
            comb(M2, L2, O2);
        }
    } else {
#pragma unroll
        for (int off = LPD / 2; off > 0; off >>= 1) comb(__shfl_xor(M, off), __shfl_xor(L, off), __shfl_xor(O, off));
    }
    *a = O / L;
    return pt == 0;
}

// 4-byte direct-to-LDS copy: lane l's word lands at LDS byte address lds + 4 l.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma4(const void *g, unsigned lds) {
    __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

}  // namespace mk
}  // namespace q3
