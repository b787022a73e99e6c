// common.h -- shared device helpers of the gfx950 kernels: storage types,
// bf16 round-to-nearest-even, wave64 reductions, 128-bit vector loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q3 {

enum Dt { DT_BF16 = 0, DT_FP32 = 1 };

// bf16 storage: the upper half of a binary32 pattern.
struct bf16 {
    uint16_t u;
};

__device__ __forceinline__ float to_f(bf16 x) { return __uint_as_float((uint32_t)x.u << 16); }
__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 with round-to-nearest-even (NaN stays NaN, quieted), in one gfx950 instruction
// (v_cvt_pk_bf16_f32).  Checked against the integer formulation
// (u + 0x7fff + ((u >> 16) & 1)) >> 16 with NaN -> (u >> 16) | 0x40 on all 2^32 inputs: equal
// everywhere, in the scalar and the packed form.  The integer form compiled to a branch per
// element inside the GEMM epilogues.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f2bf_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

template <typename T> __device__ __forceinline__ T from_f(float f);
template <> __device__ __forceinline__ bf16 from_f<bf16>(float f) { return bf16{(uint16_t)f2bf_bits(f)}; }
template <> __device__ __forceinline__ float from_f<float>(float f) { return f; }

// rho: round to the storage type and back (identity for fp32).
template <typename T> __device__ __forceinline__ float rho(float f) { return to_f(from_f<T>(f)); }

template <typename T> struct DtOf;
template <> struct DtOf<bf16> { static constexpr Dt value = DT_BF16; };
template <> struct DtOf<float> { static constexpr Dt value = DT_FP32; };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// a + w . x over one 16-byte piece of each (8 bf16 or 4 fp32 elements).  bf16 pairs go through
// v_dot2c_f32_bf16 (the products are exact in fp32, the sum is accumulated in fp32); the words
// are copied out of the vectors first (a bit cast applied to a vector element directly was
// compiled as a read of element 0).
template <typename T> __device__ __forceinline__ float dot16(u32x4 w, u32x4 x, float a);
template <> __device__ __forceinline__ float dot16<bf16>(u32x4 w, u32x4 x, float a) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t wq = w[q], xq = x[q];
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wq), __builtin_bit_cast(bf16x2, xq), a, false);
    }
    return a;
}
template <> __device__ __forceinline__ float dot16<float>(u32x4 w, u32x4 x, float a) {
#pragma unroll
    for (int q = 0; q < 4; ++q) a += __uint_as_float(w[q]) * __uint_as_float(x[q]);
    return a;
}

// 16-byte global loads: streamed (non-temporal) for weights read once, plain otherwise.
__device__ __forceinline__ u32x4 ld_stream(const void *p) {
    return __builtin_nontemporal_load((const u32x4 *)p);
}
__device__ __forceinline__ u32x4 ld16(const void *p) { return *(const u32x4 *)p; }

// 16 codes of one 128-bit word against 16 activations: sum_i x_i * q_i (8-bit
// affine weights: kernels_q8.hip, kernels_moe.hip).
__device__ __forceinline__ float dot16_q8(u32x4 c, const float *xf) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int b = 0; b < 4; ++b) a += xf[4 * i + b] * (float)((w[i] >> (8 * b)) & 0xffu);
    return a;
}

// Eight codes (two words, little-endian bytes) as exact bf16 values: the integer through fp32,
// whose low 16 bits are zero for 0..255, then the high halves packed.
__device__ __forceinline__ bf16x8 codes8(uint32_t w0, uint32_t w1) {
    u32x4 r;
    const uint32_t w[2] = {w0, w1};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const float f0 = (float)(w[h] & 0xffu), f1 = (float)((w[h] >> 8) & 0xffu);
        const float f2 = (float)((w[h] >> 16) & 0xffu), f3 = (float)(w[h] >> 24);
        r[2 * h] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
        r[2 * h + 1] = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
    }
    return __builtin_bit_cast(bf16x8, r);
}

// Expand 16 bytes of storage type T into fp32 values: 8 for bf16, 4 for fp32.
template <typename T> struct Vec;
template <> struct Vec<bf16> {
    static constexpr int N = 8;
    __device__ static __forceinline__ void expand(u32x4 v, float *o) {
        o[0] = bf_lo(v.x); o[1] = bf_hi(v.x); o[2] = bf_lo(v.y); o[3] = bf_hi(v.y);
        o[4] = bf_lo(v.z); o[5] = bf_hi(v.z); o[6] = bf_lo(v.w); o[7] = bf_hi(v.w);
    }
};
template <> struct Vec<float> {
    static constexpr int N = 4;
    __device__ static __forceinline__ void expand(u32x4 v, float *o) {
        o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
        o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
    }
};

// Cross-lane reductions on DPP lane moves (VALU; no trip through the LDS crossbar).  The
// wave must be fully active.  DPP controls: quad_perm [1,0,3,2] and [2,3,0,1] (lane ^ 1,
// lane ^ 2), row_half_mirror (lane 7-i within 8), row_mirror (lane 15-i within 16).
#define Q3_DPP(v, ctrl) __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), (ctrl), 0xf, 0xf, false))
// Sum over each 16-lane row; every lane of the row gets the row's total.
__device__ __forceinline__ float row16_sum(float v) {
    v += Q3_DPP(v, 0xb1);
    v += Q3_DPP(v, 0x4e);
    v += Q3_DPP(v, 0x141);
    v += Q3_DPP(v, 0x140);
    return v;
}
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, Q3_DPP(v, 0xb1));
    v = fmaxf(v, Q3_DPP(v, 0x4e));
    v = fmaxf(v, Q3_DPP(v, 0x141));
    v = fmaxf(v, Q3_DPP(v, 0x140));
    return v;
}
__device__ __forceinline__ float lane_f(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// Sum / max over the wave (64 lanes); the result is wave-uniform.
__device__ __forceinline__ float wave_sum(float v) {
    v = row16_sum(v);
    return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
    v = row16_max(v);
    return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

// Sum over a block of nwaves wave64s; every thread gets the total.  red: LDS of >= nwaves floats.
__device__ __forceinline__ float block_sum(float v, float *red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    v = wave_sum(v);
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float t = 0.f;
    for (int i = 0; i < nw; ++i) t += red[i];
    return t;
}

// One 16-byte-per-lane copy from global memory straight into LDS (gfx950
// global_load_lds_dwordx4): lane i's 16 bytes at g land at LDS byte address lds + 16 i
// (lds wave-uniform).  Written as asm so the compiler does not see an LDS write it cannot
// place: with the builtin it conservatively waits for every copy in flight before each later
// LDS access of the issuing wave.  The caller tracks completion with wait_vm (the copies
// count in the wave's vector-memory counter).  M0 carries the LDS address; the nop covers the
// M0-write-to-LDS-DMA hazard.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void *g, unsigned lds) {
    __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds)
                     : "memory", "m0");
}
// The same with the non-temporal policy, for data read once per call (the decode kernels'
// weight and K/V stream): 1.7B decode ~765 -> ~735 us per step, MoE ~1850 -> ~1815 us
// (interleaved runs on one box; the plain copies also varied more from run to run).
__device__ __forceinline__ void dma16_nt(const void *g, unsigned lds) {
    __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "s"(lds)
                     : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt with only the vector-memory count constrained (expcnt and lgkmcnt at maximum).
template <int N> __device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Returns p unchanged through an empty asm the compiler cannot see into: addresses derived
// from it are then computed where they are used instead of being hoisted out of the layer
// loop and kept live (in registers, or spilled) across every step.  The pointer must be
// wave-uniform (readfirstlane places lane 0's value in scalar registers; a per-lane choice
// between two arrays would silently become lane 0's choice) and point to global memory:
// going through a global-address-space pointer keeps the accesses global, not flat (flat
// accesses also count against the LDS wait counter).
template <typename T> __device__ __forceinline__ T *opaque(T *p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    uint64_t q = ((uint64_t)hi << 32) | lo;
    __asm__ volatile("" : "+s"(q));
    typedef __attribute__((address_space(1))) T GT;
    return (T *)(GT *)q;
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }

// Block-cooperative RMSNorm prologue of a decode projection (one row of K values):
// h = res ? rho(h_in + res) : h_in; ys = rho(w * rho(h * r)), r = 1/sqrt(mean(h^2) + eps),
// stored in LDS in the storage type (values are exactly representable there).  Block 0
// also writes h to h_out when both res and h_out are given.  Ends with a barrier.
template <typename T>
__device__ __forceinline__ void norm_prologue(const T *__restrict__ h_in, const T *__restrict__ res,
                                              const T *__restrict__ w, float eps, T *__restrict__ h_out, int K,
                                              T *ys, float *red) {
    constexpr int VN = Vec<T>::N;
    const int nc = K / VN;
    float ss = 0.f;
    for (int c = threadIdx.x; c < nc; c += blockDim.x) {
        float hv[VN];
        Vec<T>::expand(ld16(h_in + (size_t)c * VN), hv);
        if (res) {
            float rv[VN];
            Vec<T>::expand(ld16(res + (size_t)c * VN), rv);
#pragma unroll
            for (int e = 0; e < VN; ++e) hv[e] = rho<T>(hv[e] + rv[e]);
        }
#pragma unroll
        for (int e = 0; e < VN; ++e) {
            ss += hv[e] * hv[e];
            ys[c * VN + e] = from_f<T>(hv[e]);
            if (res && h_out && blockIdx.x == 0) h_out[c * VN + e] = from_f<T>(hv[e]);
        }
    }
    const float r = 1.0f / sqrtf(block_sum(ss, red) / (float)K + eps);
    for (int c = threadIdx.x; c < nc; c += blockDim.x) {
        float wv[VN];
        Vec<T>::expand(ld16(w + (size_t)c * VN), wv);
#pragma unroll
        for (int e = 0; e < VN; ++e) ys[c * VN + e] = from_f<T>(wv[e] * rho<T>(to_f(ys[c * VN + e]) * r));
    }
    __syncthreads();
}

}  // namespace q3
