// attn_core.h -- device building blocks of split-K decode attention, shared by the
// decode kernels in kernels_attn.hip and the persistent decode kernel.
//
// What is computed ("maya2_mlx/backbone.py", forward: attention over keys 0..pos with an
// fp32 softmax; "rlx_flow/blocks/qwen3_decoder.rs", repeat_kv group mapping): one block
// scores a contiguous chunk of keys of one kv head against the G query heads of that head's
// group, scores = fp32(q.k) * D^-1/2, and keeps the chunk's max, sum of exponentials and
// exponential-weighted value sums in fp32 for a later log-sum-exp merge.
#pragma once

#include <math.h>

#include "common.h"

namespace q3 {

// Lane geometry: a key row of D values is LPK lanes x 16 bytes; a wave covers KPW keys per
// step and the block's 4 waves KPB keys.  The first DEC_PF steps of K and V are loaded into
// registers before any other work of the block so HBM latency overlaps the q/k prologue.
constexpr int DEC_PF = 4;

template <typename T, int D, int NWV = 4> struct DecGeo {
    static constexpr int VN = Vec<T>::N, LPK = D / VN, KPW = 64 / LPK, KPB = KPW * NWV;
};

template <typename T, int D, int NWV = 4>
__device__ __forceinline__ void decode_prefetch(const T *__restrict__ Kg, const T *__restrict__ Vg, int j0, int j1,
                                                u32x4 *kp, u32x4 *vp) {
    using G_ = DecGeo<T, D, NWV>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % G_::LPK, kslot = lane / G_::LPK;
#pragma unroll
    for (int i = 0; i < DEC_PF; ++i) {
        const int j = j0 + wave * G_::KPW + i * G_::KPB + kslot;
        const bool ok = j < j1;
        kp[i] = ok ? ld_stream(Kg + (size_t)j * D + sub * G_::VN) : u32x4{0, 0, 0, 0};
        vp[i] = ok ? ld_stream(Vg + (size_t)j * D + sub * G_::VN) : u32x4{0, 0, 0, 0};
    }
}

// Core of one (split, kv head) block: keys [j0, j1) of kv head g against the G query
// heads in qs (LDS, fp32 values of the model-dtype q).  Key `jspec` (if in range) is taken
// from kspec / vspec in LDS instead of the cache (the fused kernel's fresh entry).
// The block's NWV waves split the keys; per-wave partial outputs land in red[NWV][G][D] and
// the per-head max / sum of exponentials in mrow / lrow (all LDS).  decode_core_reduce then
// sums red over the waves.
template <typename T, int D, int G, int NWV = 4>
__device__ __forceinline__ void decode_core_lds(const float *qs, const T *__restrict__ Kg, const T *__restrict__ Vg,
                                                const u32x4 *kp, const u32x4 *vp, int j0, int j1, int jspec,
                                                const float *kspec, const float *vspec, float scale, float *sc,
                                                int chunk, float *red, float *mrow, float *lrow) {
    using G_ = DecGeo<T, D, NWV>;
    constexpr int VN = G_::VN, LPK = G_::LPK, KPW = G_::KPW, KPB = G_::KPB;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane % LPK, kslot = lane / LPK;
    const int nj = j1 - j0;

    float qf[G][VN];
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
        for (int e = 0; e < VN; ++e) qf[i][e] = qs[i * D + sub * VN + e];

    auto score_step = [&](int jb, u32x4 kraw) {
        const int j = jb + kslot;
        const bool valid = j < j1;
        float kf[VN];
        if (j == jspec) {
#pragma unroll
            for (int e = 0; e < VN; ++e) kf[e] = kspec[sub * VN + e];
        } else {
            Vec<T>::expand(kraw, kf);
        }
#pragma unroll
        for (int i = 0; i < G; ++i) {
            float p = 0.f;
#pragma unroll
            for (int e = 0; e < VN; ++e) p += qf[i][e] * kf[e];
#pragma unroll
            for (int o = LPK / 2; o > 0; o >>= 1) p += __shfl_xor(p, o, 64);
            if (sub == 0 && valid) sc[i * chunk + (j - j0)] = p * scale;
        }
    };
#pragma unroll
    for (int i = 0; i < DEC_PF; ++i) {
        const int jb = j0 + wave * KPW + i * KPB;
        if (jb < j1) score_step(jb, kp[i]);
    }
    for (int jb = j0 + wave * KPW + DEC_PF * KPB; jb < j1; jb += KPB) {
        const int j = jb + kslot;
        score_step(jb, j < j1 ? ld_stream(Kg + (size_t)j * D + sub * VN) : u32x4{0, 0, 0, 0});
    }
    __syncthreads();
    for (int i = wave; i < G; i += NWV) {
        float m = -INFINITY;
        for (int j = lane; j < nj; j += 64) m = fmaxf(m, sc[i * chunk + j]);
        m = wave_max(m);
        float l = 0.f;
        for (int j = lane; j < nj; j += 64) {
            const float e = __expf(sc[i * chunk + j] - m);
            sc[i * chunk + j] = e;
            l += e;
        }
        l = wave_sum(l);
        if (lane == 0) {
            mrow[i] = m;
            lrow[i] = l;
        }
    }
    __syncthreads();

    float o[G][VN];
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
        for (int e = 0; e < VN; ++e) o[i][e] = 0.f;
    auto pv_step = [&](int jb, u32x4 vraw) {
        const int j = jb + kslot;
        if (j < j1) {
            float vf[VN];
            if (j == jspec) {
#pragma unroll
                for (int e = 0; e < VN; ++e) vf[e] = vspec[sub * VN + e];
            } else {
                Vec<T>::expand(vraw, vf);
            }
#pragma unroll
            for (int i = 0; i < G; ++i) {
                const float e = sc[i * chunk + (j - j0)];
#pragma unroll
                for (int x = 0; x < VN; ++x) o[i][x] += e * vf[x];
            }
        }
    };
#pragma unroll
    for (int i = 0; i < DEC_PF; ++i) {
        const int jb = j0 + wave * KPW + i * KPB;
        if (jb < j1) pv_step(jb, vp[i]);
    }
    for (int jb = j0 + wave * KPW + DEC_PF * KPB; jb < j1; jb += KPB) {
        const int j = jb + kslot;
        pv_step(jb, j < j1 ? ld_stream(Vg + (size_t)j * D + sub * VN) : u32x4{0, 0, 0, 0});
    }
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
        for (int x = 0; x < VN; ++x) {
            float v = o[i][x];
#pragma unroll
            for (int off = LPK; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
            o[i][x] = v;
        }
    if (kslot == 0) {
#pragma unroll
        for (int i = 0; i < G; ++i)
#pragma unroll
            for (int x = 0; x < VN; ++x) red[(wave * G + i) * D + sub * VN + x] = o[i][x];
    }
    __syncthreads();
}

// Sum of the waves' partial outputs for head i, dimension d.
template <int D, int G, int NWV>
__device__ __forceinline__ float decode_core_reduce(const float *red, int i, int d) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) v += red[(w * G + i) * D + d];
    return v;
}

}  // namespace q3
