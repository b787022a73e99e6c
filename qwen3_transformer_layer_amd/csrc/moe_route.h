// moe_route.h -- the MoE router's softmax, top-k selection and renormalisation for one
// token, as one wave computes them ("@mlx-bun/inference" qwen3-moe.ts,
// Qwen3MoeSparseMoeBlock.forward: softmax over all experts in fp32 with the probabilities
// stored in the model dtype, the k largest with ties to the lower index and slots in
// descending probability, then the renormalising sum and quotient, each in the model dtype).
// Shared by the MoE block kernels and the persistent MoE decode kernel.
#pragma once
#include "common.h"

namespace q3 {

// The k largest of the wave's values (lane l holds experts l + 64 i), ties to the lower
// expert index: each round takes the maximum over the experts not taken yet (DPP) and the
// lowest index holding it (ballots in index order).  A NaN ranks as -inf and experts e >= E
// are never candidates, so every round picks a valid, new expert (k <= E).
template <int EPL>
__device__ __forceinline__ void select_topk(const float (&v)[EPL], int E, int k, int lane, float *psel, int *isel) {
    float x[EPL];
    unsigned taken = 0;  // bit i: expert lane + 64 i is selected or does not exist
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        x[i] = v[i] == v[i] ? v[i] : -INFINITY;
        if (lane + 64 * i >= E) taken |= 1u << i;
    }
    for (int s = 0; s < k; ++s) {
        float lm = -INFINITY;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (!((taken >> i) & 1u)) lm = fmaxf(lm, x[i]);
        const float m = wave_max(lm);
        int bi = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const unsigned long long msk = __ballot(!((taken >> i) & 1u) && x[i] == m);
            if (msk) {
                bi = 64 * i + (int)__builtin_ctzll(msk);
                break;
            }
        }
        psel[s] = m;
        isel[s] = bi;
        if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    }
}

// Softmax in place over the token's E logits v[i] (expert lane + 64 i; -inf past E), in fp32;
// the probabilities are rounded to the model dtype.
template <typename T, int EPL>
__device__ __forceinline__ void softmax_inplace(int E, int lane, float (&v)[EPL]) {
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) m = fmaxf(m, v[i]);
    m = wave_max(m);
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E ? __expf(v[i] - m) : 0.f;
        z += v[i];
    }
    z = wave_sum(z);
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E ? rho<T>(v[i] / z) : -INFINITY;
    }
}

}  // namespace q3
