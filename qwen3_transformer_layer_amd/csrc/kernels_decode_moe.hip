// kernels_decode_moe.hip -- the whole T = 1 decode step of a Qwen3-MoE stack as one
// persistent kernel.
//
// What is computed: the attention half of the layer of "maya2_mlx/backbone.py"
// (Backbone.forward and its docstring's rounding points) and the sparse MoE block of
// "@mlx-bun/inference" qwen3-moe.ts (Qwen3MoeSparseMoeBlock.forward: router logits, softmax
// over all experts stored in the model dtype, the top k with ties to the lower index and
// slots in descending probability, the renormalised weights, each chosen expert's SwiGLU
// MLP, each weighted expert output rounded, and the slot sum rounded once), for one token at
// position p through every layer, then the final norm.  The kernels of kernels_linear.hip,
// kernels_attn.hip and kernels_moe.hip compute the same values one step at a time.
//
// Shape: hidden 2048, head_dim 128, 8 query heads per kv head, n_heads * head_dim = 4096
// (the attention output, o_proj's input), E <= 128 experts, top 8, expert intermediate 768.
// Block roles (8 compute waves, 4 stream waves), the LDS ring of 4 KB chunks and the exchange
// protocol between blocks are those of kernels_decode_mk.hip.  What differs:
//  - Attention: a block holds the 8 query heads of its kv head for one split of the keys;
//    compute wave h takes head h (its scores over every K chunk of the split, its softmax
//    and its p.V over every V chunk), so no cross-wave reduction is needed.  Every K and V
//    chunk is read by all 8 waves; the ring's release count is therefore kept in eighths:
//    a chunk with one consumer adds 8 to its slot's count, a shared chunk 1 per wave.
//  - o_proj rows have 4096 inputs, two chunks each.
//  - Router: block b < E computes router row b and publishes the logit; every block polls
//    the E logits and its wave 0 repeats the softmax, top-k and renormalisation (the same
//    code in every block, so all agree), puts the k experts and weights in LDS and raises a
//    flag that the stream waves wait on before they copy the layer's first expert row.
//  - The k chosen experts form one virtual SwiGLU of k * 768 = 6144 outputs: output i is
//    row i mod 768 of the expert in slot i / 768, so block b's 24 outputs (gate and up row of
//    each, as in the dense kernel) belong to the expert in slot b / 32.
//  - Down: row n of the virtual down projection is the concatenation over the slots of row n
//    of each slot's expert (6144 inputs, three chunks); the stream waves gather each lane's 16
//    bytes from the expert of the slot they fall in.  A lane adds each 8-input piece to its
//    slot's sum, the wave reduces the k sums, and the output is rho(sum_s rho(rho(y_s) w_s))
//    with the sum in slot order.
// 8-bit weights (router and experts included; u8 codes, bf16 scale and bias per 64 inputs) as in
// the dense kernel: a ring chunk holds the codes of two q|k|v rows, one o_proj row (4096 codes),
// one router row, the gate and the up row of one SwiGLU output, or one third of a virtual down
// row, and a 256-byte side slot their groups' scales and biases; every chunk is five copies.
#include "common.h"
#include "decode_mk_common.h"
#include "kernels.h"
#include "moe_route.h"

namespace q3 {
namespace mkm {

using namespace mk;

constexpr int G = 8;            // query heads per kv head
constexpr int HD = 4096;        // n_heads * head_dim
constexpr int NQKV = 5120;      // q|k|v rows: (32 + 2 * 4) * 128
constexpr int QPB = NQKV / NB;  // q|k|v rows per block (20)
constexpr int OPB = HID / NB;   // o_proj rows = down rows per block (8)
constexpr int KSEL = 8;         // experts per token
constexpr int IE = 768;         // expert intermediate size
constexpr int IM = KSEL * IE;   // outputs of the virtual SwiGLU (6144)
constexpr int GPB = IM / NB;    // SwiGLU outputs per block (24)
constexpr int DCH = IM * 2 / CHB;  // chunks per virtual down row (3)
constexpr int EMAX = 128;       // experts (two per lane in the routing wave)
constexpr int CHM = 128;        // keys per attention split
constexpr int NSM = 29;         // ring slots (116 KB)
constexpr int NSMQ = 27;        // ring slots with 8-bit weights (108 KB + 6.75 KB of scale/bias slots)
constexpr int SBM = 256;        // scale/bias bytes per chunk (8-bit weights)
static_assert(NQKV % NB == 0 && IE % GPB == 0 && GPB == 3 * NC && IM * 2 == DCH * CHB && OPB == NC, "shape");
static_assert(NSMQ >= NL * DL, "the ring holds every stream wave's chunks in flight");
template <bool Q8> __host__ __device__ constexpr int ring_slots() { return Q8 ? NSMQ : NSM; }

struct DevLayer {  // q_norm / k_norm both null: no per-head q/k norm; qkv_bias null: no bias
    const bf16 *in_norm, *post_norm, *q_norm, *k_norm, *qkv, *o, *router, *exp_gu, *exp_down, *qkv_bias;
};

struct DevLayerQ {  // 8-bit weights: (scale, bias) array pairs [rows][K / 64] of q|k|v, o, router, experts
    const bf16 *qkv_s, *qkv_b, *o_s, *o_b, *router_s, *router_b, *egu_s, *egu_b, *edown_s, *edown_b;
};
static_assert(sizeof(DevLayerQ) == 80, "five (scale, bias) pairs of 16 bytes, read as pairs");

struct Args {
    const DevLayer *layers;
    const DevLayerQ *layersq;  // 8-bit weights only
    int n_layers, H, KV, E, cap, p, nsplit, chunk, window, norm_topk;  // window 0: causal
    float eps, scale;
    const bf16 *x, *final_norm, *cos_t, *sin_t;
    bf16 *out, *kc, *vc;
    uint32_t *x_qkv, *x_a, *x_h2, *x_r, *x_m, *x_pend;
    uint64_t *x_part;
    unsigned *ctr;
    int *err;
};

// Per layer the block consumes, in this order: its QPB q|k|v rows, nK K chunks and nK V chunks of
// its attention split, its OPB o_proj rows, its router row (blocks b < E), its GPB gate/up row
// pairs, OPB virtual down rows of DCH chunks each.  Chunks: bf16 -- one q|k|v row, half an o_proj
// row, one router row, a gate or an up row, a third of a down row; 8-bit -- two q|k|v rows, one
// o_proj row, one router row, a gate/up pair, a third of a down row.
template <bool Q8> struct Seq {
    static constexpr int QC = Q8 ? QPB / 2 : QPB, OC = Q8 ? OPB : 2 * OPB, GC = Q8 ? GPB : 2 * GPB, DC = OPB * DCH;
    int nK, rc, cpl;
    __device__ Seq(int nK_, int rc_) : nK(nK_), rc(rc_), cpl(QC + 2 * nK_ + OC + rc_ + GC + DC) {}
    __device__ int oK() const { return QC; }
    __device__ int oV() const { return QC + nK; }
    __device__ int oO() const { return QC + 2 * nK; }
    __device__ int oR() const { return QC + 2 * nK + OC; }
    __device__ int oG() const { return QC + 2 * nK + OC + rc; }
    __device__ int oD() const { return QC + 2 * nK + OC + rc + GC; }
};

// Release weights of a chunk: the stream wave refills slot s for chunk g once done[s] reaches
// 8 (g / NSM), each earlier chunk of the slot having added 8 in all.
constexpr unsigned REL = 8;
template <int NSL> __device__ __forceinline__ void chunk_put_w(unsigned *done, unsigned g, int lane, unsigned w) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (lane == 0) __hip_atomic_fetch_add(done + g % NSL, w, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// The (scale, bias) array pointers of field pair `pair` (0 q|k|v, 1 o, 2 router, 3 expert gate|up,
// 4 expert down) of a layer's 8-bit entry, read with one scalar load completed inside the asm (a
// vector load would sit in the stream wave's counter beside the ring copies).
__device__ __forceinline__ void load_sb_pair(const DevLayerQ *e, int pair, const bf16 *&sc, const bf16 *&bi) {
    const uint64_t a = (uint64_t)e + 16u * (unsigned)pair;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a), hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    u32x4 v;
    __asm__ volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(((uint64_t)hi << 32) | lo) : "memory");
    typedef __attribute__((address_space(1))) const bf16 GB;
    sc = (const bf16 *)(GB *)(((uint64_t)v[1] << 32) | v[0]);
    bi = (const bf16 *)(GB *)(((uint64_t)v[3] << 32) | v[2]);
}

// 8-bit: one 16-code piece against 16 activations, s (x . q) + b (sum x), for the down thirds.
__device__ __forceinline__ float q8_piece(const unsigned char *c, int piece, float s, float b, u32x4 xa, u32x4 xb,
                                          float xs, int lane) {
    const u32x4 cw = *(const u32x4 *)(c + piece * 1024 + lane * 16);
    return s * dot16_codes(cw, xa, xb, 0.f) + b * xs;
}

// A lane's four 8-input partial dots of a chunk (the X4 interleave: piece k covers inputs
// (lane + 64 k) * 8 .. + 7), not summed.
__device__ __forceinline__ void dot_pieces(const unsigned char *c, const X4 &x, int lane, float (&pk)[4]) {
    u32x4 w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = *(const u32x4 *)(c + k * 1024 + lane * 16);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float a = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t wq = w[k][q], xq = x.v[k][q];
            a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wq), __builtin_bit_cast(bf16x2, xq), a, false);
        }
        pk[k] = a;
    }
}

// Stream wave j: chunks g = j, j + NL, ... of the whole step, in order.  Expert rows wait for
// the layer's routing (rgen, route_e in LDS).
template <bool Q8>
__device__ void stream_wave(const Args &A, const DevLayer *lay, unsigned char *ring, unsigned char *sbring,
                            unsigned *ready, const unsigned *done, const unsigned *rgen, const int (*route_e)[KSEL],
                            unsigned *abt, int j, int ag, int j0, int j1, int nK) {
    constexpr int NSM = ring_slots<Q8>(), VPC = Q8 ? 5 : 4;  // slots; copies per chunk
    const int lane = tid_now() & 63, b = blockIdx.x;
    const Seq<Q8> S(nK, b < A.E ? 1 : 0);
    const unsigned total = (unsigned)A.n_layers * (unsigned)S.cpl;
    auto publish = [&](unsigned g) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (lane == 0) __hip_atomic_store(ready + g % NSM, g / NSM + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };
    wait_vm<0>();  // clears the compiler's wait bookkeeping (see the dense kernel's stream wave)
    unsigned n = 0, pub = 0;
    int routed = 0;  // layers whose routing this wave has seen
    for (unsigned g = j; g < total; g += NL) {
        const int l = (int)(g / (unsigned)S.cpl), idx = (int)(g - (unsigned)l * (unsigned)S.cpl);
        const DevLayer &L = lay[l];
        if (idx >= S.oG() && routed <= l) {
            // expert rows: land and publish everything in flight (the router row among it may be
            // what the routing waits for), then wait for the layer's routing
            wait_vm<0>();
            for (; pub < n; ++pub) publish(j + NL * pub);
            lds_wait_ge(rgen, (unsigned)l + 1u, abt, nullptr);
            routed = l + 1;
        }
        const unsigned char *src[4];
        const void *sbsrc = nullptr;  // 8-bit: the lane's 4 bytes of the chunk's scale/bias copy
        if (Q8 && (idx < S.oK() || idx >= S.oO())) {
            // codes: pieces 0, 1 from row r0 (at w0), pieces 2, 3 from row r1 (at w1); scale/bias copy:
            // lanes 0-15 s[r0], 16-31 b[r0], 32-47 s[r1], 48-63 b[r1], two groups per lane from group
            // g0 of r0 and g1 of r1 (ng groups per row)
            const bf16 *sc, *bi;
            const unsigned char *w0, *w1;
            size_t r0, r1;
            int ng = HID / 64, g0 = 0, g1 = 0;
            if (idx < S.oK()) {
                load_sb_pair(A.layersq + l, 0, sc, bi);
                r0 = (size_t)b * QPB + 2 * idx, r1 = r0 + 1;
                w0 = (const unsigned char *)opaque(L.qkv) + r0 * HID, w1 = w0 + HID;
            } else if (idx < S.oR()) {  // o_proj row r (4096 codes): its halves as r0 and r1
                load_sb_pair(A.layersq + l, 1, sc, bi);
                r0 = r1 = (size_t)b * OPB + (idx - S.oO());
                w0 = (const unsigned char *)opaque(L.o) + r0 * HD, w1 = w0 + HID;
                ng = HD / 64, g1 = HID / 64;
            } else if (idx < S.oG()) {  // router row b (pieces 2, 3 repeat 0, 1)
                load_sb_pair(A.layersq + l, 2, sc, bi);
                r0 = r1 = (size_t)b;
                w0 = w1 = (const unsigned char *)opaque(L.router) + r0 * HID;
            } else if (idx < S.oD()) {  // gate row and up row of output b * GPB + i
                load_sb_pair(A.layersq + l, 3, sc, bi);
                const int o = b * GPB + (idx - S.oG());
                const int e = min(max(route_e[l & 1][o / IE], 0), A.E - 1);
                r0 = (size_t)e * (2 * IE) + o % IE, r1 = r0 + IE;
                w0 = (const unsigned char *)opaque(L.exp_gu) + r0 * HID, w1 = (const unsigned char *)opaque(L.exp_gu) + r1 * HID;
            } else {
                load_sb_pair(A.layersq + l, 4, sc, bi);
                r0 = r1 = 0;
                w0 = w1 = nullptr;
            }
            if (idx < S.oD()) {
                src[0] = w0 + lane * 16;
                src[1] = w0 + 1024 + lane * 16;
                src[2] = w1 + lane * 16;
                src[3] = w1 + 1024 + lane * 16;
                if (idx >= S.oR() && idx < S.oG()) {  // router: one row
                    src[2] = src[0];
                    src[3] = src[1];
                }
                const int q = lane >> 4;
                const bf16 *arr = (q & 1) ? bi : sc;  // a per-lane choice between two uniform arrays
                sbsrc = (const void *)(arr + (q < 2 ? r0 * ng + g0 : r1 * ng + g1) + 2 * (lane & 15));
            } else {  // third t of virtual down row n: codes 2048 t + 1024 k + 16 lane (k = 0, 1), gathered
                const int i = idx - S.oD(), n_ = b * OPB + i / DCH, t = i % DCH;
                const unsigned char *W = (const unsigned char *)opaque(L.exp_down);
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const int v = 2048 * t + 1024 * k + 16 * lane, s = v / IE, o = v - s * IE;
                    const int e = min(max(route_e[l & 1][s], 0), A.E - 1);
                    src[k] = W + ((size_t)e * HID + n_) * IE + o;
                }
                src[2] = src[0];
                src[3] = src[1];
                // the third's 32 groups: lanes 0-15 two scales each, 16-31 two biases; 32-63 repeat
                const int gi = 2 * (lane & 15), vg = 2048 * t + 64 * gi, s = vg / IE;
                const int e = min(max(route_e[l & 1][s], 0), A.E - 1);
                const bf16 *arr = ((lane >> 4) & 1) ? bi : sc;
                sbsrc = (const void *)(arr + ((size_t)e * HID + n_) * (IE / 64) + (vg - s * IE) / 64);
            }
        } else if (idx < S.oK()) {
            const unsigned char *base = (const unsigned char *)opaque(L.qkv) + ((size_t)b * QPB + idx) * CHB;
#pragma unroll
            for (int k = 0; k < 4; ++k) src[k] = base + k * 1024 + lane * 16;
        } else if (idx < S.oO()) {
            const bool isV = idx >= S.oV();
            const int i = idx - (isV ? S.oV() : S.oK());
            const bf16 *cache = (isV ? opaque(A.vc) : opaque(A.kc)) + ((size_t)l * A.KV + ag) * A.cap * D;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                // keys past the split's end (a partial last chunk) re-read its last key
                const int key = min(j0 + i * KPC + 4 * k + lane / 16, j1 - 1);
                src[k] = (const unsigned char *)(cache + (size_t)key * D) + (lane % 16) * 16;
            }
            sbsrc = src[0];  // 8-bit: a fifth copy into the unused side slot keeps five per chunk
        } else if (idx < S.oR()) {  // half h of o_proj row r
            const int i = idx - S.oO();
            const unsigned char *base =
                (const unsigned char *)opaque(L.o) + ((size_t)b * OPB + (i >> 1)) * (HD * 2) + (size_t)(i & 1) * CHB;
#pragma unroll
            for (int k = 0; k < 4; ++k) src[k] = base + k * 1024 + lane * 16;
        } else if (idx < S.oG()) {  // router row b
            const unsigned char *base = (const unsigned char *)opaque(L.router) + (size_t)b * CHB;
#pragma unroll
            for (int k = 0; k < 4; ++k) src[k] = base + k * 1024 + lane * 16;
        } else if (idx < S.oD()) {  // gate (even) or up (odd) row of output b * GPB + i / 2
            const int i = idx - S.oG(), o = b * GPB + (i >> 1);
            const int e = min(max(route_e[l & 1][o / IE], 0), A.E - 1);
            const size_t row = (size_t)e * (2 * IE) + ((i & 1) ? IE : 0) + o % IE;
            const unsigned char *base = (const unsigned char *)opaque(L.exp_gu) + row * CHB;
#pragma unroll
            for (int k = 0; k < 4; ++k) src[k] = base + k * 1024 + lane * 16;
        } else {  // chunk q of virtual down row n: inputs 2048 q .. + 2047
            const int i = idx - S.oD(), n_ = b * OPB + i / DCH, q = i % DCH;
            const unsigned char *W = (const unsigned char *)opaque(L.exp_down);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int v = 2048 * q + 512 * k + 8 * lane, s = v / IE, o = v - s * IE;
                const int e = min(max(route_e[l & 1][s], 0), A.E - 1);
                src[k] = W + (((size_t)e * HID + n_) * IE + o) * 2;
            }
        }
        const unsigned s = g % NSM, gen = g / NSM;
        if (lds_acquire(done + s) < REL * gen) {
            wait_vm<0>();
            for (; pub < n; ++pub) publish(j + NL * pub);
            lds_wait_ge(done + s, REL * gen, abt, nullptr);
        }
        const unsigned dlds = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(ring + (size_t)s * CHB));
#pragma unroll
        for (int k = 0; k < 4; ++k) dma16_nt(src[k], dlds + k * 1024);
        if constexpr (Q8) dma4(sbsrc, __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(sbring + (size_t)s * SBM)));
        ++n;
        if (n - pub >= DL) {
            wait_vm<VPC * (DL - 1)>();  // all but this wave's last DL-1 chunks have landed
            for (; pub + (DL - 1) < n; ++pub) publish(j + NL * pub);
        }
    }
    wait_vm<0>();
    for (; pub < n; ++pub) publish(j + NL * pub);
}

template <bool Q8>
__global__ void __launch_bounds__(NTH) decode_moe_kernel(Args A) {
    constexpr int NSM = ring_slots<Q8>();
    constexpr int HPT = HID / NCT;  // words per compute thread of a hidden vector
    constexpr int APT = HD / NCT;   // of the attention output
    constexpr int RSH = rep_stride(HID), RSA = rep_stride(HD), RSM = rep_stride(IM), RSR = rep_stride(EMAX);
    __shared__ __attribute__((aligned(16))) unsigned char ring[NSM * CHB];
    __shared__ __attribute__((aligned(16))) unsigned char sbring[Q8 ? NSM * SBM : 16];  // 8-bit: scales and biases
    __shared__ unsigned ready[NSM], done[NSM], bar, abt, rgen;
    __shared__ DevLayer lay[MAXL];
    __shared__ float hs[HID];                                 // residual stream h (fp32 of bf16 values)
    __shared__ __attribute__((aligned(16))) uint16_t ys[IM];  // current projection input (bf16 bits)
    __shared__ __attribute__((aligned(16))) uint16_t qraw[G * D + 2 * D];
    __shared__ float qs[G * D], kvs[2 * D];
    __shared__ float sc[G * CHM];
    __shared__ float rsum[2][NC];
    __shared__ float po[64 * (HD / NB)];  // split merge: [ns][dims per block]
    __shared__ float pm[64], pl[64];
    __shared__ int route_e[2][KSEL];
    __shared__ float route_w[2][KSEL];

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), b = blockIdx.x;
    const int H = A.H, KV = A.KV;
    const int p = A.p, nkeys = p + 1;
    const int bpg = NB / KV;               // attention blocks per kv head (= splits)
    const int ag = b / bpg, as = b % bpg;  // this block's (kv head, split)
    const int lo = A.window > 0 ? max(0, nkeys - A.window) : 0;  // first visible key (sliding window)
    const int j0 = lo + as * A.chunk, j1 = min(nkeys, j0 + A.chunk);
    const int nK = j0 < j1 ? (j1 - j0 + KPC - 1) / KPC : 0;
    const bool has_p = j0 < nkeys && j1 == nkeys;
    const Seq<Q8> S(nK, b < A.E ? 1 : 0);

    for (int i = tid; i < NSM; i += NTH) {
        ready[i] = 0;
        done[i] = 0;
    }
    if (tid == 0) {
        bar = 0;
        abt = 0;
        rgen = 0;
    }
    if (tid < 2 * KSEL) route_e[tid / KSEL][tid % KSEL] = 0;  // a valid expert even if a wait gives up
    for (int i = tid; i < A.n_layers; i += NTH) lay[i] = A.layers[i];
    const unsigned tag0 = A.ctr[0] * 64u;
    __syncthreads();  // the only barrier of the whole block; the roles split here

    if (wave >= NC) {
        stream_wave<Q8>(A, lay, ring, sbring, ready, done, &rgen, route_e, &abt, wave - NC, ag, j0, j1, nK);
        return;
    }

    // ================================================================ compute waves
    unsigned ep = 0, par = 0;
    const int ns = A.nsplit;
    constexpr int dpb = HD / NB;  // merged attention outputs per block (16)
    const int mh = b / (NB / H), md0 = (b % (NB / H)) * dpb;
    constexpr int half = D / 2;
    const int jspec = has_p ? p : -1;  // the new key, taken from LDS
    const int lane0 = tid & 63;
    for (int k = 0; k < HPT; ++k) hs[tid + NCT * k] = to_f(opaque(A.x)[tid + NCT * k]);
    float w_in[HPT], w_post[HPT], w_qn[2], w_kn[2];
    const float c1 = to_f(opaque(A.cos_t)[(size_t)p * D + lane0]), s1 = to_f(opaque(A.sin_t)[(size_t)p * D + lane0]);
    const float c2 = to_f(opaque(A.cos_t)[(size_t)p * D + lane0 + half]);
    const float s2 = to_f(opaque(A.sin_t)[(size_t)p * D + lane0 + half]);
    auto load_small = [&](int l) {
        const DevLayer &L = lay[l];
        const int tid = tid_now(), lane = tid & 63;
#pragma unroll
        for (int k = 0; k < HPT; ++k) {
            w_in[k] = to_f(opaque(L.in_norm)[tid + NCT * k]);
            w_post[k] = to_f(opaque(L.post_norm)[tid + NCT * k]);
        }
        if (L.q_norm) {
            w_qn[0] = to_f(opaque(L.q_norm)[lane]);
            w_qn[1] = to_f(opaque(L.q_norm)[lane + half]);
            w_kn[0] = to_f(opaque(L.k_norm)[lane]);
            w_kn[1] = to_f(opaque(L.k_norm)[lane + half]);
        }
    };
    load_small(0);

    for (int l = 0; l < A.n_layers; ++l) {
        const int tid = tid_now(), lane = tid & 63;
        const int sub = lane % 16, kslot = lane / 16;  // K/V pieces: 16 lanes per 128-dim key row
        const unsigned tag = (tag0 + (unsigned)l) & 0xffffu;
        const unsigned ptag = (tag0 + (unsigned)l - 1u) & 0xffffu;
        const unsigned gb = (unsigned)l * (unsigned)S.cpl;
        bf16 *Kg = opaque(A.kc) + ((size_t)l * KV + ag) * A.cap * D;
        bf16 *Vg = opaque(A.vc) + ((size_t)l * KV + ag) * A.cap * D;

        // ---------------- step 1: h = rho(h + pend); y = RMSNorm(h); q|k|v rows
        cbar(&bar, ep, &abt, opaque(A.err), lane);  // every wave is done reading ys (the previous layer's m)
        if (l > 0) {
            poll_pause<PAUSE_VEC>();
            poll_bf16<HPT>(opaque(A.x_pend) + (b % NREP) * RSH, HID, ptag, ys, opaque(A.err), &abt, tid);
#pragma unroll
            for (int k = 0; k < HPT; ++k) {  // a thread's own elements only: no barrier needed
                const int i = tid + NCT * k;
                hs[i] = rho<bf16>(hs[i] + bfv(ys[i]));
            }
        }
        {
            float ss = 0.f;
#pragma unroll
            for (int k = 0; k < HPT; ++k) ss += hs[tid + NCT * k] * hs[tid + NCT * k];
            const float r = 1.0f / sqrtf(csum(ss, rsum, par, &bar, ep, &abt, opaque(A.err), tid) / (float)HID + A.eps);
#pragma unroll
            for (int k = 0; k < HPT; ++k) {
                const int i = tid + NCT * k;
                ys[i] = (uint16_t)f2bf_bits(w_in[k] * rho<bf16>(hs[i] * r));
            }
        }
        cbar(&bar, ep, &abt, opaque(A.err), lane);
        if constexpr (Q8) {
            const bf16 *qb = lay[l].qkv_bias;
            const X8 xq = load_x8(ys, lane);
            for (int i = wave; i < S.QC; i += NC) {  // chunk i: rows 2 i and 2 i + 1 of the block's QPB
                const unsigned g = gb + i;
                const unsigned char *c = chunk_get<NSM>(ring, ready, g, &abt, opaque(A.err));
                const uint16_t *sb = (const uint16_t *)(sbring + (size_t)(g % NSM) * SBM);
                float a0 = wave_sum(dot_q8_row(c, 0, 1, sb, xq, lane));
                float a1 = wave_sum(dot_q8_row(c, 2, 3, sb + 64, xq, lane));
                chunk_put_w<NSM>(done, g, lane, REL);
                const int r0 = b * QPB + 2 * i;
                if (qb) {
                    a0 = rho<bf16>(a0) + to_f(opaque(qb)[r0]);
                    a1 = rho<bf16>(a1) + to_f(opaque(qb)[r0 + 1]);
                }
                if (lane == 0) xstore(opaque(A.x_qkv) + r0, tagw(tag, a0));
                if (lane == 1) xstore(opaque(A.x_qkv) + r0 + 1, tagw(tag, a1));
            }
        } else {
            // a q|k|v bias is its own rounded add after the projection: rho(rho(x W^T) + b)
            const bf16 *qb = lay[l].qkv_bias;
            const X4 xq = load_x(ys, lane);
            for (int i = wave; i < QPB; i += NC) {
                const unsigned g = gb + i;
                const unsigned char *c = chunk_get<NSM>(ring, ready, g, &abt, opaque(A.err));
                float acc = wave_sum(dot_chunk(c, xq, lane, 0.f));
                chunk_put_w<NSM>(done, g, lane, REL);
                if (qb) acc = rho<bf16>(acc) + to_f(opaque(qb)[(size_t)b * QPB + i]);
                if (lane == 0) xstore(opaque(A.x_qkv) + (size_t)b * QPB + i, tagw(tag, acc));
            }
        }

        poll_pause<PAUSE_VEC>();
        // ---------------- step 2: per-head q/k norm + RoPE + cache write, split-K attention
        if (nK > 0) {
            // the group's q heads, and for the block holding the new key its k and v heads:
            // word t < G*D is q word t; then the k words; then the v words
            constexpr int NPW = (G * D + 2 * D + NCT - 1) / NCT;
            const int nw = G * D + (has_p ? 2 * D : 0);
            uint32_t v[NPW];
            const uint32_t *w[NPW];
#pragma unroll
            for (int k = 0; k < NPW; ++k) {
                const int t = tid + NCT * k;
                const int src = t < G * D ? ag * G * D + t
                                          : (t < G * D + D ? (H + ag) * D + t - G * D : (H + KV + ag) * D + t - G * D - D);
                w[k] = opaque(A.x_qkv) + (t < nw ? src : 0);
                v[k] = t < nw ? xload(w[k]) : (tag << 16);
            }
            long sp = 0;
            while (true) {
                bool ok = true;
#pragma unroll
                for (int k = 0; k < NPW; ++k) ok &= (v[k] >> 16) == tag;
                if (ok || spin_out(++sp, opaque(A.err), &abt)) break;
#pragma unroll
                for (int k = 0; k < NPW; ++k)
                    if ((v[k] >> 16) != tag) v[k] = xload(w[k]);
            }
#pragma unroll
            for (int k = 0; k < NPW; ++k) {
                const int t = tid + NCT * k;
                if (t < nw) qraw[t] = (uint16_t)(v[k] & 0xffffu);
            }
        }
        cbar(&bar, ep, &abt, opaque(A.err), lane);
        if (nK > 0) {
            for (int hh = wave; hh < G + (has_p ? 1 : 0); hh += NC) {
                const bool is_q = hh < G;
                const uint16_t *row = qraw + hh * D;
                const float x1 = bfv(row[lane]), x2 = bfv(row[lane + half]);
                float n1 = x1, n2 = x2;  // without the per-head norm RoPE takes the projection as it is
                if (lay[l].q_norm) {
                    const float r = 1.0f / sqrtf(wave_sum(x1 * x1 + x2 * x2) / (float)D + A.eps);
                    const float wn1 = is_q ? w_qn[0] : w_kn[0], wn2 = is_q ? w_qn[1] : w_kn[1];
                    n1 = rho<bf16>(wn1 * rho<bf16>(x1 * r));
                    n2 = rho<bf16>(wn2 * rho<bf16>(x2 * r));
                }
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
        cbar(&bar, ep, &abt, opaque(A.err), lane);
        if (nK > 0) {
            // wave h: head h.  Scores: K chunk i holds keys j0 + KPC*i ..; the lane's piece k is key
            // 4k + kslot, dims sub*8 .. sub*8+7 (q and the new key are bf16 values, so packing
            // them is exact; each piece is four v_dot2c_f32_bf16)
            const int h = wave;
            const float *qh = qs + h * D + sub * 8;
            const u32x4 qp = {pack_bf2(qh[0], qh[1]), pack_bf2(qh[2], qh[3]), pack_bf2(qh[4], qh[5]),
                              pack_bf2(qh[6], qh[7])};
            const float *kn = kvs + sub * 8;
            const u32x4 knew = {pack_bf2(kn[0], kn[1]), pack_bf2(kn[2], kn[3]), pack_bf2(kn[4], kn[5]),
                                pack_bf2(kn[6], kn[7])};
            // per chunk i: the scores of its KPC keys, their exponentials against the wave's running
            // maximum (earlier chunks rescaled), then p . V with V chunk i; the probabilities go
            // through the wave's own row of sc.  In p . V lane l owns dims 2l, 2l+1 of every key.
            float m = -INFINITY, ls = 0.f, o0 = 0.f, o1 = 0.f;
            const float vs0 = kvs[D + 2 * lane], vs1 = kvs[D + 2 * lane + 1];
            for (int i = 0; i < nK; ++i) {
                const unsigned gk = gb + S.oK() + i;
                const unsigned char *c = chunk_get<NSM>(ring, ready, gk, &abt, opaque(A.err));
                u32x4 kr[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) kr[k] = *(const u32x4 *)(c + k * 1024 + lane * 16);
                float sv[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int j = j0 + i * KPC + 4 * k + kslot;
                    const u32x4 kw = j == jspec ? knew : kr[k];
                    const float sdot = row16_sum(dot16<bf16>(qp, kw, 0.f));  // the key's 16 lanes form one DPP row
                    sv[k] = j < j1 ? sdot * A.scale : -INFINITY;
                }
                chunk_put_w<NSM>(done, gk, lane, 1u);  // one of the chunk's G readers
                const int jb = j0 + i * KPC;
                float cm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
                cm = fmaxf(fmaxf(lane_f(cm, 0), lane_f(cm, 16)), fmaxf(lane_f(cm, 32), lane_f(cm, 48)));
                const float mn = fmaxf(m, cm);  // finite: key jb is below j1
                const float alpha = __expf(m - mn);
                float ps = 0.f;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float e = __expf(sv[k] - mn);
                    ps += e;
                    if (sub == 0) sc[h * CHM + (jb + 4 * k + kslot - j0)] = e;
                }
                ps = (lane_f(ps, 0) + lane_f(ps, 16)) + (lane_f(ps, 32) + lane_f(ps, 48));
                ls = ls * alpha + ps;
                o0 *= alpha;
                o1 *= alpha;
                m = mn;
                const unsigned gv = gb + S.oV() + i;
                c = chunk_get<NSM>(ring, ready, gv, &abt, opaque(A.err));
                uint32_t vw[KPC];
                float pe[KPC];
#pragma unroll
                for (int kk = 0; kk < KPC; ++kk) vw[kk] = *(const uint32_t *)(c + kk * (D * 2) + lane * 4);
#pragma unroll
                for (int kk = 0; kk < KPC; ++kk) pe[kk] = sc[h * CHM + (jb + kk - j0)];
#pragma unroll
                for (int kk = 0; kk < KPC; ++kk) {
                    float v0 = bf_lo(vw[kk]), v1 = bf_hi(vw[kk]);
                    if (jb + kk == jspec) {
                        v0 = vs0;
                        v1 = vs1;
                    }
                    o0 += pe[kk] * v0;
                    o1 += pe[kk] * v1;
                }
                chunk_put_w<NSM>(done, gv, lane, 1u);  // one of the chunk's G readers
            }
            uint64_t *pp = opaque(A.x_part) + ((size_t)(ag * G + h) * ns + as) * (D + 2);
            xstore64(pp + 2 + 2 * lane, ((uint64_t)tag << 32) | __float_as_uint(o0));
            xstore64(pp + 3 + 2 * lane, ((uint64_t)tag << 32) | __float_as_uint(o1));
            if (lane == 0) {
                xstore64(pp, ((uint64_t)tag << 32) | __float_as_uint(m));
                xstore64(pp + 1, ((uint64_t)tag << 32) | __float_as_uint(ls));
            }
        } else {  // an empty split (fewer keys than splits): max -inf, sum 0
            for (int idx = tid; idx < G * (D + 2); idx += NCT) {
                const int i = idx / (D + 2), e = idx % (D + 2);
                const float v = e == 0 ? -INFINITY : 0.f;
                xstore64(opaque(A.x_part) + ((size_t)(ag * G + i) * ns + as) * (D + 2) + e,
                         ((uint64_t)tag << 32) | __float_as_uint(v));
            }
        }

        // ---------------- step 3: merge the splits of (head mh, dims md0 .. md0 + dpb)
        // Barriers before this poll and the merged-output poll keep the block's early waves from
        // polling while the others still work (MoE step ~1804 -> ~1752 us, 8-bit ~1856 -> ~1803 us).
        cbar(&bar, ep, &abt, opaque(A.err), lane);
        poll_pause<PAUSE_SPLIT>();
        {
            // the split maxima, sums and this block's dims of every split's output, each word polled
            // by one thread, all of a thread's words in flight together
            constexpr int NPM = (64 * (2 + dpb) + NCT - 1) / NCT;
            const int nwords = ns * (2 + dpb);
            uint64_t v[NPM];
            const uint64_t *src[NPM];
#pragma unroll
            for (int k = 0; k < NPM; ++k) {
                const int t = tid + NCT * k, u = t - 2 * ns;
                src[k] = opaque(A.x_part) + (t >= nwords ? 0
                                             : t < 2 * ns ? ((size_t)mh * ns + t / 2) * (D + 2) + (t % 2)
                                                          : ((size_t)mh * ns + u / dpb) * (D + 2) + 2 + md0 + u % dpb);
                v[k] = t < nwords ? xload64(src[k]) : ((uint64_t)tag << 32);
            }
            long sp = 0;
            while (true) {
                bool ok = true;
#pragma unroll
                for (int k = 0; k < NPM; ++k) ok &= (unsigned)(v[k] >> 32) == tag;
                if (ok || spin_out(++sp, opaque(A.err), &abt)) break;
#pragma unroll
                for (int k = 0; k < NPM; ++k)
                    if ((unsigned)(v[k] >> 32) != tag) v[k] = xload64(src[k]);
            }
#pragma unroll
            for (int k = 0; k < NPM; ++k) {
                const int t = tid + NCT * k;
                const float f = __uint_as_float((uint32_t)v[k]);
                if (t < 2 * ns) {
                    if (t % 2 == 0) pm[t / 2] = f;
                    else pl[t / 2] = f;
                } else if (t < nwords) {
                    po[t - 2 * ns] = f;
                }
            }
            cbar(&bar, ep, &abt, opaque(A.err), lane);
            float av;
            if (merge_lds<8>(pm, pl, po, ns, dpb, tid, &av)) {  // waves 0-1: 8 lanes per dim
                const uint32_t w = tagw(tag, av);
#pragma unroll
                for (int r = 0; r < NREP; ++r) xstore(opaque(A.x_a) + r * RSA + mh * D + md0 + tid / 8, w);
            }
        }

        // ---------------- step 4: h = rho(h + rho(a . Wo^T)) for this wave's row (two chunks)
        cbar(&bar, ep, &abt, opaque(A.err), lane);
        poll_pause<PAUSE_SPLIT>();
        poll_bf16<APT>(opaque(A.x_a) + (b % NREP) * RSA, HD, tag, ys, opaque(A.err), &abt, tid);
        cbar(&bar, ep, &abt, opaque(A.err), lane);
        {
            float a;
            if constexpr (Q8) {  // one chunk: the row's two halves as the chunk's two 2048-code rows
                const unsigned g = gb + S.oO() + wave;
                const unsigned char *c = chunk_get<NSM>(ring, ready, g, &abt, opaque(A.err));
                const uint16_t *sb = (const uint16_t *)(sbring + (size_t)(g % NSM) * SBM);
                a = dot_q8_row(c, 0, 1, sb, load_x8(ys, lane), lane) + dot_q8_row(c, 2, 3, sb + 64, load_x8(ys + HID, lane), lane);
                chunk_put_w<NSM>(done, g, lane, REL);
            } else {
                const unsigned g = gb + S.oO() + 2 * wave;
                const unsigned char *c = chunk_get<NSM>(ring, ready, g, &abt, opaque(A.err));
                a = dot_chunk(c, load_x(ys, lane), lane, 0.f);
                chunk_put_w<NSM>(done, g, lane, REL);
                const unsigned char *c2 = chunk_get<NSM>(ring, ready, g + 1, &abt, opaque(A.err));
                a = dot_chunk(c2, load_x(ys + HID, lane), lane, a);
                chunk_put_w<NSM>(done, g + 1, lane, REL);
            }
            const float acc = wave_sum(a);
            const int row = b * OPB + wave;
            if (lane < NREP) xstore(opaque(A.x_h2) + lane * RSH + row, tagw(tag, hs[row] + rho<bf16>(acc)));
        }

        // ---------------- step 5: y2 = RMSNorm(h); router row; routing; gate|up row pairs + SwiGLU
        cbar(&bar, ep, &abt, opaque(A.err), lane);  // every wave has read ys and hs before they are replaced
        poll_pause<PAUSE_VEC>();
        poll_bf16<HPT>(opaque(A.x_h2) + (b % NREP) * RSH, HID, tag, ys, opaque(A.err), &abt, tid);
        {
            float ss = 0.f;
#pragma unroll
            for (int k = 0; k < HPT; ++k) {
                const int i = tid + NCT * k;
                const float v = bfv(ys[i]);
                hs[i] = v;
                ss += v * v;
            }
            const float r = 1.0f / sqrtf(csum(ss, rsum, par, &bar, ep, &abt, opaque(A.err), tid) / (float)HID + A.eps);
#pragma unroll
            for (int k = 0; k < HPT; ++k) {
                const int i = tid + NCT * k;
                ys[i] = (uint16_t)f2bf_bits(w_post[k] * rho<bf16>(hs[i] * r));
            }
        }
        if (l + 1 < A.n_layers) load_small(l + 1);
        cbar(&bar, ep, &abt, opaque(A.err), lane);
        const X4 xg = load_x(ys, lane);
        const X8 xg8 = Q8 ? load_x8(ys, lane) : X8{};
        if (S.rc && wave == NC - 1) {  // router logit b = rho(y2 . Wr[b])
            const unsigned g = gb + S.oR();
            const unsigned char *c = chunk_get<NSM>(ring, ready, g, &abt, opaque(A.err));
            float acc;
            if constexpr (Q8)
                acc = wave_sum(dot_q8_row(c, 0, 1, (const uint16_t *)(sbring + (size_t)(g % NSM) * SBM), xg8, lane));
            else
                acc = wave_sum(dot_chunk(c, xg, lane, 0.f));
            chunk_put_w<NSM>(done, g, lane, REL);
            if (lane < NREP) xstore(opaque(A.x_r) + lane * RSR + b, tagw(tag, rho<bf16>(acc)));
        }
        if (wave == 0) {  // the token's routing, the same in every block
            poll_pause<PAUSE_VEC>();
            const uint32_t *src = opaque(A.x_r) + (b % NREP) * RSR;
            const int E = A.E;
            uint32_t v[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) v[i] = lane + 64 * i < E ? xload(src + lane + 64 * i) : (tag << 16);
            long sp = 0;
            while (true) {
                const bool ok = ((v[0] >> 16) == tag) && ((v[1] >> 16) == tag);
                if (__all(ok) || spin_out(++sp, opaque(A.err), &abt)) break;
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    if ((v[i] >> 16) != tag) v[i] = xload(src + lane + 64 * i);
            }
            float pr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) pr[i] = lane + 64 * i < E ? bfv((uint16_t)(v[i] & 0xffffu)) : -INFINITY;
            softmax_inplace<bf16, 2>(E, lane, pr);
            float psel[KSEL];
            int isel[KSEL];
            select_topk<2>(pr, E, KSEL, lane, psel, isel);
            float den = 0.f;
            for (int s = 0; s < KSEL; ++s) den += psel[s];
            const float denr = rho<bf16>(den);
            if (lane == 0) {
                for (int s = 0; s < KSEL; ++s) {
                    route_e[l & 1][s] = isel[s];
                    route_w[l & 1][s] = rho<bf16>(A.norm_topk ? psel[s] / denr : psel[s]);
                }
                __hip_atomic_store(&rgen, (unsigned)l + 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
        static_assert(GPB == 3 * NC, "three SwiGLU outputs per wave, packed into one exchange word");
        uint64_t mword = (uint64_t)tag << 48;
        for (int i = wave; i < GPB; i += NC) {
            float gs, us;
            if constexpr (Q8) {  // chunk i: the gate row and the up row of output i
                const unsigned g = gb + S.oG() + i;
                const unsigned char *c = chunk_get<NSM>(ring, ready, g, &abt, opaque(A.err));
                const uint16_t *sb = (const uint16_t *)(sbring + (size_t)(g % NSM) * SBM);
                gs = wave_sum(dot_q8_row(c, 0, 1, sb, xg8, lane));
                us = wave_sum(dot_q8_row(c, 2, 3, sb + 64, xg8, lane));
                chunk_put_w<NSM>(done, g, lane, REL);
            } else {
                const unsigned g = gb + S.oG() + 2 * i;
                const unsigned char *c = chunk_get<NSM>(ring, ready, g, &abt, opaque(A.err));
                gs = wave_sum(dot_chunk(c, xg, lane, 0.f));
                chunk_put_w<NSM>(done, g, lane, REL);
                const unsigned char *cu = chunk_get<NSM>(ring, ready, g + 1, &abt, opaque(A.err));
                us = wave_sum(dot_chunk(cu, xg, lane, 0.f));
                chunk_put_w<NSM>(done, g + 1, lane, REL);
            }
            const float mv = rho<bf16>(silu_f32(rho<bf16>(gs))) * rho<bf16>(us);
            mword |= (uint64_t)f2bf_bits(mv) << (16 * ((i - wave) / NC));
        }
        if (lane < NREP) xstore64((uint64_t *)opaque(A.x_m) + lane * (RSM / 2) + b * NC + wave, mword);

        // ---------------- step 6: pend = rho(sum_s rho(rho(m_s . Wdown_e(s)[n]) w_s)) for this wave's row n
        cbar(&bar, ep, &abt, opaque(A.err), lane);  // ys (y2) fully consumed; the routing weights are in LDS
        poll_pause<PAUSE_VEC>();
        static_assert(RSM % 2 == 0 && NB * NC % NCT == 0, "packed SwiGLU words: replica spacing, words per thread");
        poll_m3<NB * NC / NCT, GPB>((const uint64_t *)opaque(A.x_m) + (b % NREP) * (RSM / 2), NB * NC, tag, ys,
                                    opaque(A.err), &abt, tid);
        cbar(&bar, ep, &abt, opaque(A.err), lane);
        {
            float sacc[KSEL];
#pragma unroll
            for (int s = 0; s < KSEL; ++s) sacc[s] = 0.f;
#pragma unroll
            for (int q = 0; q < DCH; ++q) {
                const unsigned g = gb + S.oD() + wave * DCH + q;
                const unsigned char *c = chunk_get<NSM>(ring, ready, g, &abt, opaque(A.err));
                if constexpr (Q8) {
                    // third q: the lane's pieces are codes 2048 q + 1024 k + 16 lane .. + 15 (k = 0, 1), in
                    // groups 16 k + lane / 4 of the third; slot s0 for lanes below lb, else s0 + 1
                    const uint16_t *sb = (const uint16_t *)(sbring + (size_t)(g % NSM) * SBM);
                    const X8 x8 = load_x8(ys + q * HID, lane);
                    float pk[2];
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        const int gq = 16 * k + (lane >> 2);
                        pk[k] = q8_piece(c, k, bfv(sb[gq]), bfv(sb[32 + gq]), x8.v[2 * k], x8.v[2 * k + 1],
                                         k ? x8.s1 : x8.s0, lane);
                    }
                    chunk_put_w<NSM>(done, g, lane, REL);
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        const int base = 2048 * q + 1024 * k, s0 = base / IE, lb = ((s0 + 1) * IE - base) / 16;
                        const bool first = lane < lb;
                        sacc[s0] += first ? pk[k] : 0.f;
                        if (s0 + 1 < KSEL) sacc[s0 + 1] += first ? 0.f : pk[k];
                    }
                } else {
                    float pk[4];
                    dot_pieces(c, load_x(ys + q * HID, lane), lane, pk);
                    chunk_put_w<NSM>(done, g, lane, REL);
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        // inputs 2048 q + 512 k + 8 lane ..: slot s0 for lanes below lb, else s0 + 1
                        const int base = 2048 * q + 512 * k, s0 = base / IE, lb = ((s0 + 1) * IE - base) / 8;
                        const bool first = lane < lb;
                        sacc[s0] += first ? pk[k] : 0.f;
                        if (s0 + 1 < KSEL) sacc[s0 + 1] += first ? 0.f : pk[k];
                    }
                }
            }
            float acc = 0.f;
#pragma unroll
            for (int s = 0; s < KSEL; ++s) acc += rho<bf16>(rho<bf16>(wave_sum(sacc[s])) * route_w[l & 1][s]);
            const int row = b * OPB + wave;
            if (lane < NREP) xstore(opaque(A.x_pend) + lane * RSH + row, tagw(tag, acc));
        }
    }

    // ---------------- out = RMSNorm(rho(h + pend), final_norm) (block 0), then advance the counter
    if (b == 0) {
        const unsigned ltag = (tag0 + (unsigned)A.n_layers - 1u) & 0xffffu;
        cbar(&bar, ep, &abt, opaque(A.err), lane0);
        poll_bf16<HPT>(opaque(A.x_pend) + (b % NREP) * RSH, HID, ltag, ys, opaque(A.err), &abt, tid);
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < HPT; ++k) {
            const int i = tid + NCT * k;
            hs[i] = rho<bf16>(hs[i] + bfv(ys[i]));
            ss += hs[i] * hs[i];
        }
        const float r = 1.0f / sqrtf(csum(ss, rsum, par, &bar, ep, &abt, opaque(A.err), tid) / (float)HID + A.eps);
#pragma unroll
        for (int k = 0; k < HPT; ++k) {
            const int i = tid + NCT * k;
            opaque(A.out)[i] = bf16{(uint16_t)f2bf_bits(to_f(opaque(A.final_norm)[i]) * rho<bf16>(hs[i] * r))};
        }
        if (tid == 0) __hip_atomic_store(A.ctr, tag0 / 64u + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace mkm

// ------------------------------------------------------------ host side
namespace {
struct MoeMkLayout {
    size_t layers, layersq, qkv, a, h2, r, m, pend, part, ctr, total;
};
MoeMkLayout moe_mk_layout(int n_layers, int H, int KV) {
    using namespace mkm;
    const size_t nsplit = mk::NB / (KV > 0 ? KV : 1);
    auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
    MoeMkLayout L{};
    size_t o = 0;
    L.layers = o; o += al(sizeof(DevLayer) * n_layers);
    L.layersq = o; o += al(sizeof(DevLayerQ) * n_layers);
    L.qkv = o; o += al((size_t)NQKV * 4);
    L.a = o; o += al((size_t)NREP * rep_stride(HD) * 4);
    L.h2 = o; o += al((size_t)NREP * rep_stride(HID) * 4);
    L.r = o; o += al((size_t)NREP * rep_stride(EMAX) * 4);
    L.m = o; o += al((size_t)NREP * rep_stride(IM) * 4);
    L.pend = o; o += al((size_t)NREP * rep_stride(HID) * 4);
    L.part = o; o += al((size_t)H * nsplit * (D + 2) * 8);
    L.ctr = o; o += al(256);
    L.total = o;
    return L;
}
int moe_mk_chunk(int nkeys, int nsplit) {  // keys per split, a multiple of a K/V chunk's keys
    const int c = (nkeys + nsplit - 1) / nsplit;
    return (c + mk::KPC - 1) / mk::KPC * mk::KPC;
}
}  // namespace

size_t decode_moe_workspace(int n_layers, int H, int KV) { return moe_mk_layout(n_layers, H, KV).total; }

bool decode_moe_supported(int n_layers, int dt, int quant_bits, int hid, int H, int KV, int D, int E, int k, int Ie,
                          int cap) {
    using namespace mkm;
    if (dt != DT_BF16 || (quant_bits != 0 && quant_bits != 8) || D != mk::D || hid != HID || H * D != HD || KV < 1 || H != G * KV) return false;
    if ((H + 2 * KV) * D != NQKV || mk::NB % KV || mk::NB % H) return false;
    if (n_layers < 1 || n_layers > mk::MAXL) return false;  // tags are call * 64 + layer
    if (E < KSEL || E > EMAX || E > mk::NB || k != KSEL || Ie != IE) return false;
    const int nsplit = mk::NB / KV;
    if (nsplit > 64 || moe_mk_chunk(cap, nsplit) > CHM) return false;  // the split merge: two splits per lane
    return true;
}

hipError_t decode_moe_init(void *ws, int n_layers, int H, int KV, const void *layer_ptrs, const void *layer_q8_ptrs,
                           hipStream_t s) {
    const MoeMkLayout L = moe_mk_layout(n_layers, H, KV);
    char *b = (char *)ws;
    hipError_t e = hipMemcpyAsync(b + L.layers, layer_ptrs, sizeof(mkm::DevLayer) * n_layers, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return e;
    if (layer_q8_ptrs) {
        e = hipMemcpyAsync(b + L.layersq, layer_q8_ptrs, sizeof(mkm::DevLayerQ) * n_layers, hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return e;
    }
    // exchange words start with tag 0xffff, never the tag of a first call's layer
    e = hipMemsetAsync(b + L.qkv, 0xff, L.ctr - L.qkv, s);
    if (e != hipSuccess) return e;
    e = hipMemsetAsync(b + L.ctr, 0, 256, s);
    if (e != hipSuccess) return e;
    return hipStreamSynchronize(s);  // layer_ptrs is a caller's host array
}

hipError_t launch_decode_moe(void *ws, int n_layers, int H, int KV, int E, int norm_topk, bool q8, int cap, int p,
                             int window,
                             float eps, const void *x, void *out, const void *final_norm, const void *cos_t,
                             const void *sin_t, void *kc, void *vc, int *err, hipStream_t s) {
    const MoeMkLayout L = moe_mk_layout(n_layers, H, KV);
    char *b = (char *)ws;
    const int nsplit = mk::NB / KV;
    const int nvis = window > 0 ? min(p + 1, window) : p + 1;  // keys the new token sees
    if (p < 0 || p >= cap || window < 0 || n_layers < 1 || n_layers > mk::MAXL || moe_mk_chunk(nvis, nsplit) > mkm::CHM)
        return hipErrorInvalidValue;
    mkm::Args A;
    A.layers = (const mkm::DevLayer *)(b + L.layers);
    A.layersq = (const mkm::DevLayerQ *)(b + L.layersq);
    A.n_layers = n_layers;
    A.H = H;
    A.KV = KV;
    A.E = E;
    A.cap = cap;
    A.p = p;
    A.nsplit = nsplit;
    A.chunk = moe_mk_chunk(nvis, nsplit);
    A.window = window;
    A.norm_topk = norm_topk;
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
    A.x_r = (uint32_t *)(b + L.r);
    A.x_m = (uint32_t *)(b + L.m);
    A.x_pend = (uint32_t *)(b + L.pend);
    A.x_part = (uint64_t *)(b + L.part);
    A.ctr = (unsigned *)(b + L.ctr);
    A.err = err;
    void *args[] = {&A};
    const void *fn = q8 ? (const void *)mkm::decode_moe_kernel<true> : (const void *)mkm::decode_moe_kernel<false>;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(s, &cs);
    if (e != hipSuccess) return e;
    if (cs == hipStreamCaptureStatusNone)
        return hipLaunchCooperativeKernel(fn, dim3(mk::NB), dim3(mk::NTH), args, 0, s);
    // graph capture: a plain launch (the grid is one block per CU and fits the device at once)
    return hipLaunchKernel(fn, dim3(mk::NB), dim3(mk::NTH), args, 0, s);
}

int decode_moe_max_blocks(bool q8) {
    int per_cu = 0, dev = 0;
    const void *fn = q8 ? (const void *)mkm::decode_moe_kernel<true> : (const void *)mkm::decode_moe_kernel<false>;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, mk::NTH, 0) != hipSuccess) return 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
    return per_cu * prop.multiProcessorCount;
}

}  // namespace q3
