// kernels_decode_mk.hip -- the whole T = 1 decode step of a dense bf16 stack as one
// persistent kernel.
//
// What is computed is the layer of "maya2_mlx/backbone.py" (Backbone.forward and its
// docstring's rounding points) for one token at position p, through every layer, then the
// final norm; the kernels of kernels_linear.hip / kernels_attn.hip compute the same values.
//
// Why one kernel.  A decode layer is six dependent steps (q|k|v projection, split-K
// attention, split merge, o_proj + residual, gate|up + SwiGLU, down) whose weight streams are
// 8 - 50 MB each.  As separate kernels every step pays launch, ramp-up and drain (~3-5 us on
// gfx950), more than the 1 - 8 us the steps need at HBM speed.  Here 256 blocks (one per CU,
// co-resident) run all steps of all layers.
//
// Roles inside a block.  Waves 0-7 compute; waves 8-11 only stream.  The stream waves copy
// every weight row (and the K/V rows of the block's attention split) that the block will
// consume, in consumption order, from HBM straight into a ring of 4 KB LDS slots
// (global_load_lds_dwordx4 with the non-temporal policy, 1 KB per instruction), keeping up to
// DL chunks in flight each and running up to a full ring ahead of the compute waves, across
// step and layer boundaries; when the ring is full a stream wave lands and publishes all its chunks in
// flight before it waits for a slot, so the compute waves always see every landed chunk.
// The compute waves never issue weight loads: a wave's vector-memory counter retires loads
// in issue order, so a wave that polls another block's results while its own weight
// prefetch is in flight waits for that prefetch as well.  With the roles split, the
// compute waves' polls see a result as soon as it lands, and HBM streams while they wait.
// Ring handshake (LDS only): slot s holds chunk g with s = g mod NS; the stream wave writes
// ready[s] = g / NS + 1 after its counter shows the chunk landed, the consuming wave bumps
// done[s] after its reads of the chunk; the stream wave waits for done[s] == g / NS before it
// overwrites the slot.  Compute waves synchronise among themselves with an LDS counter
// barrier (the stream waves take part in no barrier after the prologue).
//
// 8-bit weights (u8 codes, bf16 scale s and bias b per group of 64 along K; w = s q + b in
// fp32, never rounded): a ring chunk holds the codes of two weight rows of 2048 (two q|k|v or
// o_proj rows, or the gate and the up row of one SwiGLU output) or one third of a down row,
// and a 256-byte side slot holds their groups' scales and biases.  A lane's dot is the
// regrouped sum s (x . q) + b (sum x) over each 16-code piece it holds.
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
// error word (the step's result is then invalid) and makes every other poll give up too.
#include "common.h"
#include "decode_mk_common.h"
#include "kernels.h"

namespace q3 {
namespace mk {

constexpr int NS = 32;               // ring slots (128 KB)
constexpr int NSQ = 30;              // ring slots with 8-bit weights (120 KB + 7.5 KB of scale/bias slots)
constexpr int SBB = 256;             // scale/bias bytes per chunk (8-bit weights)
constexpr int CHUNK_MAX = 256;       // keys per attention split
static_assert(NSQ >= NL * DL, "the ring holds every stream wave's chunks in flight");
template <bool Q8> __host__ __device__ constexpr int ring_slots() { return Q8 ? NSQ : NS; }

struct DevLayer {  // q_norm / k_norm both null: no per-head q/k norm; qkv_bias null: no bias
    const bf16 *in_norm, *post_norm, *q_norm, *k_norm, *qkv, *o, *gu, *down, *qkv_bias;
};

struct DevLayerQ {  // 8-bit weights: the per-group scale and bias arrays [rows][K / 64]
    const bf16 *qkv_s, *qkv_b, *o_s, *o_b, *gu_s, *gu_b, *down_s, *down_b;
};
static_assert(sizeof(DevLayerQ) == 64, "four (scale, bias) pairs of 16 bytes, read as pairs");

struct Args {
    const DevLayer *layers;
    const DevLayerQ *layersq;  // 8-bit weights only
    int n_layers, H, KV, cap, p, nsplit, chunk, window;  // window 0: causal
    float eps, scale;
    const bf16 *x, *final_norm, *cos_t, *sin_t;
    bf16 *out, *kc, *vc;
    uint32_t *x_qkv, *x_a, *x_h2, *x_m, *x_pend;
    uint64_t *x_part;
    unsigned *ctr;
    int *err;
};

// ---------------------------------------------------------------- per-block chunk sequence
// Per layer the block consumes, in this order: QPB q|k|v rows, nK K chunks and nK V chunks
// of its attention split (KPC keys each), OPB o rows, GPB gate/up row pairs (gate, then
// up), OPB down rows of DCH chunks each.  With 8-bit weights a chunk holds two q|k|v or o rows,
// or one gate/up pair (the gate row, then the up row), or one third of a down row.
template <int QPB, int GPB, int DCH, bool Q8> struct Seq {
    static constexpr int OPB = HID / NB;  // o rows (= down rows) per block
    static constexpr int QC = Q8 ? QPB / 2 : QPB, OC = Q8 ? OPB / 2 : OPB, GC = Q8 ? GPB : 2 * GPB, DC = OPB * DCH;
    int nK, cpl;
    __device__ explicit Seq(int nK_) : nK(nK_), cpl(QC + 2 * nK_ + OC + GC + DC) {}
    __device__ int oK() const { return QC; }
    __device__ int oV() const { return QC + nK; }
    __device__ int oO() const { return QC + 2 * nK; }
    __device__ int oG() const { return QC + 2 * nK + OC; }
    __device__ int oD() const { return QC + 2 * nK + OC + GC; }
};


// The scale and bias array pointers of field pair `pair` (0 q|k|v, 1 o, 2 gate|up, 3 down) of
// a layer's 8-bit table entry, read with one scalar load that completes inside the asm.  A
// vector load here would sit in the stream wave's vector-memory counter beside the ring copies,
// and the compiler then waits for every copy in flight before it uses the pointers.
__device__ __forceinline__ void load_scale_bias_ptrs(const DevLayerQ *e, int pair, const bf16 *&sc, const bf16 *&bi) {
    const uint64_t a = (uint64_t)e + 16u * (unsigned)pair;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a), hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    u32x4 v;
    __asm__ volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(((uint64_t)hi << 32) | lo) : "memory");
    typedef __attribute__((address_space(1))) const bf16 GB;
    sc = (const bf16 *)(GB *)(((uint64_t)v[1] << 32) | v[0]);
    bi = (const bf16 *)(GB *)(((uint64_t)v[3] << 32) | v[2]);
}

// Stream wave j (0 .. NL-1): chunks g = j, j + NL, ... of the whole step, in order.  With 8-bit
// weights every chunk is five copies (four 1 KB pieces of codes and one 256-byte scale/bias
// copy into the chunk's side slot; a K/V chunk's fifth copy re-reads 256 bytes of its keys
// into the unused side slot), so each chunk counts the same in the vector-memory counter.
template <int QPB, int GPB, int DCH, bool Q8>
__device__ void stream_wave(const Args &A, const Seq<QPB, GPB, DCH, Q8> &S, const DevLayer *lay, unsigned char *ring,
                            unsigned char *sbring, unsigned *ready, const unsigned *done, unsigned *abt, int j, int ag,
                            int j0, int j1) {
    constexpr int IM = GPB * NB;
    constexpr int NSL = ring_slots<Q8>(), VPC = Q8 ? 5 : 4;  // copies per chunk
    const int lane = tid_now() & 63, b = blockIdx.x;
    const unsigned total = (unsigned)A.n_layers * (unsigned)S.cpl;
    auto publish = [&](unsigned g) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (lane == 0) __hip_atomic_store(ready + g % NSL, g / NSL + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };
    // The compiler places this code after the compute waves' code and merges their pending
    // loads into its wait bookkeeping here; it cannot see the ring copies, which are asm, so
    // registers it still believes in flight would get waits inside the issue sequence below.
    // An explicit wait at entry (nothing of this wave is in flight yet) clears that state.
    wait_vm<0>();
    // n: own chunks issued; pub: own chunks published (chunk k of this wave is g = j + NL k)
    unsigned n = 0, pub = 0;
    for (unsigned g = j; g < total; g += NL) {
        const int l = (int)(g / (unsigned)S.cpl), idx = (int)(g - (unsigned)l * (unsigned)S.cpl);
        const DevLayer &L = lay[l];
        // the lane's source address for each of the chunk's four 1 KB pieces (and, 8-bit, of
        // its 4 bytes of the scale/bias copy)
        const unsigned char *src[4];
        const void *sbsrc = nullptr;
        if (idx < S.oK() || idx >= S.oO()) {
            if constexpr (Q8) {
                // codes rows of 2048 bytes: pieces 0, 1 of row r0 and 2, 3 of row r1; the scale/bias
                // copy: lanes 0-15 s[r0], 16-31 b[r0], 32-47 s[r1], 48-63 b[r1] (32 groups, 64 bytes each)
                const unsigned char *W;
                int r0, r1, ld = HID, ng = HID / 64, g0 = 0, pair;  // pair: the (scale, bias) field pair
                if (idx < S.oK()) {
                    W = (const unsigned char *)opaque(L.qkv), pair = 0;
                    r0 = b * QPB + 2 * idx, r1 = r0 + 1;
                } else if (idx < S.oG()) {
                    W = (const unsigned char *)opaque(L.o), pair = 1;
                    r0 = b * S.OPB + 2 * (idx - S.oO()), r1 = r0 + 1;
                } else if (idx < S.oD()) {
                    W = (const unsigned char *)opaque(L.gu), pair = 2;
                    r0 = b * GPB + (idx - S.oG()), r1 = IM + r0;
                } else {  // third t of down row r: codes t * 2048 .. + 2047, groups 32 t .. 32 t + 31
                    const int i = idx - S.oD(), t = i % DCH;
                    W = (const unsigned char *)opaque(L.down) + t * 2048, pair = 3;
                    r0 = r1 = b * S.OPB + i / DCH, ld = IM, ng = IM / 64, g0 = 32 * t;
                }
                const bf16 *sc, *bi;
                load_scale_bias_ptrs(A.layersq + l, pair, sc, bi);
                const unsigned char *w0 = W + (size_t)r0 * ld, *w1 = W + (size_t)r1 * ld;
                const bool second = idx >= S.oD();  // a down third: pieces 2, 3 repeat pieces 0, 1
                src[0] = w0 + lane * 16;
                src[1] = w0 + 1024 + lane * 16;
                src[2] = second ? src[0] : w1 + lane * 16;
                src[3] = second ? src[1] : w1 + 1024 + lane * 16;
                const int q = lane >> 4, row = (q < 2) ? r0 : r1;
                const bf16 *arr = (q & 1) ? bi : sc;  // a per-lane choice between two uniform arrays
                sbsrc = (const void *)(arr + (size_t)row * ng + g0 + 2 * (lane & 15));
            } else {
                const unsigned char *base;
                if (idx < S.oK()) {
                    base = (const unsigned char *)opaque(L.qkv) + ((size_t)b * QPB + idx) * CHB;
                } else if (idx < S.oG()) {
                    base = (const unsigned char *)opaque(L.o) + ((size_t)b * S.OPB + (idx - S.oO())) * CHB;
                } else if (idx < S.oD()) {
                    const int i = idx - S.oG();
                    base = (const unsigned char *)opaque(L.gu) + ((size_t)((i & 1) ? IM : 0) + (size_t)b * GPB + (i >> 1)) * CHB;
                } else {
                    const int i = idx - S.oD();
                    base = (const unsigned char *)opaque(L.down) + ((size_t)b * S.OPB + i / DCH) * ((size_t)IM * 2) +
                           (size_t)(i % DCH) * CHB;
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) src[k] = base + k * 1024 + lane * 16;
            }
        } else {
            const bool isV = idx >= S.oV();
            const int i = idx - (isV ? S.oV() : S.oK());
            const bf16 *cache = (isV ? opaque(A.vc) : opaque(A.kc)) + ((size_t)l * A.KV + ag) * A.cap * D;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                // keys past the split's end (a partial last chunk) re-read its last key
                const int key = min(j0 + i * KPC + 4 * k + lane / 16, j1 - 1);
                src[k] = (const unsigned char *)(cache + (size_t)key * D) + (lane % 16) * 16;
            }
            sbsrc = src[0];
        }
        const unsigned s = g % NSL, gen = g / NSL;
        if (lds_acquire(done + s) < gen) {
            // The ring is full: the compute waves still read the slot's previous chunk.  Land
            // and publish everything in flight first (nothing else can be issued meanwhile),
            // so the compute waves see the whole ring, then wait for the slot.
            wait_vm<0>();
            for (; pub < n; ++pub) publish(j + NL * pub);
            lds_wait_ge(done + s, gen, abt, nullptr);
        }
        unsigned char *dst = ring + (size_t)s * CHB;
        const unsigned dlds = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)dst);
#pragma unroll
        for (int k = 0; k < 4; ++k) dma16_nt(src[k], dlds + k * 1024);
        if constexpr (Q8) dma4(sbsrc, __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(sbring + (size_t)s * SBB)));
        ++n;
        if (n - pub >= DL) {
            wait_vm<VPC * (DL - 1)>();  // all but this wave's last DL-1 chunks have landed
            for (; pub + (DL - 1) < n; ++pub) publish(j + NL * pub);
        }
    }
    wait_vm<0>();
    for (; pub < n; ++pub) publish(j + NL * pub);
}

// ---------------------------------------------------------------- the kernel
// QPB q|k|v rows and GPB gate/up pairs per block; DCH chunks per down row; G query heads
// per kv head; Q8: 8-bit weights.
template <int QPB, int GPB, int DCH, int G, bool Q8>
__global__ void __launch_bounds__(NTH) decode_mk_kernel(Args A) {
    constexpr int IM = GPB * NB;
    constexpr int NSL = ring_slots<Q8>();
    constexpr int HPT = HID / NCT;  // words per compute thread of a hidden vector
    constexpr int OPB = HID / NB;
    constexpr int RSH = rep_stride(HID), RSM = rep_stride(IM);
    static_assert(IM * 2 == DCH * CHB && HID % NCT == 0 && IM % NCT == 0 && OPB == NC, "shape");
    __shared__ __attribute__((aligned(16))) unsigned char ring[NSL * CHB];
    __shared__ __attribute__((aligned(16))) unsigned char sbring[Q8 ? NSL * SBB : 16];  // 8-bit: scales and biases
    __shared__ unsigned ready[NSL], done[NSL], bar, abt;
    __shared__ DevLayer lay[MAXL];
    __shared__ float hs[HID];                                 // residual stream h (fp32 of bf16 values)
    __shared__ __attribute__((aligned(16))) uint16_t ys[IM];  // current projection input (bf16 bits)
    __shared__ __attribute__((aligned(16))) uint16_t qraw[G * D + 2 * D];
    __shared__ float qs[G * D], kvs[2 * D];
    // the attention's probabilities and per-wave partial outputs (then the split merge's buffer)
    // live in ys, which holds nothing between the q|k|v rows and the merged-output poll
    static_assert((G * CHUNK_MAX + NC * G * D) * 4 <= IM * 2, "attention buffers fit in ys");
    float *const sc = (float *)ys;
    float *const red = (float *)ys + G * CHUNK_MAX;
    __shared__ float rsum[2][NC];
    __shared__ float pm[NSPLIT_MAX], pl[NSPLIT_MAX];
    __shared__ float mwv[NC * G], lwv[NC * G];  // each wave's attention max and sum

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), b = blockIdx.x;
    const int H = A.H, KV = A.KV;
    const int p = A.p, nkeys = p + 1;
    const int bpg = NB / KV;               // attention blocks per kv head (= splits)
    const int ag = b / bpg, as = b % bpg;  // this block's (kv head, split)
    const int lo = A.window > 0 ? max(0, nkeys - A.window) : 0;  // first visible key (sliding window)
    const int j0 = lo + as * A.chunk, j1 = min(nkeys, j0 + A.chunk);
    const int nK = j0 < j1 ? (j1 - j0 + KPC - 1) / KPC : 0;
    const bool has_p = j0 < nkeys && j1 == nkeys;
    const Seq<QPB, GPB, DCH, Q8> S(nK);

    for (int i = tid; i < NSL; i += NTH) {
        ready[i] = 0;
        done[i] = 0;
    }
    if (tid == 0) {
        bar = 0;
        abt = 0;
    }
    for (int i = tid; i < A.n_layers; i += NTH) lay[i] = A.layers[i];
    const unsigned tag0 = A.ctr[0] * 64u;
    __syncthreads();  // the only barrier of the whole block; the roles split here

    if (wave >= NC) {
        stream_wave<QPB, GPB, DCH, Q8>(A, S, lay, ring, sbring, ready, done, &abt, wave - NC, ag, j0, j1);
        return;
    }

    // ================================================================ compute waves
    unsigned ep = 0, par = 0;
    const int dpb = H * D / NB;  // merged attention outputs per block
    const int mh = b / (NB / H), md0 = (b % (NB / H)) * dpb;
    constexpr int half = D / 2;
    const int jspec = has_p ? p : -1;              // the new key, taken from LDS

    const int lane0 = tid & 63;
    for (int k = 0; k < HPT; ++k) hs[tid + NCT * k] = to_f(opaque(A.x)[tid + NCT * k]);
    // per-layer vectors of this thread, loaded a step ahead of their use
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
        cbar(&bar, ep, &abt, opaque(A.err), lane);  // every wave is done reading ys (the previous layer's down rows)
        if (l > 0) {
            poll_pause<PAUSE_LONG>();
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
        // a q|k|v bias is its own rounded add after the projection: rho(rho(x W^T) + b)
        const bf16 *qb = lay[l].qkv_bias;
        if constexpr (Q8) {
            const X8 xq = load_x8(ys, lane);
            for (int i = wave; i < S.QC; i += NC) {  // chunk i: rows 2 i and 2 i + 1 of the block's QPB
                const unsigned g = gb + i;
                const unsigned char *c = chunk_get<NSL>(ring, ready, g, &abt, opaque(A.err));
                const uint16_t *sb = (const uint16_t *)(sbring + (size_t)(g % NSL) * SBB);
                float a0 = wave_sum(dot_q8_row(c, 0, 1, sb, xq, lane));
                float a1 = wave_sum(dot_q8_row(c, 2, 3, sb + 64, xq, lane));
                chunk_put<NSL>(done, g, lane);
                const int r0 = b * QPB + 2 * i;
                if (qb) {
                    a0 = rho<bf16>(a0) + to_f(opaque(qb)[r0]);
                    a1 = rho<bf16>(a1) + to_f(opaque(qb)[r0 + 1]);
                }
                if (lane == 0) xstore(opaque(A.x_qkv) + r0, tagw(tag, a0));
                if (lane == 1) xstore(opaque(A.x_qkv) + r0 + 1, tagw(tag, a1));
            }
        } else {
            const X4 xq = load_x(ys, lane);
            for (int i = wave; i < QPB; i += NC) {
                const unsigned g = gb + i;
                const unsigned char *c = chunk_get<NSL>(ring, ready, g, &abt, opaque(A.err));
                float acc = wave_sum(dot_chunk(c, xq, lane, 0.f));
                chunk_put<NSL>(done, g, lane);
                if (qb) acc = rho<bf16>(acc) + to_f(opaque(qb)[(size_t)b * QPB + i]);
                if (lane == 0) xstore(opaque(A.x_qkv) + (size_t)b * QPB + i, tagw(tag, acc));
            }
        }

        poll_pause<PAUSE_LONG>();
        // ---------------- step 2: per-head q/k norm + RoPE + cache write, split-K attention
        if (nK > 0) {
            // the group's q heads, and for the block holding the new key its k and v heads, in
            // one round of loads (thread t < G*D: q word t; then k words; then v words)
            static_assert(G * D + 2 * D <= NCT, "one word per thread");
            const int nw = G * D + (has_p ? 2 * D : 0);
            if (tid < nw) {
                const int src = tid < G * D ? ag * G * D + tid
                                            : (tid < G * D + D ? (H + ag) * D + tid - G * D
                                                               : (H + KV + ag) * D + tid - G * D - D);
                const uint32_t *w = opaque(A.x_qkv) + src;
                uint32_t v = xload(w);
                long sp = 0;
                while ((v >> 16) != tag) {
                    if (spin_out(++sp, opaque(A.err), &abt)) break;
                    v = xload(w);
                }
                qraw[tid] = (uint16_t)(v & 0xffffu);
            }
        }
        cbar(&bar, ep, &abt, opaque(A.err), lane);
        if (nK > 0 && wave < G + (has_p ? 1 : 0)) {
            const int hh = wave;
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
        cbar(&bar, ep, &abt, opaque(A.err), lane);
        if (nK > 0) {
            // Each wave takes K chunk i and V chunk i (i = wave, wave + NC, ...): the scores of the
            // chunk's KPC keys, their exponentials against the wave's running maximum, and p . V,
            // so the waves need no barrier between scores, softmax and p . V; the waves' (max,
            // sum, o) are combined once below.  K chunk i holds keys j0 + KPC*i ..; the lane's
            // piece k is key 4k + kslot, dims sub*8 .. sub*8+7.  q and the new key are bf16 values
            // (rounded after RoPE), so packing them is exact and each 8-dim piece of a score is
            // four v_dot2c_f32_bf16.  In p . V lane l owns dims 2l, 2l+1 of every key; the
            // probabilities go through the wave's own rows of sc (no other wave reads them).
            u32x4 qp[G];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float *qh = qs + h * D + sub * 8;
                qp[h] = u32x4{pack_bf2(qh[0], qh[1]), pack_bf2(qh[2], qh[3]), pack_bf2(qh[4], qh[5]),
                              pack_bf2(qh[6], qh[7])};
            }
            const float *kn = kvs + sub * 8;
            const u32x4 knew = {pack_bf2(kn[0], kn[1]), pack_bf2(kn[2], kn[3]), pack_bf2(kn[4], kn[5]),
                                pack_bf2(kn[6], kn[7])};
            const float vs0 = kvs[D + 2 * lane], vs1 = kvs[D + 2 * lane + 1];
            float mw[G], lw[G], o[G][2];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                mw[h] = -INFINITY;
                lw[h] = 0.f;
                o[h][0] = o[h][1] = 0.f;
            }
            for (int i = wave; i < nK; i += NC) {
                const unsigned gk = gb + S.oK() + i;
                const unsigned char *c = chunk_get<NSL>(ring, ready, gk, &abt, opaque(A.err));
                u32x4 kr[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) kr[k] = *(const u32x4 *)(c + k * 1024 + lane * 16);
                float sv[G][4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int j = j0 + i * KPC + 4 * k + kslot;
                    const u32x4 kw = j == jspec ? knew : kr[k];
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        const float sdot = row16_sum(dot16<bf16>(qp[h], kw, 0.f));  // the key's 16 lanes form one DPP row
                        sv[h][k] = j < j1 ? sdot * A.scale : -INFINITY;
                    }
                }
                chunk_put<NSL>(done, gk, lane);
                const int jb = j0 + i * KPC;
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    float cm = fmaxf(fmaxf(sv[h][0], sv[h][1]), fmaxf(sv[h][2], sv[h][3]));
                    cm = fmaxf(fmaxf(lane_f(cm, 0), lane_f(cm, 16)), fmaxf(lane_f(cm, 32), lane_f(cm, 48)));
                    const float mn = fmaxf(mw[h], cm);  // finite: key jb is below j1
                    const float alpha = __expf(mw[h] - mn);
                    float ps = 0.f;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const float e = __expf(sv[h][k] - mn);
                        ps += e;
                        if (sub == 0) sc[h * CHUNK_MAX + (jb + 4 * k + kslot - j0)] = e;
                    }
                    ps = (lane_f(ps, 0) + lane_f(ps, 16)) + (lane_f(ps, 32) + lane_f(ps, 48));
                    lw[h] = lw[h] * alpha + ps;
                    o[h][0] *= alpha;
                    o[h][1] *= alpha;
                    mw[h] = mn;
                }
                const unsigned gv = gb + S.oV() + i;
                c = chunk_get<NSL>(ring, ready, gv, &abt, opaque(A.err));
                // all KPC rows are read (rows past the split's end hold a copy of its last key
                // and have probability 0); reads first, then the arithmetic
                uint32_t vw[KPC];
                float pe[G][KPC];
#pragma unroll
                for (int kk = 0; kk < KPC; ++kk) vw[kk] = *(const uint32_t *)(c + kk * (D * 2) + lane * 4);
#pragma unroll
                for (int h = 0; h < G; ++h)
#pragma unroll
                    for (int kk = 0; kk < KPC; ++kk) pe[h][kk] = sc[h * CHUNK_MAX + (jb + kk - j0)];
#pragma unroll
                for (int kk = 0; kk < KPC; ++kk) {
                    float v0 = bf_lo(vw[kk]), v1 = bf_hi(vw[kk]);
                    if (jb + kk == jspec) {
                        v0 = vs0;
                        v1 = vs1;
                    }
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        o[h][0] += pe[h][kk] * v0;
                        o[h][1] += pe[h][kk] * v1;
                    }
                }
                chunk_put<NSL>(done, gv, lane);
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                red[(wave * G + h) * D + 2 * lane] = o[h][0];
                red[(wave * G + h) * D + 2 * lane + 1] = o[h][1];
                if (lane == 0) {
                    mwv[wave * G + h] = mw[h];
                    lwv[wave * G + h] = lw[h];
                }
            }
        }
        cbar(&bar, ep, &abt, opaque(A.err), lane);
        if (nK > 0) {
            // the split's (max, sum, o) from the waves' (waves without a chunk hold max -inf, sum 0)
            for (int idx = tid; idx < G * D; idx += NCT) {
                const int i = idx / D, d = idx % D;
                float m = -INFINITY;
#pragma unroll
                for (int w = 0; w < NC; ++w) m = fmaxf(m, mwv[w * G + i]);
                float v = 0.f;
#pragma unroll
                for (int w = 0; w < NC; ++w) v += red[(w * G + i) * D + d] * __expf(mwv[w * G + i] - m);
                xstore64(opaque(A.x_part) + ((size_t)(ag * G + i) * A.nsplit + as) * (D + 2) + 2 + d,
                         ((uint64_t)tag << 32) | __float_as_uint(v));
            }
            if (tid < G) {
                float m = -INFINITY, ls = 0.f;
#pragma unroll
                for (int w = 0; w < NC; ++w) m = fmaxf(m, mwv[w * G + tid]);
#pragma unroll
                for (int w = 0; w < NC; ++w) ls += lwv[w * G + tid] * __expf(mwv[w * G + tid] - m);
                uint64_t *pp = opaque(A.x_part) + ((size_t)(ag * G + tid) * A.nsplit + as) * (D + 2);
                xstore64(pp, ((uint64_t)tag << 32) | __float_as_uint(m));
                xstore64(pp + 1, ((uint64_t)tag << 32) | __float_as_uint(ls));
            }
        } else {  // an empty split (fewer keys than splits): max -inf, sum 0
            for (int idx = tid; idx < G * (D + 2); idx += NCT) {
                const int i = idx / (D + 2), e = idx % (D + 2);
                const float v = e == 0 ? -INFINITY : 0.f;
                xstore64(opaque(A.x_part) + ((size_t)(ag * G + i) * A.nsplit + as) * (D + 2) + e,
                         ((uint64_t)tag << 32) | __float_as_uint(v));
            }
        }

        // ---------------- step 3: merge the splits of (head mh, dims md0 .. md0 + dpb)
        cbar(&bar, ep, &abt, opaque(A.err), lane);  // red has been read before it becomes the merge buffer
        poll_pause<PAUSE_SPLIT>();
        {
            const int ns = A.nsplit;
            const int nwords = ns * (2 + dpb);
            float *po = red;  // [ns][dpb]
            for (int t = tid; t < nwords; t += NCT) {
                const uint64_t *src;
                if (t < 2 * ns) src = opaque(A.x_part) + ((size_t)mh * ns + t / 2) * (D + 2) + (t % 2);
                else {
                    const int u = t - 2 * ns;
                    src = opaque(A.x_part) + ((size_t)mh * ns + u / dpb) * (D + 2) + 2 + md0 + u % dpb;
                }
                uint64_t v = xload64(src);
                long sp = 0;
                while ((unsigned)(v >> 32) != tag) {
                    if (spin_out(++sp, opaque(A.err), &abt)) break;
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
            cbar(&bar, ep, &abt, opaque(A.err), lane);
            float av;
            if (merge_lds<8>(pm, pl, po, ns, dpb, tid, &av)) {  // wave 0: 8 lanes per dim
                const uint32_t w = tagw(tag, av);
#pragma unroll
                for (int r = 0; r < NREP; ++r) xstore(opaque(A.x_a) + r * RSH + mh * D + md0 + tid / 8, w);
            }
        }

        // ---------------- step 4: h = rho(h + rho(a . Wo^T)) for this wave's row
        // the merge has read its buffer (in ys) before ys receives a; the barrier also keeps the other
        // waves' polls of a from starting while wave 0 still merges (1.7B step ~723 -> ~708 us; with
        // the ring's two extra slots ~705; a barrier before the q|k|v poll instead cost ~5 us)
        cbar(&bar, ep, &abt, opaque(A.err), lane);
        poll_pause<PAUSE_SPLIT>();
        poll_bf16<HPT>(opaque(A.x_a) + (b % NREP) * RSH, HID, tag, ys, opaque(A.err), &abt, tid);
        cbar(&bar, ep, &abt, opaque(A.err), lane);
        if constexpr (Q8) {
            if (wave < S.OC) {  // chunk wave: rows 2 wave and 2 wave + 1 of the block's OPB
                const unsigned g = gb + S.oO() + wave;
                const unsigned char *c = chunk_get<NSL>(ring, ready, g, &abt, opaque(A.err));
                const uint16_t *sb = (const uint16_t *)(sbring + (size_t)(g % NSL) * SBB);
                const X8 xo = load_x8(ys, lane);
                const float a0 = wave_sum(dot_q8_row(c, 0, 1, sb, xo, lane));
                const float a1 = wave_sum(dot_q8_row(c, 2, 3, sb + 64, xo, lane));
                chunk_put<NSL>(done, g, lane);
                const int row = b * OPB + 2 * wave;
                if (lane < NREP) xstore(opaque(A.x_h2) + lane * RSH + row, tagw(tag, hs[row] + rho<bf16>(a0)));
                else if (lane >= 32 && lane < 32 + NREP)
                    xstore(opaque(A.x_h2) + (lane - 32) * RSH + row + 1, tagw(tag, hs[row + 1] + rho<bf16>(a1)));
            }
        } else {
            const unsigned g = gb + S.oO() + wave;
            const unsigned char *c = chunk_get<NSL>(ring, ready, g, &abt, opaque(A.err));
            const float acc = wave_sum(dot_chunk(c, load_x(ys, lane), lane, 0.f));
            chunk_put<NSL>(done, g, lane);
            const int row = b * OPB + wave;
            if (lane < NREP) xstore(opaque(A.x_h2) + lane * RSH + row, tagw(tag, hs[row] + rho<bf16>(acc)));
        }

        // ---------------- step 5: y2 = RMSNorm(h); gate|up row pairs + SwiGLU
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
        static_assert(GPB == 3 * NC, "three SwiGLU outputs per wave, packed into one exchange word");
        uint64_t mword = (uint64_t)tag << 48;
        if constexpr (Q8) {
            const X8 xg = load_x8(ys, lane);
            for (int i = wave; i < GPB; i += NC) {  // chunk i: the gate row and the up row of output i
                const unsigned g = gb + S.oG() + i;
                const unsigned char *c = chunk_get<NSL>(ring, ready, g, &abt, opaque(A.err));
                const uint16_t *sb = (const uint16_t *)(sbring + (size_t)(g % NSL) * SBB);
                const float gs = wave_sum(dot_q8_row(c, 0, 1, sb, xg, lane));
                const float us = wave_sum(dot_q8_row(c, 2, 3, sb + 64, xg, lane));
                chunk_put<NSL>(done, g, lane);
                const float mv = rho<bf16>(silu_f32(rho<bf16>(gs))) * rho<bf16>(us);
                mword |= (uint64_t)f2bf_bits(mv) << (16 * ((i - wave) / NC));
            }
        } else {
            const X4 xg = load_x(ys, lane);
            for (int i = wave; i < GPB; i += NC) {
                const unsigned g = gb + S.oG() + 2 * i;
                const unsigned char *c = chunk_get<NSL>(ring, ready, g, &abt, opaque(A.err));
                const float gs = wave_sum(dot_chunk(c, xg, lane, 0.f));
                chunk_put<NSL>(done, g, lane);
                const unsigned char *cu = chunk_get<NSL>(ring, ready, g + 1, &abt, opaque(A.err));
                const float us = wave_sum(dot_chunk(cu, xg, lane, 0.f));
                chunk_put<NSL>(done, g + 1, lane);
                const float mv = rho<bf16>(silu_f32(rho<bf16>(gs))) * rho<bf16>(us);
                mword |= (uint64_t)f2bf_bits(mv) << (16 * ((i - wave) / NC));
            }
        }
        if (lane < NREP) xstore64((uint64_t *)opaque(A.x_m) + lane * (RSM / 2) + b * NC + wave, mword);

        // ---------------- step 6: pend = rho(m . Wdown^T) for this wave's row
        cbar(&bar, ep, &abt, opaque(A.err), lane);  // ys (y2) fully consumed before it receives m
        poll_pause<PAUSE_VEC>();
        static_assert(RSM % 2 == 0 && NB * NC % NCT == 0, "packed SwiGLU words: replica spacing, words per thread");
        poll_m3<NB * NC / NCT, GPB>((const uint64_t *)opaque(A.x_m) + (b % NREP) * (RSM / 2), NB * NC, tag, ys,
                                    opaque(A.err), &abt, tid);
        cbar(&bar, ep, &abt, opaque(A.err), lane);
        {
            float a = 0.f;
#pragma unroll
            for (int q = 0; q < DCH; ++q) {
                const unsigned g = gb + S.oD() + wave * DCH + q;
                const unsigned char *c = chunk_get<NSL>(ring, ready, g, &abt, opaque(A.err));
                if constexpr (Q8) {  // third q of the row: codes q * 2048 .. + 2047
                    const uint16_t *sb = (const uint16_t *)(sbring + (size_t)(g % NSL) * SBB);
                    a += dot_q8_row(c, 0, 1, sb, load_x8(ys + q * HID, lane), lane);
                } else {
                    a = dot_chunk(c, load_x(ys + q * HID, lane), lane, a);
                }
                chunk_put<NSL>(done, g, lane);
            }
            const float acc = wave_sum(a);
            if (lane < NREP) xstore(opaque(A.x_pend) + lane * RSH + b * OPB + wave, tagw(tag, acc));
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

}  // namespace mk

// ------------------------------------------------------------ host side
namespace {
struct MkLayout {
    size_t layers, layersq, qkv, a, h2, m, pend, part, ctr, total;
};
MkLayout mk_layout(int n_layers, int H, int KV, int hid, int I) {
    const size_t nsplit = mk::NB / (KV > 0 ? KV : 1);
    auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
    const size_t nqkv = (size_t)(H + 2 * KV) * mk::D;
    MkLayout L{};
    size_t o = 0;
    L.layers = o; o += al(sizeof(mk::DevLayer) * n_layers);
    L.layersq = o; o += al(sizeof(mk::DevLayerQ) * n_layers);
    L.qkv = o; o += al(nqkv * 4);
    const size_t rh = (size_t)mk::NREP * mk::rep_stride(hid) * 4, rm = (size_t)mk::NREP * mk::rep_stride(I) * 4;
    L.a = o; o += al(rh);
    L.h2 = o; o += al(rh);
    L.m = o; o += al(rm);
    L.pend = o; o += al(rh);
    L.part = o; o += al((size_t)H * nsplit * (mk::D + 2) * 8);
    L.ctr = o; o += al(256);
    L.total = o;
    return L;
}

template <int QPB, int GPB, int DCH, int G, bool Q8> const void *mk_fn() {
    return (const void *)mk::decode_mk_kernel<QPB, GPB, DCH, G, Q8>;
}

const void *mk_select(int hid, int I, int G, int nqkv, bool q8) {
    if (hid == 2048 && I == 6144 && nqkv == 4096 && G == 2) return q8 ? mk_fn<16, 24, 3, 2, true>() : mk_fn<16, 24, 3, 2, false>();
    return nullptr;
}

int mk_chunk(int nkeys, int nsplit) {  // keys per split, a multiple of a K/V chunk's keys
    const int c = (nkeys + nsplit - 1) / nsplit;
    return (c + mk::KPC - 1) / mk::KPC * mk::KPC;
}
}  // namespace

size_t decode_mk_workspace(int n_layers, int H, int KV, int hid, int I) { return mk_layout(n_layers, H, KV, hid, I).total; }

bool decode_mk_supported(int n_layers, int dt, int n_experts, int quant_bits, int hid, int H, int KV, int D, int I,
                         int cap) {
    if (dt != DT_BF16 || n_experts > 0 || (quant_bits != 0 && quant_bits != 8) || D != mk::D) return false;
    if (n_layers < 1 || n_layers > mk::MAXL) return false;  // tags are call * 64 + layer
    if (hid != mk::HID || H * D != hid || H % KV || mk::NB % KV || mk::NB % H) return false;
    const int nsplit = mk::NB / KV;
    if (nsplit > mk::NSPLIT_MAX || mk_chunk(cap, nsplit) > mk::CHUNK_MAX) return false;
    if (nsplit * (2 + H * D / mk::NB) > mk::NC * (H / KV) * mk::D) return false;  // merge buffer fits in LDS
    if (8 * (H * D / mk::NB) > 64) return false;  // the merge: one wave, 8 lanes per dim
    return mk_select(hid, I, H / KV, (H + 2 * KV) * D, quant_bits == 8) != nullptr;
}

hipError_t decode_mk_init(void *ws, int n_layers, int H, int KV, int hid, int I, const void *layer_ptrs,
                          const void *layer_q8_ptrs, hipStream_t s) {
    const MkLayout L = mk_layout(n_layers, H, KV, hid, I);
    char *b = (char *)ws;
    hipError_t e = hipMemcpyAsync(b + L.layers, layer_ptrs, sizeof(mk::DevLayer) * n_layers, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return e;
    if (layer_q8_ptrs) {
        e = hipMemcpyAsync(b + L.layersq, layer_q8_ptrs, sizeof(mk::DevLayerQ) * n_layers, hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return e;
    }
    // exchange words start with tag 0xffff, never the tag of a first call's layer
    e = hipMemsetAsync(b + L.qkv, 0xff, L.ctr - L.qkv, s);
    if (e != hipSuccess) return e;
    e = hipMemsetAsync(b + L.ctr, 0, 256, s);
    if (e != hipSuccess) return e;
    return hipStreamSynchronize(s);  // layer_ptrs is a caller's host array
}

hipError_t launch_decode_mk(void *ws, int n_layers, int H, int KV, int hid, int I, bool q8, int cap, int p, int window,
                            float eps, const void *x, void *out, const void *final_norm, const void *cos_t,
                            const void *sin_t, void *kc, void *vc, int *err, hipStream_t s) {
    const MkLayout L = mk_layout(n_layers, H, KV, hid, I);
    char *b = (char *)ws;
    const int nsplit = mk::NB / KV;
    const void *fn = mk_select(hid, I, H / KV, (H + 2 * KV) * mk::D, q8);
    const int nvis = window > 0 ? min(p + 1, window) : p + 1;  // keys the new token sees
    if (!fn || p < 0 || p >= cap || window < 0 || n_layers < 1 || n_layers > mk::MAXL ||
        mk_chunk(nvis, nsplit) > mk::CHUNK_MAX)
        return hipErrorInvalidValue;
    mk::Args A;
    A.layers = (const mk::DevLayer *)(b + L.layers);
    A.layersq = (const mk::DevLayerQ *)(b + L.layersq);
    A.n_layers = n_layers;
    A.H = H;
    A.KV = KV;
    A.cap = cap;
    A.p = p;
    A.nsplit = nsplit;
    A.chunk = mk_chunk(nvis, nsplit);
    A.window = window;
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
    void *args[] = {&A};
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(s, &cs);
    if (e != hipSuccess) return e;
    if (cs == hipStreamCaptureStatusNone)
        return hipLaunchCooperativeKernel(fn, dim3(mk::NB), dim3(mk::NTH), args, 0, s);
    // graph capture: a plain launch (the grid is one block per CU and fits the device at once)
    return hipLaunchKernel(fn, dim3(mk::NB), dim3(mk::NTH), args, 0, s);
}

int decode_mk_max_blocks(int hid, int I, int H, int KV, bool q8) {
    const void *fn = mk_select(hid, I, H / KV, (H + 2 * KV) * mk::D, q8);
    if (!fn) return 0;
    int per_cu = 0, dev = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, mk::NTH, 0) != hipSuccess) return 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
    return per_cu * prop.multiProcessorCount;
}

int decode_mk_blocks() { return mk::NB; }

}  // namespace q3
