// paged_attn_decode: one query token per sequence over an E4M3 paged cache.
//
// Math [P1, llama-graph.cpp build_attn_scale_kv_inputs/_output; tests
// check_fp8_attention]: with K_t, V_t the stored codes' values,
//   s_t = (q . K_t) * k_scale * sm_scale,   o = v_scale * sum_t softmax(s)_t V_t,
// i.e. attention over the dequantized cache with both scales moved out of
// the inner products.  Query head h reads kv-head h / G (G = Hq / Hkv).
//
// Work decomposition.  A 1-D grid of units (pair = sequence * Hkv + kv-head,
// split), spread evenly over the 8 XCDs (decode_unit); a workgroup of four
// waves owns one chunk of one sequence's tokens for one kv-head and all G
// query heads of that group.  Each wave walks 32-token steps (two 16-token
// tiles) of the chunk, interleaved with the other waves:
//   * lane (m = lane%16, g = lane/16) loads, per tile, D/4 elements of K
//     (token m, column quarter g) and D/4 elements of V (four tokens
//     4g..4g+3 for dims (D/16)m .. (D/16)m + D/16 - 1); in the tile layout
//     both are contiguous, so a wave reads each tile with 16-byte loads
//     covering it exactly;
//   * S^T[token][head] = K Q^T on v_mfma_f32_16x16x32_bf16 (E4M3 codes ->
//     bf16 is exact; a bf16 pool is the operand as stored); its output
//     layout (lane (n, g) holds tokens 4g..4g+3 of head n) is exactly the B
//     operand of the next product;
//   * O^T[d][head] += V^T P^T on v_mfma_f32_16x16x32_f16 for E4M3 V (codes ->
//     f16 exact, P split into two f16 terms), or on the bf16 MFMA for a bf16
//     V pool with P split into two bf16 terms, over 32 tokens per
//     instruction;
//   * the online softmax runs in the log2 domain against a per-head reference
//     max that only moves when a score exceeds it by more than 2^8 (lazy
//     rescale), with per-lane partial sums.
// The loads of the next NBUF - 1 steps are in flight in a per-lane register
// ring (inline loads with explicit vmcnt waits for E4M3 pools); a wave's
// block ids are preloaded.
// The four waves then combine through LDS; with one split the workgroup
// writes the output, otherwise it writes (max, sum, acc) partials that
// decode_reduce combines.

#include "fp8_device.hpp"
#include "decode_args.hpp"


namespace kvf8 {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
static_assert(kThreads == kDecodeThreads, "host launch checks assume this workgroup size");
constexpr int kStep = 32;                 // tokens per wave step
constexpr float kLazy = 8.0f;             // log2 headroom of the lazy softmax reference

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);   // quiet NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ void store_out(void *out, int64_t idx, float v, int bf16) {
    if (bf16)
        static_cast<uint16_t *>(out)[idx] = f32_to_bf16_rne(v);
    else
        static_cast<float *>(out)[idx] = v;
}

// Registers of one 32-token step of one lane: per 16-token tile, its D/4
// elements of one key (K) and 4 keys x D/16 dims (V).  KB / VB are the pools'
// element bytes: 1 (E4M3 codes) or 2 (bf16 values).
template <int D, int KB, int VB>
struct StepRegs {
    static constexpr int NK = D * KB / 64;     // 16-byte loads per lane per tile, K
    static constexpr int NV = D * VB / 64;     // and V
    u32x4 k[2][NK];
    u32x4 v[2][NV];
    __device__ __forceinline__ uint32_t kw(int t, int j) const { return k[t][j >> 2][j & 3]; }
    __device__ __forceinline__ uint32_t vw(int t, int j) const { return v[t][j >> 2][j & 3]; }
};

// The all-E4M3 ring issues its loads as inline global_load_dwordx4 and waits
// for them explicitly (below): the compiler's own wait placement drained
// every outstanding load at the loop head.  That is only sound while the
// register allocator neither copies, reuses nor spills a ring register
// between its load and its wait.  tests/test_decode_ring_asm.py proves that on
// the compiled assembly of every all-E4M3 instance (a dataflow pass over the
// kernel's branches and loop); the bf16 and mixed-type rings are heavier and
// use plain loads, whose waits the compiler places itself.
template <int KB, int VB>
struct AsmRing { static constexpr bool ON = KB == 1 && VB == 1; };

// 16 bytes at p + OFF (OFF an immediate of the instruction).
template <bool ASM, int OFF>
__device__ __forceinline__ void gload16(u32x4 &dst, const uint8_t *p) {
    if constexpr (ASM)
        asm volatile("global_load_dwordx4 %0, %1, off offset:%2" : "=v"(dst) : "v"(p), "n"(OFF) : "memory");
    else
        dst = *reinterpret_cast<const u32x4 *>(p + OFF);
}

// N consecutive 16-byte loads at p + 16*I, I = 0..N-1 (immediate offsets).
template <bool ASM, int I, int N>
struct LoadRun {
    static __device__ __forceinline__ void run(u32x4 *dst, const uint8_t *p) {
        if constexpr (I < N) {
            gload16<ASM, 16 * I>(dst[I], p);
            LoadRun<ASM, I + 1, N>::run(dst, p);
        }
    }
};

// A 64-bit address that is the same in every lane, kept as one scalar value
// (so that the per-lane part of a load address is a single add).
__device__ __forceinline__ const uint8_t *uniform_ptr(const uint8_t *p) {
    const uint64_t u = (uint64_t)p;
    return reinterpret_cast<const uint8_t *>(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(u >> 32)) << 32) |
                                             (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)u));
}

// Wait until at most N vector-memory loads are outstanding, then hand the
// step's registers on: every register of the buffer is an operand of the
// wait, so no use of it can be scheduled before the wait.
template <int N, int D, int KB, int VB>
__device__ __forceinline__ void wait_step(StepRegs<D, KB, VB> &r) {
    if constexpr (!AsmRing<KB, VB>::ON) return;
    asm volatile("s_waitcnt vmcnt(%1)" : "+v"(r.k[0][0]) : "n"(N) : "memory");
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int i = 0; i < StepRegs<D, KB, VB>::NK; ++i) asm volatile("" : "+v"(r.k[t][i]));
#pragma unroll
        for (int i = 0; i < StepRegs<D, KB, VB>::NV; ++i) asm volatile("" : "+v"(r.v[t][i]));
    }
}

// Issue the loads of one 32-token step: per lane, for each of the two
// 16-token tiles, the D/4 elements of key m in column quarter g (K) and keys
// 4g..4g+3 of dims (D/16)m.. (V), as 16-byte loads.  blk0 / blk1 are the
// pool blocks of the two tiles.  A tile's base (block, kv-head and first
// in-block key) is the same for the whole wave and is formed as a scalar; the
// lane adds its fixed offsets koff / voff ((g*BS + m)*D/4 and
// (g*D + (D/16)m)*4 elements), and the 16-byte pieces are immediate offsets
// of the loads.  A step past the wave's end (live == false) keeps the same
// number of loads but reads the first bytes of the K pool, so the ring stays
// branch-free without moving extra bytes.
template <int D, int BS, int KB, int VB>
__device__ __forceinline__ void load_step(StepRegs<D, KB, VB> &r, const uint8_t *k_pool, const uint8_t *v_pool,
                                          uint32_t blk0, uint32_t blk1, int kv_heads, int kvh, int p,
                                          uint32_t koff, uint32_t voff, bool live) {
    constexpr int Q4 = D / 4;
    using R = StepRegs<D, KB, VB>;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const uint32_t blk = t == 0 ? blk0 : blk1;
        const int tb = (p + 16 * t) % BS;
        const int64_t tile = ((int64_t)blk * kv_heads + kvh) * (BS * D);     // element index of the tile
        const uint8_t *kb = uniform_ptr(live ? k_pool + (tile + (int64_t)tb * Q4) * KB : k_pool);
        const uint8_t *vb = uniform_ptr(live ? v_pool + (tile + (int64_t)(tb / 4) * D * 4) * VB : k_pool);
        const uint8_t *kp = kb + (live ? koff : 0u);
        const uint8_t *vp = vb + (live ? voff : 0u);
        LoadRun<AsmRing<KB, VB>::ON, 0, R::NK>::run(r.k[t], kp);
        LoadRun<AsmRing<KB, VB>::ON, 0, R::NV>::run(r.v[t], vp);
    }
}

// Online-softmax state of one wave: the O^T accumulators of its lane and the
// running max / partial sum of its head column.
template <int D>
struct SoftmaxState {
    f32x4 acc[D / 16];
    float run_max;
    float run_sum;
};

// Smallest positive normal fp32 value.  A split partial may hold an infinity
// (bf16 V); the reduce never weights it by an underflowed 0 (0 * Inf = NaN):
// a weight below this is raised to it, which changes a finite result by less
// than 2^-126 of that partial.
constexpr float kMinNormal = 0x1p-126f;

// One 32-token step of one wave: S^T = K Q^T, online softmax, O^T += V^T P^T.
// E4M3 K codes become bf16 exactly; bf16 K words are the operand as they are.
// E4M3 V codes become f16 exactly, with P as a sum of two f16 terms; bf16 V
// uses the bf16 product with P as a sum of two bf16 terms.
template <int D, int KB, int VB>
__device__ __forceinline__ void compute_step(SoftmaxState<D> &st, StepRegs<D, KB, VB> &cur, const bf16x8 *qb,
                                             int p, int c1, int m, int g, float qk_scale, int *vflags) {
    constexpr int KK = D / 32;
    constexpr int MT = D / 16;
    using R = StepRegs<D, KB, VB>;
    // ---- S^T = K Q^T for the two tiles
    f32x4 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            bf16x8 ka;
            if constexpr (KB == 1) {
                const uint32_t w0 = cur.kw(t, 2 * kk), w1 = cur.kw(t, 2 * kk + 1);
                const bf16x2 e0 = codes_to_bf16x2<false>(w0), e1 = codes_to_bf16x2<true>(w0);
                const bf16x2 e2 = codes_to_bf16x2<false>(w1), e3 = codes_to_bf16x2<true>(w1);
                ka = bf16x8{e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
            } else {
                ka = __builtin_bit_cast(bf16x8, cur.k[t][kk]);
            }
            s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[kk], s[t], 0, 0, 0);
        }
    }

    // ---- scale into the log2 domain; only the last step of a chunk has tokens to mask
    const bool tail = p + kStep > c1;      // the same for the whole wave
    float x[8];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[4 * t + i] = s[t][i] * qk_scale;
    if (tail) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (p + 16 * t + 4 * g + i >= c1) x[4 * t + i] = -__builtin_inff();
    }
    float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // Lazy rescale: probabilities are taken relative to a per-head reference
    // that only moves when a score exceeds it by more than 2^kLazy, so P stays
    // <= 2^kLazy (well inside f16) and the accumulators are rescaled rarely.
    // The result is unchanged: the final normalization uses the same reference.
    if (__any(mx > st.run_max + kLazy)) {
        const float new_ref = fmaxf(st.run_max, mx);
        const float alpha = __builtin_amdgcn_exp2f(st.run_max - new_ref);   // 0 on the first step
        st.run_sum *= alpha;
#pragma unroll
        for (int j = 0; j < MT; ++j) st.acc[j] *= alpha;
        st.run_max = new_ref;
    }
    float pr[8];
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        pr[i] = __builtin_amdgcn_exp2f(x[i] - st.run_max);
        psum += pr[i];
    }
    st.run_sum += psum;

    // ---- tail: values of tokens past the end must not reach the product (NaN * 0)
    if (tail) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int valid = c1 - (p + 16 * t + 4 * g);          // tokens of this lane's group left
            if constexpr (VB == 1) {
                const uint32_t keep = valid >= 4 ? 0xFFFFFFFFu : valid <= 0 ? 0u : (0xFFFFFFFFu >> (32 - 8 * valid));
#pragma unroll
                for (int i = 0; i < R::NV; ++i) cur.v[t][i] &= keep;
            } else {
                // each dim's four tokens are two words: tokens (0, 1) and (2, 3)
                const uint32_t keep0 = (valid > 0 ? 0x0000FFFFu : 0u) | (valid > 1 ? 0xFFFF0000u : 0u);
                const uint32_t keep1 = (valid > 2 ? 0x0000FFFFu : 0u) | (valid > 3 ? 0xFFFF0000u : 0u);
                const u32x4 keep = {keep0, keep1, keep0, keep1};
#pragma unroll
                for (int i = 0; i < R::NV; ++i) cur.v[t][i] &= keep;
            }
        }
    }

    // ---- O^T += V^T P^T
    if constexpr (VB == 1) {
        // P as two f16 terms, hi = f16(P) and lo = f16(P - hi), about 22
        // significant bits: one f16 term (11 bits) leaves an error of up to
        // 2^-12 |V| per output, 2.5e-3 with the outlier channels of the
        // Llama-shaped workload.  The extra products are free in this
        // HBM-bound loop.
        f16x8 ph, pl;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            ph[i] = (_Float16)pr[i];
            pl[i] = (_Float16)(pr[i] - (float)ph[i]);
        }
#pragma unroll
        for (int j = 0; j < MT; ++j) {
            const f16x2 e0 = codes_to_f16x2<false>(cur.vw(0, j)), e1 = codes_to_f16x2<true>(cur.vw(0, j));
            const f16x2 e2 = codes_to_f16x2<false>(cur.vw(1, j)), e3 = codes_to_f16x2<true>(cur.vw(1, j));
            const f16x8 va = {e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
            st.acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, ph, st.acc[j], 0, 0, 0);
            st.acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pl, st.acc[j], 0, 0, 0);
        }
    } else {
        // Non-finite bf16 V values.  The definition sums p_t V_t with p_t > 0
        // for every token of the sequence, so a token holding +-Inf makes that
        // output dim an infinity of its sign (NaN with both signs) and a NaN
        // makes it NaN, whatever the token's probability.  In the product a P
        // term that is 0 (an exactly representable P has lo = 0; a tiny P
        // underflows) would turn an infinity into NaN instead.  So such values
        // are taken out of the product (zeroed) and their classes are ORed
        // into this wave's per-dim flags, which the combine adds back.  Tokens
        // past the chunk were zeroed above; every other token of the step is
        // seen by every head.
        uint32_t nf = 0;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < R::NV; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) nf |= bf16_nonfinite_halves(cur.v[t][i][e]);
        if (__any(nf != 0u)) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < R::NV; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t w = cur.v[t][i][e];
                        const uint32_t n = bf16_nonfinite_halves(w);
                        if (!n) continue;
                        // word 4i + e holds two tokens of dim (D/16)m + 2i + e/2
                        atomicOr(&vflags[(D / 16) * m + 2 * i + (e >> 1)], bf16_class_bits(w, n));
                        cur.v[t][i][e] = w & ~((n >> 15) * 0xFFFFu);
                    }
        }
        // P as two bf16 terms, hi = bf16(P) and lo = bf16(P - hi): about 16
        // significant bits, as precise as one f16 term (a single bf16 P keeps
        // 8).  The extra products are free in this HBM-bound loop.
        bf16x8 ph, pl;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            ph[i] = (__bf16)pr[i];
            pl[i] = (__bf16)(pr[i] - (float)ph[i]);
        }
        // dim j's four tokens are words 2j, 2j+1 of each tile: half of vector j/2
#pragma unroll
        for (int j = 0; j < MT; j += 2) {
            const u32x4 a = cur.v[0][j >> 1], b = cur.v[1][j >> 1];
            const bf16x8 v0 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 4, 5));
            const bf16x8 v1 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 2, 3, 6, 7));
            st.acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v0, ph, st.acc[j], 0, 0, 0);
            st.acc[j + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v1, ph, st.acc[j + 1], 0, 0, 0);
            st.acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v0, pl, st.acc[j], 0, 0, 0);
            st.acc[j + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v1, pl, st.acc[j + 1], 0, 0, 0);
        }
    }
}

// Register buffers in flight per wave: the step being computed plus
// (NBUF - 1) steps whose loads are outstanding.
// Three steps when one step's registers fit in 32 VGPRs, else two.
template <int D, int KB, int VB>
struct Depth { static constexpr int NBUF = 8 * (StepRegs<D, KB, VB>::NK + StepRegs<D, KB, VB>::NV) <= 32 ? 3 : 2; };

// Workgroups are handed to the 8 XCDs round-robin by linear id, and each XCD
// has its own CUs and L2.  Unit (pair p = seq * kv_heads + kv_head, split s)
// runs as linear id h with h % 8 == (p + s) % 8: the splits of one pair rotate
// over the XCDs and neighbouring pairs interleave, so every XCD receives an
// even share of the work whatever the sequence lengths and the split count
// (with the plain (split, head, seq) grid and 8 splits, every first chunk
// landed on one XCD).  Ids run split-major; pairs are padded to a multiple of
// 8 and padding units exit at once.
__device__ __forceinline__ bool decode_unit(uint32_t h, const DecodeArgs &a, int &pair, int &split) {
    const int pairs = a.num_seqs * a.kv_heads;
    const uint32_t per = (uint32_t)((pairs + 7) >> 3);
    const uint32_t k = h >> 3;
    split = (int)(k / per);
    pair = (((int)(h & 7) - split) & 7) + 8 * (int)(k % per);
    return pair < pairs;
}

template <int D, int BS, int KB, int VB>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
    constexpr int KK = D / 32;     // QK^T instructions per tile
    constexpr int MT = D / 16;     // PV instructions per step (one per 16 dims)
    constexpr int NBUF = Depth<D, KB, VB>::NBUF;
    static_assert(NBUF == 2 || NBUF == 3, "the ring tail below handles up to two remaining steps");
    using Regs = StepRegs<D, KB, VB>;

    // [waves][G] max, [waves][G] sum, [waves][G][D] acc; with a bf16 V pool
    // then [waves][D] flags of the non-finite values taken out of the product
    extern __shared__ float smem[];

    int pair, split;
    if (!decode_unit(blockIdx.x, a, pair, split)) return;   // padding unit
    const int kvh = pair % a.kv_heads;
    const int b = pair / a.kv_heads;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int m = lane & 15;        // MFMA row/column index of this lane
    const int g = lane >> 4;        // k-group of this lane
    const int G = a.q_heads / a.kv_heads;
    const int L = min(a.seq_lens[b], a.max_blocks * BS);   // never past the table row
    const int c0 = split * a.chunk_tokens;
    const int c1 = min(L, c0 + a.chunk_tokens);
    const uint32_t last_block = (uint32_t)(a.num_blocks - 1);

    float *s_max = smem;
    float *s_sum = smem + kWaves * G;
    float *s_acc = smem + 2 * kWaves * G;
    int *s_flags = reinterpret_cast<int *>(smem + kWaves * G * (2 + D));
    int *vflags = s_flags + wave * D;
    if constexpr (VB == 2) {
        for (int d = lane; d < D; d += 64) vflags[d] = 0;
    }

    if (c0 >= c1) {
        if (a.splits == 1) {      // empty sequence: zero output
            for (int idx = threadIdx.x; idx < G * D; idx += kThreads)
                store_out(a.out, ((int64_t)b * a.q_heads + kvh * G) * D + idx, 0.0f, a.out_bf16);
        }
        return;
    }

    // Q^T as the B operand: lane (n, g) holds head n, dims g*D/4 + 8kk .. +7 for instruction kk.
    bf16x8 qb[KK];
    {
        const int n = m;
        const uint16_t *qrow = a.q + ((int64_t)b * a.q_heads + kvh * G + n) * D + g * (D / 4);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            uint4 w = make_uint4(0, 0, 0, 0);
            if (n < G) w = *reinterpret_cast<const uint4 *>(qrow + 8 * kk);
            qb[kk] = __builtin_bit_cast(bf16x8, w);
        }
    }

    // Block ids of this wave's tiles, one per lane: tile j of the wave is step
    // j/2, half j%2, at position c0 + 32*wave + 128*(j/2) + 16*(j%2).  A chunk
    // holds at most 32 steps per wave, so 64 lanes cover it.  Positions past
    // the sequence read its last block (never used unmasked).
    const int32_t *table = a.block_tables + (int64_t)b * a.max_blocks;
    uint32_t ids;
    {
        const int pos = c0 + kStep * wave + kStep * kWaves * (lane >> 1) + 16 * (lane & 1);
        const int e = min(pos, L - 1) / BS;
        ids = min((uint32_t)table[e], last_block);   // an id outside the pool is clamped
    }
    // Q and the ids must have landed before the load ring starts, so that the
    // waits inside the ring only count ring loads.
    __builtin_amdgcn_s_waitcnt(0);

    SoftmaxState<D> st;
#pragma unroll
    for (int j = 0; j < MT; ++j) st.acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.run_max = -__builtin_inff();
    st.run_sum = 0.0f;

    const int stride = kStep * kWaves;
    const int nsteps = c1 > c0 + kStep * wave ? (c1 - c0 - kStep * wave + stride - 1) / stride : 0;
    const int p0 = c0 + kStep * wave;
    constexpr int LOADS = 2 * (Regs::NK + Regs::NV);   // loads per step
    // this lane's fixed byte offsets inside a K tile half and a V tile half
    const uint32_t koff = (uint32_t)((g * BS + m) * (D / 4) * KB);
    const uint32_t voff = (uint32_t)((g * D + (D / 16) * m) * 4 * VB);
    auto issue = [&](Regs &r, int i) {
        const bool live = i < nsteps;
        const int ii = live ? i : 0;
        const uint32_t b0 = __builtin_amdgcn_readlane(ids, 2 * ii);
        const uint32_t b1 = __builtin_amdgcn_readlane(ids, 2 * ii + 1);
        load_step<D, BS, KB, VB>(r, a.k_pool, a.v_pool, b0, b1, a.kv_heads, kvh, p0 + ii * stride, koff, voff, live);
    };
    Regs buf[NBUF];
    // Unconditional, so that every path into the loop holds the same loads in
    // flight (a wave with no steps issues dummy loads of one valid line).
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i) issue(buf[i], i);
    // Full rounds of NBUF steps, then the remaining steps (fewer than NBUF)
    // in nested branches: the loop has one exit, and a skipped step skips
    // every later one, so each path through the code is one the ring can take.
    auto step_at = [&](int step, int u) {
        // keep the next NBUF-1 steps' loads in flight while this one computes
        issue(buf[(u + NBUF - 1) % NBUF], step + NBUF - 1);
        wait_step<LOADS * (NBUF - 1)>(buf[u]);
        compute_step<D, KB, VB>(st, buf[u], qb, p0 + step * stride, c1, m, g, a.qk_scale, vflags);
    };
    const int full = nsteps - nsteps % NBUF;
    for (int i = 0; i < full; i += NBUF) {
#pragma unroll
        for (int u = 0; u < NBUF; ++u) step_at(i + u, u);
    }
    const int rest = nsteps - full;
    if (rest > 0) {
        step_at(full, 0);
        if constexpr (NBUF > 2) {
            if (rest > 1) step_at(full + 1, 1);
        }
    }
    // Drain the ring.  The wait names every ring register, so none of them can
    // be reused for anything else while a (possibly dummy) load into it is still
    // in flight.
#pragma unroll
    for (int u = 0; u < NBUF; ++u) wait_step<0>(buf[u]);
    f32x4 *acc = st.acc;
    float run_max = st.run_max;
    float run_sum = st.run_sum;

    // ---- combine the four waves
    run_sum += __shfl_xor(run_sum, 16);
    run_sum += __shfl_xor(run_sum, 32);
    const int n = m;
    if (n < G) {
        if (g == 0) {
            s_max[wave * G + n] = run_max;
            s_sum[wave * G + n] = run_sum;
        }
        float *dst = s_acc + ((int64_t)wave * G + n) * D;
#pragma unroll
        for (int j = 0; j < MT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(D / 16) * (4 * g + r) + j] = acc[j][r];
    }
    __syncthreads();

    for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
        const int hn = idx / D;
        const int d = idx - hn * D;
        float M = -__builtin_inff();
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_max[w * G + hn]);
        float num = 0.0f, den = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = s_max[w * G + hn];
            const float f = mw == -__builtin_inff() ? 0.0f : exp2f(mw - M);
            num += f * s_acc[((int64_t)w * G + hn) * D + d];
            den += f * s_sum[w * G + hn];
        }
        if constexpr (VB == 2) {
            uint32_t c = 0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) c |= (uint32_t)s_flags[w * D + d];
            num += nonfinite_from_bits(c);
        }
        const int head = kvh * G + hn;
        if (a.splits == 1) {
            store_out(a.out, ((int64_t)b * a.q_heads + head) * D + d, num * a.v_scale / den, a.out_bf16);
        } else {
            float *part = a.partials + (((int64_t)b * a.q_heads + head) * a.splits + split) * (D + 2);
            if (d == 0) {
                part[0] = M;
                part[1] = den;
            }
            part[2 + d] = num;
        }
    }
}

// Combine split partials: o = v_scale * sum_i acc_i 2^(m_i - M) / sum_i l_i 2^(m_i - M).
// The split maxima and weights are computed one split per thread and staged in
// LDS; each output dim then sums its partials with independent loads.
template <int D>
__global__ __launch_bounds__(D) void decode_reduce(DecodeArgs a) {
    constexpr int kBatch = D;            // splits weighted per pass
    __shared__ float s_w[kBatch];
    __shared__ float s_red[D / 64];
    const int head = blockIdx.x;
    const int b = blockIdx.y;
    const int t = threadIdx.x;
    const int L = a.seq_lens[b];   // clamped the same way as in decode_kernel
    const int Lc = min(L, a.max_blocks * a.block_size);
    const int nsplit = Lc <= 0 ? 0 : min(a.splits, (Lc + a.chunk_tokens - 1) / a.chunk_tokens);
    const float *part = a.partials + ((int64_t)b * a.q_heads + head) * a.splits * (D + 2);

    float m = -__builtin_inff();
    for (int i = t; i < nsplit; i += D) m = fmaxf(m, part[(int64_t)i * (D + 2)]);
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((t & 63) == 0) s_red[t >> 6] = m;
    __syncthreads();
    float M = s_red[0];
#pragma unroll
    for (int w = 1; w < D / 64; ++w) M = fmaxf(M, s_red[w]);

    float num = 0.0f, den = 0.0f;
    for (int i0 = 0; i0 < nsplit; i0 += kBatch) {
        const int n = min(kBatch, nsplit - i0);
        __syncthreads();                 // s_red / previous batch consumed
        if (t < n) {
            const float *p = part + (int64_t)(i0 + t) * (D + 2);
            const float mi = p[0];
            // raised to the smallest normal, so that a partial holding an
            // infinity (bf16 V) is never multiplied by 0
            s_w[t] = mi == -__builtin_inff() ? 0.0f : fmaxf(exp2f(mi - M), kMinNormal);
        }
        __syncthreads();
        const float *p = part + (int64_t)i0 * (D + 2);
        int i = 0;
        for (; i + 8 <= n; i += 8) {
            float x[8], l[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                x[u] = p[(int64_t)(i + u) * (D + 2) + 2 + t];
                l[u] = p[(int64_t)(i + u) * (D + 2) + 1];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                num += s_w[i + u] * x[u];
                den += s_w[i + u] * l[u];
            }
        }
        for (; i < n; ++i) {
            num += s_w[i] * p[(int64_t)i * (D + 2) + 2 + t];
            den += s_w[i] * p[(int64_t)i * (D + 2) + 1];
        }
    }
    const float o = nsplit > 0 ? num * a.v_scale / den : 0.0f;
    store_out(a.out, ((int64_t)b * a.q_heads + head) * D + t, o, a.out_bf16);
}

template <int D, int BS, int KB, int VB>
hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t stream) {
    const int G = a.q_heads / a.kv_heads;
    const size_t smem = sizeof(float) * (size_t)kWaves * G * (2 + D) + (VB == 2 ? sizeof(int) * kWaves * D : 0);
    const uint32_t units = (uint32_t)a.splits * (uint32_t)(((a.num_seqs * a.kv_heads + 7) >> 3) << 3);
    hipLaunchKernelGGL((decode_kernel<D, BS, KB, VB>), dim3(units), dim3(kThreads), smem, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    hipLaunchKernelGGL((decode_reduce<D>), dim3(a.q_heads, a.num_seqs), dim3(D), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

// Chunking: at most `max_chunk` tokens per workgroup (bounds the tail of
// long sequences), and enough workgroups to give every CU two; chunks are a
// multiple of one round of wave steps.
void decode_plan(int32_t num_seqs, int32_t kv_heads, int32_t head_dim, int32_t block_size,
                 int32_t max_seq_len, int32_t *splits, int32_t *chunk_tokens) {
    // a wave holds the block ids of at most 64 tiles (32 steps): chunk <= 4096 tokens
    // (2048-token chunks and 1024 or 2048 target workgroups measured no faster)
    constexpr int max_chunk = 32 * kStep * kWaves;
    constexpr int target_wgs = 512;
    const int round = kStep * kWaves;
    const int64_t pairs = (int64_t)num_seqs * kv_heads;
    int64_t s = (max_seq_len + max_chunk - 1) / max_chunk;
    const int64_t want = (target_wgs + pairs - 1) / pairs;
    if (want > s) s = want;
    const int64_t cap = (max_seq_len + round - 1) / round;   // never below one round per chunk
    if (s > cap) s = cap;
    if (s < 1) s = 1;
    int64_t chunk = (max_seq_len + s - 1) / s;
    chunk = ((chunk + round - 1) / round) * round;
    if (chunk < round) chunk = round;
    if (chunk > max_chunk) chunk = max_chunk;
    s = (max_seq_len + chunk - 1) / chunk;
    if (s < 1) s = 1;
    *splits = (int32_t)s;
    *chunk_tokens = (int32_t)chunk;
    (void)head_dim;
    (void)block_size;
}

namespace {

template <int D, int BS>
hipError_t launch_decode_types(const DecodeArgs &a, hipStream_t stream) {
    if (a.k_eb == 1 && a.v_eb == 1) return launch_decode_t<D, BS, 1, 1>(a, stream);
    if constexpr (D <= 128) {     // bf16 pools: head_dim 64 and 128
        if (a.k_eb == 1) return launch_decode_t<D, BS, 1, 2>(a, stream);
        if (a.v_eb == 1) return launch_decode_t<D, BS, 2, 1>(a, stream);
        return launch_decode_t<D, BS, 2, 2>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
    if (a.block_size == 16) {
        if (a.head_dim == 64) return launch_decode_types<64, 16>(a, stream);
        if (a.head_dim == 128) return launch_decode_types<128, 16>(a, stream);
        if (a.head_dim == 256) return launch_decode_types<256, 16>(a, stream);
    } else if (a.block_size == 32) {
        if (a.head_dim == 64) return launch_decode_types<64, 32>(a, stream);
        if (a.head_dim == 128) return launch_decode_types<128, 32>(a, stream);
        if (a.head_dim == 256) return launch_decode_types<256, 32>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace kvf8
