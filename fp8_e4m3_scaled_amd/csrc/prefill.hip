// paged_attn_prefill_chunk: causal attention of a chunk of new query tokens
// over an E4M3 paged cache that already holds the chunk's own K/V.
//
// [P1, tests/test-fp8.cpp check_fp8_attention: query token i at position
// ctx+i attends to positions <= ctx+i; build_attn stores K/V first and reads
// the cache views; build_attn_scale_kv_inputs/_output move the scales out of
// the products.]  As in the decode, s = (q . K_codes) * k_scale * sm_scale,
// o = v_scale * softmax(s) V_codes.
//
// Work decomposition.  A 1-D grid of (query tile, kv-head, sequence) units,
// a pair's tiles placed on one XCD.  A "row" is one (query token, head of the
// kv-head's group) pair; row r of a tile is token r / G, head r % G, so the G
// heads that share a kv-head share every K/V tile.  A workgroup of four waves
// owns 128 rows (two 16-row MFMA tiles per wave) and walks the keys 0 .. last
// row's position in 32-token steps:
//   * each step's K and V tiles (already in MFMA operand order in the cache)
//     go from HBM straight into one of four LDS stages, three steps ahead,
//     and are read from LDS by all four waves;
//   * S^T[key][row] = K Q^T on the fp8 MFMA with the K codes as stored and Q
//     split exactly into two E4M3 terms (below); its output is the B operand
//     of O^T[d][row] += V^T P^T on v_mfma_f32_16x16x32_f16;
//   * online softmax per row in the log2 domain with the same lazy reference
//     as the decode, P = exp2(fma(s, |qk|, -max)) from the raw MFMA scores;
//     causal masking only on steps that reach the tile's first query
//     position.

#include "fp8_device.hpp"
#include "internal.hpp"

namespace kvf8 {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
static_assert(kThreads == kPrefillThreads, "host launch checks assume this workgroup size");
constexpr int kStep = 32;              // keys per step (two 16-key tiles)
constexpr int kNR = 2;                 // 16-row MFMA tiles per wave
constexpr int kRows = kWaves * kNR * 16;
static_assert(kRows == kPrefillRows, "host launch checks assume this tile height");
constexpr float kLazy = 8.0f;
constexpr float kNoMax = -1.0e30f;
constexpr int kUnitScale = 127;          // E8M0 exponent of 1.0 for the scaled fp8 MFMA
constexpr int kLoScale = 127 - 5;        // E8M0 exponent of 2^-5: Q's lo term is stored times 32

typedef __attribute__((ext_vector_type(8))) int v8i;
typedef __attribute__((ext_vector_type(2))) unsigned short u16x2;

template <bool B>
struct Flag { static constexpr bool value = B; };     // running-max sentinel (finite: see the accumulators)

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Bytes of one step in LDS: K tile 0, K tile 1 (16*D elements of KB bytes
// each), V tile 0, V tile 1 (16*D elements of VB bytes).  KB, VB: 1 for E4M3
// codes, 2 for bf16 values.
template <int D, int KB, int VB>
struct StepLds {
    static constexpr int KTILE = 16 * D * KB;
    static constexpr int VTILE = 16 * D * VB;
    static constexpr int BYTES = 2 * (KTILE + VTILE);
};

// LDS image swizzle.  A lane reads PP consecutive 16-byte pieces of its key
// (K) or key group (V) at a stride of PP pieces between neighbouring lanes, so
// lanes m and m + 16/PP would hit the same banks.  Inside every aligned group
// of 16 pieces the image stores piece q at position q ^ ((q >> 4) & (PP - 1))
// (a permutation of the group, its own inverse): a lane's pieces then start
// at a lane-dependent rotation and the reads spread over all banks.  The copy
// fetches the same 16-piece groups, so every copy instruction still reads the
// same contiguous global bytes, only in another lane order.
template <int D, int EB>
struct Swz {
    static constexpr int PP = D * EB / 64;              // 16-byte pieces per lane per tile
    static __device__ __forceinline__ int pos(int q) { return PP > 1 ? q ^ ((q >> 4) & (PP - 1)) : q; }
};

// Per-thread share of one step's global->LDS copy: 16-byte chunks, rounded up
// (a lane without a last chunk repeats its previous one, so that every lane
// issues the same number of loads and the vmcnt arithmetic holds).
template <int D, int KB, int VB>
struct CopyShare {
    static constexpr int TOTAL = StepLds<D, KB, VB>::BYTES / 16;
    static constexpr int CHUNKS = (TOTAL + kThreads - 1) / kThreads;
    static_assert(TOTAL % 64 == 0, "whole waves per chunk round");
};

// K/V steps in LDS: the one being computed and kStages-1 in flight.
constexpr int kStages = 4;

// A uniform-index read of read-only memory through the constant address
// space, so that it becomes a scalar load.
__device__ __forceinline__ int32_t load_uniform(const int32_t *p, int i) {
    return ((const __attribute__((address_space(4))) int32_t *)p)[i];
}

// 16 bytes per lane from global memory straight into LDS
// (global_load_lds_dwordx4): lane i writes bytes [16i, 16i+16) of the
// wave-uniform destination.  Counted by vmcnt like any load.
__device__ __forceinline__ void load_to_lds16(const void *src, uint8_t *wave_dst) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)wave_dst, 16, 0, 0);
}

// Maximum of raw scores with the NaN-propagating v_maximum(3)_f32: fmaxf in
// IEEE mode first quiets each operand that is not known to be canonical (every
// MFMA result and every lane-swapped value), one extra VALU op per value.  A
// NaN score makes its row's maximum NaN, which only keeps that step from
// moving the reference (a NaN comparison is false); the row's output is NaN
// either way, through that key's probability.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// max(v, v of lane ^ 16) and max(v, v of lane ^ 32) with the gfx950 row
// swaps (full-rate VALU, no LDS round trip): with both operands the same
// register, each lane gets back its own value and its partner's.
__device__ __forceinline__ float max_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Wait until at most N of this wave's vector-memory loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Chunk c of a step (16 bytes of the step's LDS image): tile kind (K/V),
// 16-key tile t, element offset.  K tile t: 4 quarters of 16 keys x D/4
// elements; in the cache quarter q of the tile's block starts at element
// (q*BS + tb)*(D/4) with tb the tile's first in-block key.  V tile t: 4 groups
// of 4 keys, contiguous from element (tb/4)*D*4.
template <int D, int BS, int KB, int VB>
__device__ __forceinline__ const uint8_t *chunk_src(int c, const uint8_t *k_pool, const uint8_t *v_pool,
                                                    uint32_t blk0, uint32_t blk1, int kv_heads, int kvh,
                                                    int p) {
    constexpr int Q4 = D / 4;
    constexpr int KPT = StepLds<D, KB, VB>::KTILE / 16;   // chunks per K tile
    constexpr int VPT = StepLds<D, KB, VB>::VTILE / 16;
    const bool is_k = c < 2 * KPT;
    const int cc = is_k ? c : c - 2 * KPT;
    const int t = is_k ? cc / KPT : cc / VPT;
    const uint32_t blk = t == 0 ? blk0 : blk1;
    const int tb = (p + 16 * t) % BS;
    const int64_t base = ((int64_t)blk * kv_heads + kvh) * (BS * D);   // elements
    if (is_k) {
        const int e = (cc % KPT) * 16 / KB;                   // element inside the tile image
        const int q = e / (16 * Q4);
        const int rem = e - q * 16 * Q4;
        return k_pool + (base + (int64_t)(q * BS + tb) * Q4 + rem) * KB;
    }
    const int e = (cc % VPT) * 16 / VB;
    return v_pool + (base + (int64_t)(tb / 4) * D * 4 + e) * VB;
}

// Three waves per SIMD with an E4M3 V pool and head dims up to 128 (a budget
// of 168 VGPRs; the main loop does not spill, with E4M3 or bf16 K); two with a
// bf16 V pool (the two-term P and wider operands need more registers).
template <int D, int KB, int VB>
struct Occupancy { static constexpr int WAVES = D > 128 ? 1 : (VB == 1 ? 3 : 2); };

template <int D, int BS, int KB, int VB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Occupancy<D, KB, VB>::WAVES)))
void prefill_kernel(PrefillArgs a) {
    constexpr int NC = D >= 128 ? D / 128 : 1;   // 128-dim K chunks per tile (D = 64: one, zero-padded)
    constexpr int KK = D / 32;                   // bf16 K: 16x16x32 products per tile
    constexpr int MT = D / 16;
    constexpr int Q4 = D / 4;
    constexpr int NW = D / 16;                   // 32-bit V words per tile and lane (E4M3; twice for bf16)
    constexpr int KTILE = StepLds<D, KB, VB>::KTILE;
    constexpr int VTILE = StepLds<D, KB, VB>::VTILE;
    constexpr int CH = CopyShare<D, KB, VB>::CHUNKS;
    constexpr int TOTAL = CopyShare<D, KB, VB>::TOTAL;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kStages][StepLds<D, KB, VB>::BYTES];

    // Workgroups go to the 8 XCDs round-robin by linear id; every query tile
    // of pair p = seq * kv_heads + kv_head runs on XCD p % 8, the pair's tiles
    // dispatched together, so one XCD's L2 serves all reads of the pair's K/V
    // while its tiles walk the keys side by side.  Pairs are padded to a
    // multiple of 8; padding ids exit at once.
    const uint32_t hid = blockIdx.x;
    const uint32_t kx = hid >> 3;
    const int pair = (int)(kx / (uint32_t)a.q_tiles) * 8 + (int)(hid & 7);
    // a pair's tiles go out longest first (the last query tile sees the most
    // keys), so the shorter ones fill in behind them at the end of the grid
    const int qt = a.q_tiles - 1 - (int)(kx % (uint32_t)a.q_tiles);
    if (pair >= a.num_seqs * a.kv_heads) return;
    const int kvh = pair % a.kv_heads;
    const int b = pair / a.kv_heads;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int m = lane & 15;
    const int g = lane >> 4;
    const int G = a.q_heads / a.kv_heads;
    const int q0 = a.cu_q_lens[b];
    const int q_len = a.cu_q_lens[b + 1] - q0;
    const int ctx = a.context_lens[b];
    const int tok_per_tile = kRows / G;
    const int i0 = qt * tok_per_tile;               // first query token of this tile
    if (i0 >= q_len) return;
    const int total = min(ctx + q_len, a.max_blocks * BS);
    const int kend = min(ctx + min(i0 + tok_per_tile, q_len), total);   // keys this tile needs
    const int nsteps = (kend + kStep - 1) / kStep;
    const uint32_t last_block = (uint32_t)(a.num_blocks - 1);
    const int32_t *table = a.block_tables + (int64_t)b * a.max_blocks;

    // ---- Q^T operands of this wave's two row tiles; lane (n, g) holds quarter
    // g of row n's dims (byte e = dim g*D/4 + e, the K tile's order).
    //
    // S^T = K Q^T runs on the fp8 MFMA with the K codes as they are in the
    // cache.  Q is split into two E4M3 terms per row: with 2^e the power of
    // two that puts the row's max |q| in [128, 256),
    //   y = q * 2^e,  hi = E4M3(y),  lo = E4M3(32 (y - hi)),
    // and the lo product runs with the MFMA's block scale 2^-5, so the
    // score is K.(hi + lo/32).  |y - hi| <= 8 (half a step of E4M3 at
    // [128, 256)), so 32 (y - hi) <= 256 never saturates; a bf16 significand
    // has 8 bits, E4M3 keeps 4, and the remainder of the round-to-nearest is
    // a 4-bit multiple of y's last place, so hi + lo/32 == y for every
    // element with |y| >= 2^-7 (within 2^-15 of the row max); smaller
    // elements are off by at most 2^-15, i.e. 2^-22 of the row max.  So
    // K.(hi + lo/32) = 2^e (K.q) to fp32 accumulation, and 2^-e goes into the
    // row's exp2 factor.  e is capped so that 2^e and the row factor
    // qk 2^-e stay normal fp32 numbers: a row whose max |q| is below 2^-119
    // (bf16 subnormals) gets y below 2^7 and scores of no weight, as the
    // definition's scores are then below 1e-30.  A negative qk_scale flips
    // the sign of y (exact).
    //
    // With a bf16 K pool the product runs on the bf16 MFMA instead, with Q as
    // given (sign folded in, exact) and no 2^e.
    const float qk = fabsf(a.qk_scale);
    const float qsgn = a.qk_scale < 0.0f ? -1.0f : 1.0f;
    v8i qh[kNR][KB == 1 ? NC : 1], ql[kNR][KB == 1 ? NC : 1];
    bf16x8 qb[kNR][KB == 2 ? KK : 1];
    float qk_row[kNR];
    int row_pos[kNR];          // causal limit of lane-row n in tile j (key <= row_pos)
    bool row_live[kNR];
#pragma unroll
    for (int j = 0; j < kNR; ++j) {
        const int r = (wave * kNR + j) * 16 + m;
        const int tok = i0 + r / G;
        const int head = kvh * G + r % G;
        // rows past tok_per_tile*G (when G does not divide the tile) belong to no token of this tile
        row_live[j] = r < tok_per_tile * G && tok < q_len;
        row_pos[j] = ctx + tok;
        const uint16_t *qrow = a.q + ((int64_t)(q0 + (row_live[j] ? tok : 0)) * a.q_heads + head) * D + g * (D / 4);
        float y[D / 4];
        float amax = 0.0f;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            uint4 w = make_uint4(0, 0, 0, 0);
            if (row_live[j]) w = *reinterpret_cast<const uint4 *>(qrow + 8 * kk);
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                y[8 * kk + 2 * e] = __uint_as_float(ww[e] << 16);
                y[8 * kk + 2 * e + 1] = __uint_as_float(ww[e] & 0xFFFF0000u);
            }
        }
        int bad = 0;                        // a NaN or infinite element in the row
#pragma unroll
        for (int i = 0; i < D / 4; ++i) {
            amax = fmaxf(amax, fabsf(y[i]));
            bad |= !__builtin_isfinite(y[i]);
        }
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        bad |= __shfl_xor(bad, 16);
        bad |= __shfl_xor(bad, 32);
        if constexpr (KB == 2) {
            qk_row[j] = qk;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    qb[j][kk][e] = bad ? (__bf16)__builtin_nanf("") : (__bf16)(y[8 * kk + e] * qsgn);   // exact
        } else {
            int ex = 0;
            if (!bad && amax > 0.0f) {
                int E, Eq;
                (void)frexpf(amax, &E);         // amax = f * 2^E, f in [0.5, 1)
                (void)frexpf(qk, &Eq);          // qk >= 2^(Eq - 1)
                ex = min(8 - E, min(126, Eq + 125));
            }
            qk_row[j] = ldexpf(qk, -ex);
            const float mul = ldexpf(qsgn, ex);
            uint32_t hw[D / 16], lw[D / 16];
#pragma unroll
            for (int i = 0; i < D / 16; ++i) {
                float v[4], hv[4], rv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = y[4 * i + e] * mul;     // exact: a power of two
                int h = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
                h = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], h, true);
                const f32x2 b01 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false);
                const f32x2 b23 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
                hv[0] = b01[0]; hv[1] = b01[1]; hv[2] = b23[0]; hv[3] = b23[1];
#pragma unroll
                for (int e = 0; e < 4; ++e) rv[e] = (v[e] - hv[e]) * 32.0f;  // exact, |.| <= 256
                int l = __builtin_amdgcn_cvt_pk_fp8_f32(rv[0], rv[1], 0, false);
                l = __builtin_amdgcn_cvt_pk_fp8_f32(rv[2], rv[3], l, true);
                hw[i] = (uint32_t)h;
                lw[i] = (uint32_t)l;
            }
            if (bad) {                          // a non-finite q makes the whole row NaN
#pragma unroll
                for (int i = 0; i < D / 16; ++i) hw[i] = 0x7F7F7F7Fu;
            }
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int wi = 8 * c + i;
                    qh[j][c][i] = wi < D / 16 ? (int)hw[wi < D / 16 ? wi : 0] : 0;
                    ql[j][c][i] = wi < D / 16 ? (int)lw[wi < D / 16 ? wi : 0] : 0;
                }
        }
    }

    // run_max starts at a finite sentinel far below any score, so that
    // exp2(s*qk - run_max) of a masked score (-inf) is 0 without a select and
    // the first rescale factor exp2(sentinel - ref) is 0.  With E4M3 V the
    // row sums come from the matrix cores: one more product per row tile and
    // step, of an all-ones operand with the same f16 P as the P.V product, so
    // every element of rsum[j] holds the whole row's sum of the P it used.
    // With bf16 V, run_sum holds this lane's share of the row sum (its four
    // k-groups are added at the end).
    f32x4 acc[kNR][MT];
    f32x4 rsum[kNR];
    float run_sum[kNR];
    float run_max[kNR];
    auto reset = [&]() {
#pragma unroll
        for (int j = 0; j < kNR; ++j) {
#pragma unroll
            for (int t = 0; t < MT; ++t) acc[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
            rsum[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            run_sum[j] = 0.0f;
            run_max[j] = kNoMax;
        }
    };
    reset();

    // Block ids come through the constant address space: the index is uniform,
    // so these are scalar loads (lgkmcnt), not vector loads that would make
    // the compiler wait for the in-flight LDS transfers.
    auto blocks_of = [&](int p, uint32_t &b0, uint32_t &b1) {
        const int e0 = __builtin_amdgcn_readfirstlane(min(p, total - 1) / BS);
        const int e1 = __builtin_amdgcn_readfirstlane(min(p + 16, total - 1) / BS);
        b0 = min((uint32_t)load_uniform(table, e0), last_block);
        b1 = min((uint32_t)load_uniform(table, e1), last_block);
    };
    // Step st's K/V tiles go straight from global memory into LDS stage
    // st % kStages (global_load_lds_dwordx4: lane i of a wave writes bytes
    // 16i.. of the wave's 1 KiB).  Steps past the last one re-read the
    // sequence's last block (blocks_of clamps), so every step issues the same
    // CH loads and the vmcnt arithmetic below holds.
    // A lane's CH chunks sit at fixed offsets inside their block's tile:
    // steps start on 32-key boundaries and BS divides 32, so a tile's first
    // in-block key is 16t mod BS at every step and only the block ids change.
    // Chunks are wave-aligned (TOTAL and kThreads are multiples of 64), so a
    // chunk's pool, tile and LDS destination are the same for the whole wave:
    // they are kept as scalars, and each step's source is a scalar block base
    // plus the lane's fixed 32-bit offset: one 64-bit add per chunk and step is
    // the only per-lane address arithmetic in the loop.
    uint32_t coff[CH];          // per lane: byte offset from the chunk's block base
    const uint8_t *cpool[CH];   // per wave: K or V pool
    int64_t cstride[CH];        // per wave: bytes per pool block
    int cdst[CH];               // per wave: LDS byte offset inside a stage
    int cone[CH];               // per wave: the step's second 16-key tile
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        int c = threadIdx.x + i * kThreads;
        if (c >= TOTAL) c -= kThreads;                  // whole waves: repeat the previous chunk
        constexpr int KPT = KTILE / 16, VPT = VTILE / 16;
        const int is_k = __builtin_amdgcn_readfirstlane(c < 2 * KPT ? 1 : 0);
        cpool[i] = is_k ? a.k_pool : a.v_pool;
        // LDS position c holds image piece Swz::pos(c) of its tile (positions
        // and pieces are counted from the step image's start; tiles are whole
        // 16-piece groups)
        const int piece = is_k ? Swz<D, KB>::pos(c) : 2 * KPT + Swz<D, VB>::pos(c - 2 * KPT);
        coff[i] = (uint32_t)(chunk_src<D, BS, KB, VB>(piece, a.k_pool, a.v_pool, 0u, 0u, a.kv_heads, kvh, 0) -
                             cpool[i]);
        cstride[i] = (int64_t)a.kv_heads * BS * D * (is_k ? KB : VB);
        cone[i] = __builtin_amdgcn_readfirstlane((is_k ? c / KPT : (c - 2 * KPT) / VPT) == 1 ? 1 : 0);
        cdst[i] = __builtin_amdgcn_readfirstlane((c - lane) * 16);
    }
    // this lane's piece rotation in the swizzled K and V tile images
    const int ksw = Swz<D, KB>::PP > 1 ? (((g * 16 + m) * Swz<D, KB>::PP) >> 4) & (Swz<D, KB>::PP - 1) : 0;
    const int vsw = Swz<D, VB>::PP > 1 ? (((g * D + (D / 16) * m) * 4 * VB / 16) >> 4) & (Swz<D, VB>::PP - 1) : 0;
    auto issue = [&](int st) {
        const int p = st * kStep;
        uint32_t b0, b1;
        blocks_of(p, b0, b1);
        uint8_t *stage = lds[st % kStages];
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            // the block base stays one scalar value (readfirstlane keeps the
            // compiler from folding it into a per-lane 64-bit multiply-add)
            const uint64_t bu = (uint64_t)(cpool[i] + (int64_t)(cone[i] ? b1 : b0) * cstride[i]);
            const uint64_t bs = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(bu >> 32)) << 32) |
                                (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)bu);
            load_to_lds16(reinterpret_cast<const uint8_t *>(bs) + coff[i], stage + cdst[i]);
        }
    };

    // Careful pass only: per dim of this lane's V operand ((D/16)m + i), the
    // first key of each non-finite class that was taken out of the product
    // (0 NaN; for bf16 V also 1 +Inf, 2 -Inf).
    constexpr int NCLS = VB == 1 ? 1 : 3;
    int cfirst[NCLS][D / 16];

    // One 32-key step at keys p .. p+31: S^T = K Q^T, causal mask, online
    // softmax, O^T += V^T P^T.  kpiece(t, i) / vpiece(t, i) return the lane's
    // i-th 16-byte piece of its K key / V key group in 16-key tile t; diag:
    // some key may be past some row; tail: some key is past the sequence.
    // CAREFUL: non-finite V values are taken out of the product (below).
    auto compute = [&](const int p, const bool diag, const bool tail, auto kpiece, auto vpiece, auto careful_tag) {
        constexpr bool kCareful = decltype(careful_tag)::value;
        // ---- S^T for both row tiles, one 16-key K tile at a time (its codes
        // are read right before its MFMAs, as they are: the lane's D/4 codes
        // of the key), then the row maxima, then one wave vote for the lazy
        // rescale: straight-line code for both tiles between the vote's
        // branches, so their latency chains can interleave.
        f32x4 sc[kNR][2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if constexpr (KB == 2) {
                // bf16 K: the lane's D/4 values of key m, quarter g, as KK operands
                bf16x8 kb[KK];
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) kb[kk] = __builtin_bit_cast(bf16x8, kpiece(t, kk));
#pragma unroll
                for (int j = 0; j < kNR; ++j) {
                    sc[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < KK; ++kk)
                        sc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[kk], qb[j][kk], sc[j][t], 0, 0, 0);
                }
            } else {
                v8i ka[NC];
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    u32x4 k0 = kpiece(t, 2 * c), k1 = u32x4{0u, 0u, 0u, 0u};
                    if (NW > 4) k1 = kpiece(t, 2 * c + 1);
                    ka[c] = v8i{(int)k0[0], (int)k0[1], (int)k0[2], (int)k0[3],
                                (int)k1[0], (int)k1[1], (int)k1[2], (int)k1[3]};
                }
#pragma unroll
                for (int j = 0; j < kNR; ++j) {
                    sc[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int c = 0; c < NC; ++c) {
                        sc[j][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka[c], qh[j][c], sc[j][t], 0,
                                                                                    0, 0, kUnitScale, 0, kUnitScale);
                        sc[j][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka[c], ql[j][c], sc[j][t], 0,
                                                                                    0, 0, kUnitScale, 0, kLoScale);
                    }
                }
            }
        }
        float x[kNR][8];                                   // raw scores, scaled inside exp2
        float mx[kNR];
        bool grow = false;
#pragma unroll
        for (int j = 0; j < kNR; ++j) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) x[j][4 * t + i] = sc[j][t][i];
            if (diag || tail) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int key = p + 16 * t + 4 * g + i;
                        if (key > row_pos[j] || key >= total) x[j][4 * t + i] = -__builtin_inff();
                    }
            }
            // This lane's maximum over its 8 keys of the row.  The row's maximum
            // passes the bound exactly when one of its four lanes' does (the bound
            // is the same in all four and the scaling is monotonic), so the vote
            // needs no cross-lane step; the row maximum itself is only formed in
            // the rescale branch.
            float m8 = vmax(vmax(vmax(x[j][0], x[j][1]), x[j][2]),
                            vmax(vmax(x[j][3], x[j][4]), x[j][5]));
            m8 = vmax(vmax(m8, x[j][6]), x[j][7]);
            mx[j] = m8;
            grow |= m8 * qk_row[j] > run_max[j] + kLazy;
        }
        if (__any(grow)) {
#pragma unroll
            for (int j = 0; j < kNR; ++j) {
                // the row's four k-groups: lanes n, n^16, n^32, n^48
                const float row_max = max_xor32(max_xor16(mx[j])) * qk_row[j];
                const float ref = fmaxf(run_max[j], row_max);
                const float alpha = __builtin_amdgcn_exp2f(run_max[j] - ref);
                if constexpr (VB == 1)
                    rsum[j] *= alpha;
                else
                    run_sum[j] *= alpha;
#pragma unroll
                for (int t = 0; t < MT; ++t) acc[j][t] *= alpha;
                run_max[j] = ref;
            }
        }
        // P as the B operand of the product with V: f16 for E4M3 V; for bf16 V
        // two bf16 terms hi + lo (16 significant bits; one bf16 alone would
        // leave P with 8).
        f16x8 pb[kNR];
        bf16x8 ph[kNR], pl[kNR];
#pragma unroll
        for (int j = 0; j < kNR; ++j) {
            const float nm = -run_max[j];
            float pr[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j][i], qk_row[j], nm));
            if constexpr (VB == 2) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    ph[j][i] = (__bf16)pr[i];
                    pl[j][i] = (__bf16)(pr[i] - (float)ph[j][i]);
                }
            } else {
                pb[j] = f16x8{(_Float16)pr[0], (_Float16)pr[1], (_Float16)pr[2], (_Float16)pr[3],
                              (_Float16)pr[4], (_Float16)pr[5], (_Float16)pr[6], (_Float16)pr[7]};
            }
            if constexpr (VB == 2) {
                float ps = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) ps += pr[i];
                run_sum[j] += ps;
            }
        }
        // A wave that reaches its P.V products runs them at raised priority, so
        // that the SIMD's other waves fill the matrix cores' shadow with their
        // softmax work rather than the other way round (~2.5 %); the priority
        // drops back after the next step's barrier.
        if constexpr (!kCareful) __builtin_amdgcn_s_setprio(1);
        // ---- O^T += V^T P^T, V operands read now and converted once for
        // both row tiles (lane (m, g) holds keys 4g..4g+3 of dims (D/16)m..)
        if constexpr (VB == 2) {
            // bf16 V: per dim the four keys are 8 bytes; a 16-byte word holds
            // two dims, split into the operands of output tiles 2i and 2i+1
            u32x4 vv[2][NW / 2];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < NW / 2; ++i) vv[t][i] = vpiece(t, i);
            if (tail) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int valid = total - (p + 16 * t + 4 * g);
                    const uint32_t keep0 = (valid > 0 ? 0xFFFFu : 0u) | (valid > 1 ? 0xFFFF0000u : 0u);
                    const uint32_t keep1 = (valid > 2 ? 0xFFFFu : 0u) | (valid > 3 ? 0xFFFF0000u : 0u);
                    const u32x4 keep = {keep0, keep1, keep0, keep1};
#pragma unroll
                    for (int i = 0; i < NW / 2; ++i) vv[t][i] &= keep;
                }
            }
            if constexpr (kCareful) {
                // word e of piece i holds keys 2(e % 2), +1 of the lane's group
                // for dim (D/16)m + 2i + e/2
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int i = 0; i < NW / 2; ++i)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t w = vv[t][i][e];
                            const uint32_t n = bf16_nonfinite_halves(w);
                            if (!n) continue;
#pragma unroll
                            for (int h = 0; h < 2; ++h) {
                                if (!((n >> (16 * h + 15)) & 1u)) continue;
                                const uint32_t v = (w >> (16 * h)) & 0xFFFFu;
                                const int key = p + 16 * t + 4 * g + 2 * (e & 1) + h;
                                int &f = cfirst[(v & 0x7Fu) ? 0 : (v & 0x8000u) ? 2 : 1][2 * i + (e >> 1)];
                                f = min(f, key);
                            }
                            vv[t][i][e] = w & ~((n >> 15) * 0xFFFFu);
                        }
            }
#pragma unroll
            for (int i = 0; i < NW / 2; ++i) {
                const bf16x8 v0 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vv[0][i], vv[1][i], 0, 1, 4, 5));
                const bf16x8 v1 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vv[0][i], vv[1][i], 2, 3, 6, 7));
#pragma unroll
                for (int j = 0; j < kNR; ++j) {
                    acc[j][2 * i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v0, ph[j], acc[j][2 * i], 0, 0, 0);
                    acc[j][2 * i + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v1, ph[j], acc[j][2 * i + 1], 0, 0, 0);
                    acc[j][2 * i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v0, pl[j], acc[j][2 * i], 0, 0, 0);
                    acc[j][2 * i + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v1, pl[j], acc[j][2 * i + 1], 0, 0, 0);
                }
            }
        } else {
            uint32_t vw[2][NW];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int i = 0; i < NW / 4; ++i) {
                    const u32x4 vq = vpiece(t, i);
#pragma unroll
                    for (int e = 0; e < 4; ++e) vw[t][4 * i + e] = vq[e];
                }
            }
            if (tail) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int valid = total - (p + 16 * t + 4 * g);
                    const uint32_t keep = valid >= 4 ? 0xFFFFFFFFu : valid <= 0 ? 0u : (0xFFFFFFFFu >> (32 - 8 * valid));
#pragma unroll
                    for (int i = 0; i < NW; ++i) vw[t][i] &= keep;
                }
            }
            if constexpr (kCareful) {
                // word i holds keys 4g..4g+3 (bytes 0..3) of dim (D/16)m + i;
                // the lowest NaN byte is the word's first NaN key
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int i = 0; i < NW; ++i) {
                        const uint32_t n = e4m3_nan_bytes(vw[t][i]);
                        if (!n) continue;
                        cfirst[0][i] = min(cfirst[0][i], p + 16 * t + 4 * g + (int)(__builtin_ctz(n) >> 3));
                        vw[t][i] &= ~((n >> 7) * 0xFFu);
                    }
            }
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const f16x2 e0 = codes_to_f16x2<false>(vw[0][t]), e1 = codes_to_f16x2<true>(vw[0][t]);
                const f16x2 e2 = codes_to_f16x2<false>(vw[1][t]), e3 = codes_to_f16x2<true>(vw[1][t]);
                const f16x8 va = {e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
#pragma unroll
                for (int j = 0; j < kNR; ++j)
                    acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[j], acc[j][t], 0, 0, 0);
            }
            const _Float16 one = (_Float16)1.0f;
            const f16x8 ones = {one, one, one, one, one, one, one, one};
#pragma unroll
            for (int j = 0; j < kNR; ++j)
                rsum[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb[j], rsum[j], 0, 0, 0);
        }
    };

#pragma unroll
    for (int i = 0; i < kStages - 1; ++i) issue(i);
    const int first_row_pos = ctx + i0;
    // One step of the main pass: operands from the step's LDS image.  Steps
    // before the first one that reaches the tile's first query position need
    // no causal mask (DIAG false); every step from there on, the sequence's
    // tail included, runs the DIAG form.  Two loops keep the diagonal steps'
    // extra values out of the main loop's registers.
    auto step = [&](const int s, auto diag_tag) {
        constexpr bool kDiag = decltype(diag_tag)::value;
        const int p = s * kStep;
        const int buf = s % kStages;
        wait_vmcnt<(kStages - 2) * CH>();   // this wave's share of step s has landed
        // Everyone's share has, and every wave is done with step s-1's stage.
        // A bare s_barrier: the workgroup release fence of __syncthreads would
        // also wait for the transfers still in flight.  The ds_reads of step
        // s-1 were consumed by its MFMAs, so none is pending here.
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_s_setprio(0);
        issue(s + kStages - 1);
        const u32x4 *kimg = reinterpret_cast<const u32x4 *>(&lds[buf][(g * 16 + m) * Q4 * KB]);
        const u32x4 *vimg = reinterpret_cast<const u32x4 *>(&lds[buf][2 * KTILE + (g * D + (D / 16) * m) * 4 * VB]);
        compute(p, kDiag, kDiag && p + kStep > total,
                [&](int t, int i) { return kimg[t * (KTILE / 16) + (i ^ ksw)]; },
                [&](int t, int i) { return vimg[t * (VTILE / 16) + (i ^ vsw)]; }, Flag<false>{});
    };
    const int s_diag = min(nsteps, first_row_pos / kStep);
    for (int s = 0; s < s_diag; ++s) step(s, Flag<false>{});
    for (int s = s_diag; s < nsteps; ++s) step(s, Flag<true>{});
    __builtin_amdgcn_s_setprio(0);
    wait_vmcnt<0>();    // no LDS write may still be in flight when the workgroup ends

    // ---- Non-finite V values.  The definition sums over the keys a row sees
    // and only those, so a NaN V (a storable E4M3 code; bf16 pools keep NaN
    // and infinities) at a key past a row must not reach that row, and a seen
    // +-Inf makes the dim an infinity of its sign (NaN with both signs)
    // whatever the key's probability.  In the main pass such a value meets a
    // zero probability (a key past the row, an underflowed or exactly
    // representable P with lo = 0) as 0 * NaN or 0 * Inf, and a probability
    // P > 0 as NaN or +-Inf: either way an accumulator ends non-finite, and
    // it stays so (a rescale by a positive factor keeps it).  So a wave whose
    // accumulators are all finite saw none, and one that has a non-finite
    // accumulator runs its rows again in a careful pass: operands straight
    // from the cache in HBM (no LDS, no barrier; the other waves are done with
    // the stages), non-finite V values taken out of the product, and for each
    // dim the first key of each class; a row sees a prefix of the keys, so
    // afterwards the (dim, row) gets NaN when the row sees a NaN or both
    // infinities, else an infinity of the sign it sees.  (A NaN score, from a
    // NaN K code or q, makes its rows NaN in both passes.)
    float amax_acc = 0.0f;
#pragma unroll
    for (int j = 0; j < kNR; ++j)
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) amax_acc = vmax(amax_acc, fabsf(acc[j][t][i]));
    if (__any(!(amax_acc < __builtin_inff()))) {
        reset();
#pragma unroll
        for (int c = 0; c < NCLS; ++c)
#pragma unroll
            for (int i = 0; i < D / 16; ++i) cfirst[c][i] = 0x7FFFFFFF;
        for (int s = 0; s < nsteps; ++s) {
            const int p = s * kStep;
            uint32_t b0, b1;
            blocks_of(p, b0, b1);
            const uint8_t *kt[2], *vt[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int64_t base = ((int64_t)(t ? b1 : b0) * a.kv_heads + kvh) * (BS * D);   // elements
                const int tb = (p + 16 * t) % BS;
                kt[t] = a.k_pool + (base + (int64_t)(g * BS + tb + m) * Q4) * KB;
                vt[t] = a.v_pool + (base + (int64_t)((tb / 4 + g) * D + (D / 16) * m) * 4) * VB;
            }
            compute(p, p + kStep > first_row_pos, p + kStep > total,
                    [&](int t, int i) { return reinterpret_cast<const u32x4 *>(kt[t])[i]; },
                    [&](int t, int i) { return reinterpret_cast<const u32x4 *>(vt[t])[i]; }, Flag<true>{});
        }
        // first keys over the row's four k-groups, then into the lanes that
        // hold the dims: acc[j][t][i] of lane (n, g) is dim (D/16)(4g + i) + t,
        // whose V operand lane is 4g + i
#pragma unroll
        for (int c = 0; c < NCLS; ++c)
#pragma unroll
            for (int t = 0; t < D / 16; ++t) {
                int f = cfirst[c][t];
                f = min(f, __shfl_xor(f, 16));
                cfirst[c][t] = min(f, __shfl_xor(f, 32));
            }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                int f[NCLS];
#pragma unroll
                for (int c = 0; c < NCLS; ++c) f[c] = __shfl(cfirst[c][t], 4 * g + i);
#pragma unroll
                for (int j = 0; j < kNR; ++j) {
                    float term = 0.0f;
                    if constexpr (NCLS > 1) {
                        if (f[1] <= row_pos[j]) term = __builtin_inff();
                        if (f[2] <= row_pos[j]) term = term - __builtin_inff();   // +Inf - Inf is NaN
                    }
                    if (f[0] <= row_pos[j]) term = __builtin_nanf("");
                    acc[j][t][i] += term;
                }
            }
    }

    // ---- normalize and write: lane (n, g) holds rows n of its tiles, dims (D/16)(4g+r)+t
#pragma unroll
    for (int j = 0; j < kNR; ++j) {
        float l;
        if constexpr (VB == 1) {
            l = rsum[j][0];
        } else {
            l = run_sum[j];
            l += __shfl_xor(l, 16);
            l += __shfl_xor(l, 32);
        }
        if (!row_live[j]) continue;
        const int r = (wave * kNR + j) * 16 + m;
        const int tok = i0 + r / G;
        const int head = kvh * G + r % G;
        const float f = l > 0.0f ? a.v_scale / l : 0.0f;
        const int64_t obase = ((int64_t)(q0 + tok) * a.q_heads + head) * D;
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d = (D / 16) * (4 * g + i) + t;
                const float o = acc[j][t][i] * f;
                if (a.out_bf16)
                    static_cast<uint16_t *>(a.out)[obase + d] = f32_to_bf16_rne(o);
                else
                    static_cast<float *>(a.out)[obase + d] = o;
            }
    }
}

template <int D, int BS, int KB, int VB>
hipError_t launch_t(const PrefillArgs &a, hipStream_t stream) {
    const int G = a.q_heads / a.kv_heads;
    const int tok_per_tile = kRows / G;
    const int tiles = (a.max_q_len + tok_per_tile - 1) / tok_per_tile;
    if (tiles == 0) return hipSuccess;
    PrefillArgs la = a;
    la.q_tiles = tiles;
    const uint32_t units = (uint32_t)tiles * (uint32_t)(((a.num_seqs * a.kv_heads + 7) >> 3) << 3);
    hipLaunchKernelGGL((prefill_kernel<D, BS, KB, VB>), dim3(units), dim3(kThreads), 0, stream, la);
    return hipGetLastError();
}

template <int D, int BS>
hipError_t launch_types(const PrefillArgs &a, hipStream_t stream) {
    if (a.k_eb == 1 && a.v_eb == 1) return launch_t<D, BS, 1, 1>(a, stream);
    if constexpr (D <= 128) {       // bf16 pools hold head dims up to 128
        if (a.k_eb == 1 && a.v_eb == 2) return launch_t<D, BS, 1, 2>(a, stream);
        if (a.k_eb == 2 && a.v_eb == 1) return launch_t<D, BS, 2, 1>(a, stream);
        if (a.k_eb == 2 && a.v_eb == 2) return launch_t<D, BS, 2, 2>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
    if (a.block_size == 16) {
        if (a.head_dim == 64) return launch_types<64, 16>(a, stream);
        if (a.head_dim == 128) return launch_types<128, 16>(a, stream);
        if (a.head_dim == 256) return launch_types<256, 16>(a, stream);
    } else if (a.block_size == 32) {
        if (a.head_dim == 64) return launch_types<64, 32>(a, stream);
        if (a.head_dim == 128) return launch_types<128, 32>(a, stream);
        if (a.head_dim == 256) return launch_types<256, 32>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace kvf8
