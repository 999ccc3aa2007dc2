// paged_attn_prefill_chunk: causal attention of a chunk of new query tokens
// over an E4M3 paged cache that already holds the chunk's own K/V.
//
// [P1, tests/test-fp8.cpp check_fp8_attention: query token i at position
// ctx+i attends to positions <= ctx+i; build_attn stores K/V first and reads
// the cache views; build_attn_scale_kv_inputs/_output move the scales out of
// the products.]  As in the decode, s = (q . K_codes) * k_scale * sm_scale,
// o = v_scale * softmax(s) V_codes.
//
// Work decomposition.  Grid (query tile, kv-head, sequence).  A "row" is one
// (query token, head of the kv-head's group) pair; row r of a tile is token
// r / G, head r % G, so the G heads that share a kv-head share every K/V
// tile.  A workgroup of four waves owns 128 rows (two 16-row MFMA tiles per
// wave) and walks the keys 0 .. last row's position in 32-token steps:
//   * the step's K and V tiles (already in MFMA operand order in the cache)
//     are copied once into LDS and read by all four waves;
//   * S^T[key][row] = K Q^T on v_mfma_f32_16x16x32_bf16; its output is the
//     B operand of O^T[d][row] += V^T P^T on v_mfma_f32_16x16x32_f16;
//   * online softmax per row in the log2 domain with the same lazy reference
//     as the decode, P = exp2(fma(s, |qk|, -max)) from the raw MFMA scores;
//     causal masking only on steps that reach the tile's first query
//     position; the row sums come from one more MFMA with an all-ones V.
// The next step's tiles are loaded into registers while the current one is
// computed, then written to the other LDS buffer.

#include "fp8_device.hpp"
#include "internal.hpp"

namespace kvf8 {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStep = 32;              // keys per step (two 16-key tiles)
constexpr int kNR = 2;                 // 16-row MFMA tiles per wave
constexpr int kRows = kWaves * kNR * 16;
constexpr float kLazy = 8.0f;
constexpr float kNoMax = -1.0e30f;     // running-max sentinel (finite: see the accumulators)

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Bytes of one step in LDS: K tile 0, K tile 1, V tile 0, V tile 1 (16*D each).
template <int D>
struct StepLds {
    static constexpr int TILE = 16 * D;
    static constexpr int BYTES = 4 * TILE;
};

// Per-thread share of one step's global->LDS copy: 16-byte chunks.
template <int D>
struct CopyRegs {
    static constexpr int CHUNKS = StepLds<D>::BYTES / 16 / kThreads;   // 2 (D=128), 4 (D=256), 1 (D=64)
    u32x4 w[CHUNKS];
};

// Chunk c of a step (c in [0, 4*D)): tile kind (K/V), 16-key tile t, offset.
// K tile t: 4 quarters of 16 keys x D/4 bytes; in the cache quarter q of the
// tile's block starts at (q*BS + tb)*(D/4) with tb the tile's first in-block
// key.  V tile t: 4 groups of 4 keys, contiguous from (tb/4)*D*4.
template <int D, int BS>
__device__ __forceinline__ const uint8_t *chunk_src(int c, const uint8_t *k_pool, const uint8_t *v_pool,
                                                    uint32_t blk0, uint32_t blk1, int kv_heads, int kvh,
                                                    int p) {
    constexpr int Q4 = D / 4;
    constexpr int PER_TILE = StepLds<D>::TILE / 16;      // chunks per tile
    const int which = c / PER_TILE;                       // 0,1: K tiles; 2,3: V tiles
    const int off = (c % PER_TILE) * 16;                  // byte offset inside the 16*D tile image
    const int t = which & 1;
    const uint32_t blk = t == 0 ? blk0 : blk1;
    const int tb = (p + 16 * t) % BS;
    const int64_t base = ((int64_t)blk * kv_heads + kvh) * (BS * D);
    if (which < 2) {
        const int q = off / (16 * Q4);
        const int rem = off - q * 16 * Q4;
        return k_pool + base + (int64_t)(q * BS + tb) * Q4 + rem;
    }
    return v_pool + base + (int64_t)(tb / 4) * D * 4 + off;
}

template <int D, int BS>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs a) {
    constexpr int KK = D / 32;
    constexpr int MT = D / 16;
    constexpr int Q4 = D / 4;
    constexpr int NW = D / 16;
    constexpr int TILE = StepLds<D>::TILE;
    constexpr int CH = CopyRegs<D>::CHUNKS;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][StepLds<D>::BYTES];

    const int qt = blockIdx.x;
    const int kvh = blockIdx.y;
    const int b = blockIdx.z;
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

    // ---- Q^T operands of this wave's two row tiles; lane (n, g) holds row n.
    // A negative qk_scale is folded into Q (an exact sign flip of every bf16),
    // so the MFMA yields s / |qk_scale| * qk_scale's sign and the softmax works
    // with qk = |qk_scale| > 0.
    const uint32_t qsign = a.qk_scale < 0.0f ? 0x80008000u : 0u;
    const float qk = fabsf(a.qk_scale);
    bf16x8 qb[kNR][KK];
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
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            uint4 w = make_uint4(0, 0, 0, 0);
            if (row_live[j]) w = *reinterpret_cast<const uint4 *>(qrow + 8 * kk);
            w.x ^= qsign;
            w.y ^= qsign;
            w.z ^= qsign;
            w.w ^= qsign;
            qb[j][kk] = __builtin_bit_cast(bf16x8, w);
        }
    }

    // run_max starts at a finite sentinel far below any score, so that
    // exp2(s*qk - run_max) of a masked score (-inf) is 0 without a select and
    // the first rescale factor exp2(sentinel - ref) is 0.  The row sums are
    // accumulated by the MFMA with an all-ones A operand (sum_k P[row][k] in
    // every output dim), from the same f16 P as the numerator.
    f32x4 acc[kNR][MT];
    f32x4 lsum[kNR];
    float run_max[kNR];
#pragma unroll
    for (int j = 0; j < kNR; ++j) {
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        lsum[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        run_max[j] = kNoMax;
    }
    const f16x8 ones = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f,
                        (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f};

    auto blocks_of = [&](int p, uint32_t &b0, uint32_t &b1) {
        const int e0 = min(p, total - 1) / BS;
        const int e1 = min(p + 16, total - 1) / BS;
        b0 = min((uint32_t)table[e0], last_block);
        b1 = min((uint32_t)table[e1], last_block);
    };
    auto fetch = [&](CopyRegs<D> &r, int p) {
        uint32_t b0, b1;
        blocks_of(p, b0, b1);
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = threadIdx.x + i * kThreads;
            r.w[i] = *reinterpret_cast<const u32x4 *>(chunk_src<D, BS>(c, a.k_pool, a.v_pool, b0, b1,
                                                                         a.kv_heads, kvh, p));
        }
    };
    auto stash = [&](const CopyRegs<D> &r, int buf) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = threadIdx.x + i * kThreads;
            *reinterpret_cast<u32x4 *>(&lds[buf][c * 16]) = r.w[i];
        }
    };

    CopyRegs<D> cr;
    if (nsteps > 0) {
        fetch(cr, 0);
        stash(cr, 0);
    }
    __syncthreads();
    const int first_row_pos = ctx + i0;
    for (int s = 0; s < nsteps; ++s) {
        const int p = s * kStep;
        const int buf = s & 1;
        if (s + 1 < nsteps) fetch(cr, p + kStep);

        // ---- operands of this step from LDS (same lane mapping as the decode's loads)
        uint32_t kw[2][NW], vw[2][NW];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const u32x4 *kp = reinterpret_cast<const u32x4 *>(&lds[buf][t * TILE + (g * 16 + m) * Q4]);
            const u32x4 *vp = reinterpret_cast<const u32x4 *>(&lds[buf][(2 + t) * TILE + (g * D + (D / 16) * m) * 4]);
#pragma unroll
            for (int i = 0; i < NW / 4; ++i) {
                const u32x4 kq = kp[i], vq = vp[i];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kw[t][4 * i + e] = kq[e];
                    vw[t][4 * i + e] = vq[e];
                }
            }
        }
        const bool diag = p + kStep > first_row_pos;      // some key may be past some row
        const bool tail = p + kStep > total;              // keys past the sequence's cache
        if (tail) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int valid = total - (p + 16 * t + 4 * g);
                const uint32_t keep = valid >= 4 ? 0xFFFFFFFFu : valid <= 0 ? 0u : (0xFFFFFFFFu >> (32 - 8 * valid));
#pragma unroll
                for (int i = 0; i < NW; ++i) vw[t][i] &= keep;
            }
        }
        // K operands converted once for both row tiles
        bf16x8 ka[2][KK];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const uint32_t w0 = kw[t][2 * kk], w1 = kw[t][2 * kk + 1];
                const bf16x2 e0 = codes_to_bf16x2<false>(w0), e1 = codes_to_bf16x2<true>(w0);
                const bf16x2 e2 = codes_to_bf16x2<false>(w1), e3 = codes_to_bf16x2<true>(w1);
                ka[t][kk] = bf16x8{e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
            }
        f16x8 pb[kNR];
#pragma unroll
        for (int j = 0; j < kNR; ++j) {
            f32x4 sc[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                sc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[t][kk], qb[j][kk], sc[t], 0, 0, 0);
            }
            float x[8];                                    // raw scores, scaled inside exp2
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) x[4 * t + i] = sc[t][i];
            if (diag || tail) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int key = p + 16 * t + 4 * g + i;
                        if (key > row_pos[j] || key >= total) x[4 * t + i] = -__builtin_inff();
                    }
            }
            float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            mx *= qk;
            if (__any(mx > run_max[j] + kLazy)) {
                const float ref = fmaxf(run_max[j], mx);
                const float alpha = __builtin_amdgcn_exp2f(run_max[j] - ref);
                lsum[j] *= alpha;
#pragma unroll
                for (int t = 0; t < MT; ++t) acc[j][t] *= alpha;
                run_max[j] = ref;
            }
            const float nm = -run_max[j];
            float pr[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], qk, nm));
            pb[j] = f16x8{(_Float16)pr[0], (_Float16)pr[1], (_Float16)pr[2], (_Float16)pr[3],
                          (_Float16)pr[4], (_Float16)pr[5], (_Float16)pr[6], (_Float16)pr[7]};
            lsum[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb[j], lsum[j], 0, 0, 0);
        }
        // ---- O^T += V^T P^T, V operands converted once for both row tiles
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const f16x2 e0 = codes_to_f16x2<false>(vw[0][t]), e1 = codes_to_f16x2<true>(vw[0][t]);
            const f16x2 e2 = codes_to_f16x2<false>(vw[1][t]), e3 = codes_to_f16x2<true>(vw[1][t]);
            const f16x8 va = {e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
#pragma unroll
            for (int j = 0; j < kNR; ++j)
                acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[j], acc[j][t], 0, 0, 0);
        }
        if (s + 1 < nsteps) stash(cr, buf ^ 1);
        __syncthreads();
    }

    // ---- normalize and write: lane (n, g) holds rows n of its tiles, dims (D/16)(4g+r)+t
#pragma unroll
    for (int j = 0; j < kNR; ++j) {
        const float l = lsum[j][0];          // every output dim of the ones product holds the row sum
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

template <int D, int BS>
hipError_t launch_t(const PrefillArgs &a, hipStream_t stream) {
    const int G = a.q_heads / a.kv_heads;
    const int tok_per_tile = kRows / G;
    const int tiles = (a.max_q_len + tok_per_tile - 1) / tok_per_tile;
    if (tiles == 0) return hipSuccess;
    hipLaunchKernelGGL((prefill_kernel<D, BS>), dim3(tiles, a.kv_heads, a.num_seqs), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
    if (a.block_size == 16) {
        if (a.head_dim == 64) return launch_t<64, 16>(a, stream);
        if (a.head_dim == 128) return launch_t<128, 16>(a, stream);
        if (a.head_dim == 256) return launch_t<256, 16>(a, stream);
    } else if (a.block_size == 32) {
        if (a.head_dim == 64) return launch_t<64, 32>(a, stream);
        if (a.head_dim == 128) return launch_t<128, 32>(a, stream);
        if (a.head_dim == 256) return launch_t<256, 32>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace kvf8
