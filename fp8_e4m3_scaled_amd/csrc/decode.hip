// paged_attn_decode: one query token per sequence over an E4M3 paged cache.
//
// Math [P1, llama-graph.cpp build_attn_scale_kv_inputs/_output; tests
// check_fp8_attention]: with K_t, V_t the stored codes' values,
//   s_t = (q . K_t) * k_scale * sm_scale,   o = v_scale * sum_t softmax(s)_t V_t,
// i.e. attention over the dequantized cache with both scales moved out of
// the inner products.  Query head h reads kv-head h / G (G = Hq / Hkv).
//
// Work decomposition.  Grid (split, kv-head, sequence); a workgroup of four
// waves owns one chunk of one sequence's tokens for one kv-head and all G
// query heads of that group.  Each wave walks 32-token steps (two 16-token
// tiles) of the chunk, interleaved with the other waves:
//   * lane (m = lane%16, g = lane/16) loads, per tile, D/4 bytes of K (token
//     m, column quarter g) and D/4 bytes of V (four tokens 4g..4g+3 for dims
//     (D/16)m .. (D/16)m + D/16 - 1); in the tile layout both are contiguous,
//     so a wave reads each tile with 16-byte loads covering it exactly;
//   * S^T[token][head] = K Q^T on v_mfma_f32_16x16x32_bf16 (codes -> bf16 is
//     exact); its output layout (lane (n, g) holds tokens 4g..4g+3 of head n)
//     is exactly the B operand of the next product;
//   * O^T[d][head] += V^T P^T on v_mfma_f32_16x16x32_f16 (codes -> f16 exact,
//     P in f16), over 32 tokens per instruction;
//   * the online softmax runs in the log2 domain: running max per head,
//     per-lane partial sums, a rescale of the accumulators when the max moves.
// The next step's K/V bytes and block ids are loaded before the current step
// is computed.  The four waves then combine through LDS; with one split the
// workgroup writes the output, otherwise it writes (max, sum, acc) partials
// that decode_reduce combines.

#include "fp8_device.hpp"
#include "internal.hpp"

#include <cstdlib>

namespace kvf8 {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStep = 32;                 // tokens per wave step

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

template <int D>
struct StepRegs {
    static constexpr int NW = D / 16;     // dwords per lane per tile (K and V each)
    uint32_t k[2][NW];
    uint32_t v[2][NW];
};

template <int D, int BS>
__device__ __forceinline__ void load_step(StepRegs<D> &r, const uint8_t *k_pool, const uint8_t *v_pool,
                                          const int32_t *table, uint32_t last_block, int kv_heads, int kvh,
                                          int p, int end, int m, int g) {
    constexpr int Q4 = D / 4;
    constexpr int NW = D / 16;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int pt = p + 16 * t;
        if (pt < end) {
            // a block id outside the pool is a caller error; clamp it so it cannot fault
            const uint32_t blk = min((uint32_t)table[pt / BS], last_block);
            const int tb = pt % BS;
            const int64_t base = ((int64_t)blk * kv_heads + kvh) * (BS * D);
            const u32x4 *kp = reinterpret_cast<const u32x4 *>(k_pool + base + (g * BS + tb + m) * Q4);
            const u32x4 *vp = reinterpret_cast<const u32x4 *>(v_pool + base + ((tb / 4 + g) * D + (D / 16) * m) * 4);
#pragma unroll
            for (int i = 0; i < NW / 4; ++i) {
                const u32x4 kq = __builtin_nontemporal_load(kp + i);
                const u32x4 vq = __builtin_nontemporal_load(vp + i);
                r.k[t][4 * i + 0] = kq.x; r.k[t][4 * i + 1] = kq.y; r.k[t][4 * i + 2] = kq.z; r.k[t][4 * i + 3] = kq.w;
                r.v[t][4 * i + 0] = vq.x; r.v[t][4 * i + 1] = vq.y; r.v[t][4 * i + 2] = vq.z; r.v[t][4 * i + 3] = vq.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < NW; ++i) { r.k[t][i] = 0; r.v[t][i] = 0; }
        }
    }
}

template <int D, int BS>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
    constexpr int NW = D / 16;     // dwords of K (and of V) per lane per tile
    constexpr int KK = D / 32;     // QK^T instructions per tile
    constexpr int MT = D / 16;     // PV instructions per step (one per 16 dims)

    extern __shared__ float smem[];   // [waves][G] max, [waves][G] sum, [waves][G][D] acc

    const int split = blockIdx.x;
    const int kvh = blockIdx.y;
    const int b = blockIdx.z;
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

    const int32_t *table = a.block_tables + (int64_t)b * a.max_blocks;
    f32x4 acc[MT];
#pragma unroll
    for (int j = 0; j < MT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float run_max = -__builtin_inff();
    float run_sum = 0.0f;

    const int stride = kStep * kWaves;
    int p = c0 + kStep * wave;
    StepRegs<D> cur, nxt;
    if (p < c1) load_step<D, BS>(cur, a.k_pool, a.v_pool, table, last_block, a.kv_heads, kvh, p, c1, m, g);

    for (; p < c1; p += stride) {
        const int pn = p + stride;
        if (pn < c1) load_step<D, BS>(nxt, a.k_pool, a.v_pool, table, last_block, a.kv_heads, kvh, pn, c1, m, g);

        // ---- S^T = K Q^T for the two tiles
        f32x4 s[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const uint32_t w0 = cur.k[t][2 * kk], w1 = cur.k[t][2 * kk + 1];
                const bf16x2 e0 = codes_to_bf16x2<false>(w0), e1 = codes_to_bf16x2<true>(w0);
                const bf16x2 e2 = codes_to_bf16x2<false>(w1), e3 = codes_to_bf16x2<true>(w1);
                const bf16x8 ka = {e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
                s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[kk], s[t], 0, 0, 0);
            }
        }

        // ---- scale into the log2 domain, mask tokens past the chunk end
        float x[8];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = p + 16 * t + 4 * g + i;
                x[4 * t + i] = tok < c1 ? s[t][i] * a.qk_scale : -__builtin_inff();
            }
        float mx = x[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float new_max = fmaxf(run_max, mx);
        const float alpha = exp2f(run_max - new_max);
        float pr[8];
        float psum = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            pr[i] = exp2f(x[i] - new_max);
            psum += pr[i];
        }
        run_sum = run_sum * alpha + psum;
        run_max = new_max;
#pragma unroll
        for (int j = 0; j < MT; ++j) acc[j] *= alpha;

        // ---- tail: codes of tokens past the end must not reach the product (NaN * 0)
        if (p + kStep > c1) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int valid = c1 - (p + 16 * t + 4 * g);          // tokens of this lane's group left
                const uint32_t keep = valid >= 4 ? 0xFFFFFFFFu : valid <= 0 ? 0u : (0xFFFFFFFFu >> (32 - 8 * valid));
#pragma unroll
                for (int j = 0; j < NW; ++j) cur.v[t][j] &= keep;
            }
        }

        // ---- O^T += V^T P^T
        const f16x8 pb = {(_Float16)pr[0], (_Float16)pr[1], (_Float16)pr[2], (_Float16)pr[3],
                          (_Float16)pr[4], (_Float16)pr[5], (_Float16)pr[6], (_Float16)pr[7]};
#pragma unroll
        for (int j = 0; j < MT; ++j) {
            const f16x2 e0 = codes_to_f16x2<false>(cur.v[0][j]), e1 = codes_to_f16x2<true>(cur.v[0][j]);
            const f16x2 e2 = codes_to_f16x2<false>(cur.v[1][j]), e3 = codes_to_f16x2<true>(cur.v[1][j]);
            const f16x8 va = {e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb, acc[j], 0, 0, 0);
        }
        if (pn < c1) cur = nxt;
    }

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
template <int D>
__global__ __launch_bounds__(D) void decode_reduce(DecodeArgs a) {
    const int head = blockIdx.x;
    const int b = blockIdx.y;
    const int d = threadIdx.x;
    const int L = a.seq_lens[b];   // clamped the same way as in decode_kernel
    const int Lc = min(L, a.max_blocks * a.block_size);
    const int nsplit = Lc <= 0 ? 0 : min(a.splits, (Lc + a.chunk_tokens - 1) / a.chunk_tokens);
    const float *part = a.partials + ((int64_t)b * a.q_heads + head) * a.splits * (D + 2);
    float M = -__builtin_inff();
    for (int i = 0; i < nsplit; ++i) M = fmaxf(M, part[i * (D + 2)]);
    float num = 0.0f, den = 0.0f;
    for (int i = 0; i < nsplit; ++i) {
        const float mi = part[i * (D + 2)];
        const float f = mi == -__builtin_inff() ? 0.0f : exp2f(mi - M);
        num += f * part[i * (D + 2) + 2 + d];
        den += f * part[i * (D + 2) + 1];
    }
    const float o = nsplit > 0 ? num * a.v_scale / den : 0.0f;
    store_out(a.out, ((int64_t)b * a.q_heads + head) * D + d, o, a.out_bf16);
}

template <int D, int BS>
hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t stream) {
    const int G = a.q_heads / a.kv_heads;
    const size_t smem = sizeof(float) * (size_t)kWaves * G * (2 + D);
    hipLaunchKernelGGL((decode_kernel<D, BS>), dim3(a.splits, a.kv_heads, a.num_seqs), dim3(kThreads), smem,
                       stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    hipLaunchKernelGGL((decode_reduce<D>), dim3(a.q_heads, a.num_seqs), dim3(D), 0, stream, a);
    return hipGetLastError();
}

int env_int(const char *name, int dflt) {
    const char *s = std::getenv(name);
    if (!s || !*s) return dflt;
    const int v = std::atoi(s);
    return v > 0 ? v : dflt;
}

}  // namespace

// Chunking: at most `max_chunk` tokens per workgroup (bounds the tail of
// long sequences), and enough workgroups to give every CU two; chunks are a
// multiple of one round of wave steps.
void decode_plan(int32_t num_seqs, int32_t kv_heads, int32_t head_dim, int32_t block_size,
                 int32_t max_seq_len, int32_t *splits, int32_t *chunk_tokens) {
    static const int max_chunk = env_int("KVF8_DECODE_MAX_CHUNK", 4096);
    static const int target_wgs = env_int("KVF8_DECODE_TARGET_WGS", 512);
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
    s = (max_seq_len + chunk - 1) / chunk;
    if (s < 1) s = 1;
    *splits = (int32_t)s;
    *chunk_tokens = (int32_t)chunk;
    (void)head_dim;
    (void)block_size;
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
    if (a.block_size == 16) {
        if (a.head_dim == 64) return launch_decode_t<64, 16>(a, stream);
        if (a.head_dim == 128) return launch_decode_t<128, 16>(a, stream);
        if (a.head_dim == 256) return launch_decode_t<256, 16>(a, stream);
    } else if (a.block_size == 32) {
        if (a.head_dim == 64) return launch_decode_t<64, 32>(a, stream);
        if (a.head_dim == 128) return launch_decode_t<128, 32>(a, stream);
        if (a.head_dim == 256) return launch_decode_t<256, 32>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace kvf8
