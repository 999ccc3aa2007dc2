// kv_store_fp8: quantize new bf16 K/V rows to E4M3 codes and scatter them
// into the paged pools by slot.
//
// [P1, llama-graph.cpp build_attn_scale_kv_inputs]: the cache holds K/s_k and
// V/s_v; here y = fl32(x * fl32(1/s)) and code = saturating RNE E4M3 of y
// [P2, ggml_fp32_to_f8_e4m3].  Negative slots and slots past the pool are
// skipped.
//
// One workgroup handles sixteen consecutive input tokens (in a call of few
// tokens up to kv_heads workgroups share them, each taking a range of the
// kv-heads, so that a decode step's append still spreads over the chip).
// When they go to sixteen consecutive slots starting at a multiple of 16
// (every fill and every prefill chunk: a whole block, or half of a 32-token
// block), the workgroup writes each head's part of the K and V tiles as one
// contiguous run (K: 16 tokens x D codes of a column-quarter layout; V: 4
// groups of 4 tokens), each thread with several 16-byte loads in flight.
// Otherwise each
// of its four waves takes four of the tokens on the path below, where each
// lane reads a 16-byte-aligned run of bf16 values (coalesced across the
// wave) and writes whole 16-byte runs of codes:
//   K: 16 consecutive dims of one token lie inside one column quarter of the
//      tile, which is contiguous in the layout -> one 16-byte store;
//   V: when the four tokens fill one aligned 4-token group of a block (the
//      common case of prefill and fills), four dims x four tokens are 16
//      consecutive bytes -> one 16-byte store.  Otherwise each token's V byte
//      is written on its own (the decode-step case of one token per sequence).
// A bf16 pool gets the input bits at the same element positions (two bytes
// each): 32-byte runs for K and for a V group, two-byte writes otherwise.
//
// A piece of values that holds no NaN (one integer test per two values) is
// encoded without the per-value NaN tests and NaN rebuild, the same codes in
// about half the instructions; with them the arithmetic cost the fill about
// 9 % over a copy of its bytes through the same addresses.

#include "fp8_device.hpp"
#include "internal.hpp"

namespace kvf8 {
namespace {

constexpr int kStoreThreads = 256;
constexpr int64_t kMinStoreWgs = 1024;   // 4 workgroups per CU

// Bit 15 of each half of w that holds a bf16 NaN (exponent all ones and a
// nonzero fraction: magnitude bits above 0x7F80).
__device__ __forceinline__ uint32_t bf16_nan_halves(uint32_t w) {
    return ((w & 0x7FFF7FFFu) + 0x007F007Fu) & 0x80008000u;
}

// Four codes of four bf16 values (two words) that hold no NaN: the product
// with the reciprocal scale, clamped to +-448 (Inf included), converted with
// round-half-even; equal to encode4(scaled(..)) for such values.
__device__ __forceinline__ uint32_t encode4_no_nan(uint32_t p0, uint32_t p1, float inv) {
    return encode4_finite(__uint_as_float(p0 << 16) * inv, __uint_as_float(p0 & 0xFFFF0000u) * inv,
                          __uint_as_float(p1 << 16) * inv, __uint_as_float(p1 & 0xFFFF0000u) * inv);
}

// Sixteen consecutive bf16 values (two 16-byte words) -> sixteen codes.
__device__ __forceinline__ u32x4 encode16(u32x4 lo, u32x4 hi, float inv) {
    const uint32_t w[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    uint32_t nan = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) nan |= bf16_nan_halves(w[j]);
    u32x4 out;
    if (nan == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) out[j] = encode4_no_nan(w[2 * j], w[2 * j + 1], inv);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t p0 = w[2 * j], p1 = w[2 * j + 1];
            out[j] = encode4(scaled(p0 & 0xFFFF, inv), scaled(p0 >> 16, inv), scaled(p1 & 0xFFFF, inv),
                             scaled(p1 >> 16, inv));
        }
    }
    return out;
}

// Four consecutive input tokens tok0.. (those at or past num_tokens are
// absent), each to its own slot.  KB / VB: element bytes of the K / V pool,
// 1 (E4M3 codes) or 2 (the bf16 values as given, at the same positions).
template <int KB, int VB>
__device__ __forceinline__ void store_quad(const StoreArgs &a, int64_t tok0, int tid, int nthr, int h0, int nh) {
    const int D = a.head_dim;
    const int H = a.kv_heads;
    const int BS = a.block_size;
    const int quarter = D >> 2;
    const int64_t tile = (int64_t)BS * D;
    const uint16_t *__restrict__ kin = a.k;
    const uint16_t *__restrict__ vin = a.v;
    uint8_t *__restrict__ kout = a.k_pool;
    uint8_t *__restrict__ vout = a.v_pool;
    const int runs = D >> 4;            // 16-dim runs per head
    const int quads = D >> 2;           // 4-dim runs per head
    const int k_items = 4 * nh * runs;  // 4 tokens x nh heads (h0 ..) x runs
    const int v_items = nh * quads;     // nh heads x quads, each over the four tokens

    int64_t slot[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        slot[k] = (tok0 + k < a.num_tokens) ? a.slots[tok0 + k] : -1;
        if (slot[k] >= a.pool_slots) slot[k] = -1;    // outside the pool: skipped, never written
    }

    // Every data load below depends only on the token count, not on the
    // slots, so the slot reads and the K/V reads are in flight together;
    // the slots only decide where (and whether) the results are written.

    // ---------------- K: 16 dims of one token -> one 16-byte run of codes
    for (int it = tid; it < k_items; it += nthr) {
        const int k = it / (nh * runs);
        const int rem = it - k * (nh * runs);
        const int hh = rem / runs;
        const int r = rem - hh * runs;
        const int h = h0 + hh;
        if (tok0 + k >= a.num_tokens) continue;
        const u32x4 *src = reinterpret_cast<const u32x4 *>(kin + (tok0 + k) * a.k_stride + (int64_t)h * D + r * 16);
        const u32x4 lo = src[0], hi = src[1];
        const int64_t s = slot[k];
        if (s < 0) continue;
        const int64_t blk = s / BS;
        const int t = (int)(s - blk * BS);
        const int d0 = r * 16;
        const int64_t off = (blk * H + h) * tile + ((int64_t)(d0 / quarter) * BS + t) * quarter + d0 % quarter;
        if constexpr (KB == 1) {
            *reinterpret_cast<u32x4 *>(kout + off) = encode16(lo, hi, a.k_inv);
        } else {
            u32x4 *dst = reinterpret_cast<u32x4 *>(kout + 2 * off);
            dst[0] = lo;
            dst[1] = hi;
        }
    }

    // ---------------- V: an item is four dims of the four tokens
    const bool group = slot[0] >= 0 && (slot[0] & 3) == 0 && slot[1] == slot[0] + 1 &&
                       slot[2] == slot[0] + 2 && slot[3] == slot[0] + 3;
    for (int it = tid; it < v_items; it += nthr) {
        const int hh = it / quads;
        const int d4 = it - hh * quads;
        const int h = h0 + hh;
        uint32_t b[4][4];   // [token][dim] bf16 bits
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint2 w = make_uint2(0u, 0u);
            if (tok0 + k < a.num_tokens)
                w = *reinterpret_cast<const uint2 *>(vin + (tok0 + k) * a.v_stride + (int64_t)h * D + d4 * 4);
            b[k][0] = w.x & 0xFFFF;
            b[k][1] = w.x >> 16;
            b[k][2] = w.y & 0xFFFF;
            b[k][3] = w.y >> 16;
        }
        if (group) {
            // the four tokens fill one aligned 4-token group: 16 consecutive codes
            const int64_t blk = slot[0] / BS;
            const int t0 = (int)(slot[0] - blk * BS);
            const int64_t off = (blk * H + h) * tile + ((int64_t)(t0 >> 2) * D + d4 * 4) * 4;
            if constexpr (VB == 1) {
                u32x4 out;
                uint32_t nan = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k) nan |= bf16_nan_halves(b[k][0] | (b[k][1] << 16)) |
                                                   bf16_nan_halves(b[k][2] | (b[k][3] << 16));
                if (nan == 0) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        out[j] = encode4_finite(bf16_to_f32(b[0][j]) * a.v_inv, bf16_to_f32(b[1][j]) * a.v_inv,
                                                bf16_to_f32(b[2][j]) * a.v_inv, bf16_to_f32(b[3][j]) * a.v_inv);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        out[j] = encode4(scaled(b[0][j], a.v_inv), scaled(b[1][j], a.v_inv),
                                         scaled(b[2][j], a.v_inv), scaled(b[3][j], a.v_inv));
                }
                *reinterpret_cast<u32x4 *>(vout + off) = out;
            } else {
                // dim j: tokens 0..3 as four consecutive bf16 values
                u32x4 o0, o1;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    o0[2 * j] = b[0][j] | (b[1][j] << 16);
                    o0[2 * j + 1] = b[2][j] | (b[3][j] << 16);
                    o1[2 * j] = b[0][j + 2] | (b[1][j + 2] << 16);
                    o1[2 * j + 1] = b[2][j + 2] | (b[3][j + 2] << 16);
                }
                u32x4 *dst = reinterpret_cast<u32x4 *>(vout + 2 * off);
                dst[0] = o0;
                dst[1] = o1;
            }
        } else {
            // token by token: a token's four codes sit 4 bytes apart
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int64_t s = slot[k];
                if (s < 0) continue;
                const int64_t blk = s / BS;
                const int t = (int)(s - blk * BS);
                const int64_t e = (blk * H + h) * tile + ((int64_t)(t >> 2) * D + d4 * 4) * 4 + (t & 3);
                if constexpr (VB == 1) {
                    const uint32_t c = encode4(scaled(b[k][0], a.v_inv), scaled(b[k][1], a.v_inv),
                                               scaled(b[k][2], a.v_inv), scaled(b[k][3], a.v_inv));
                    uint8_t *dst = vout + e;
                    dst[0] = (uint8_t)(c & 0xFF);
                    dst[4] = (uint8_t)((c >> 8) & 0xFF);
                    dst[8] = (uint8_t)((c >> 16) & 0xFF);
                    dst[12] = (uint8_t)(c >> 24);
                } else {
                    uint16_t *dst = reinterpret_cast<uint16_t *>(vout) + e;
                    dst[0] = (uint16_t)b[k][0];
                    dst[4] = (uint16_t)b[k][1];
                    dst[8] = (uint16_t)b[k][2];
                    dst[12] = (uint16_t)b[k][3];
                }
            }
        }
    }
}

// Sixteen consecutive input tokens tok0.. to the sixteen consecutive slots
// s0.. (s0 a multiple of 16, all inside the pool), E4M3 pools: a whole
// 16-token run of every head's K and V tiles.
//   K: piece (h, q, t, j) = 16 codes of token t, dims q D/4 + 16j.. (j <
//      D/64), at tile byte (q BS + t0 + t) D/4 + 16j; for a fixed (h, q) the
//      pieces of the 16 tokens are one contiguous 16 D/4-byte run.
//   V: piece (h, g, o) = 8 dims (8o..) x the four tokens 4g.. of a group, 32
//      codes at tile byte ((t0/4 + g) D + 8o) 4: contiguous over (g, o).
// Consecutive threads take consecutive pieces, so a wave's stores are
// contiguous runs; each thread has all its loads in flight before it
// encodes.
__device__ __forceinline__ void store_run16(const StoreArgs &a, int64_t tok0, int64_t s0, int h0, int nh) {
    const int D = a.head_dim;
    const int H = a.kv_heads;
    const int BS = a.block_size;
    const int Q4 = D >> 2;
    const int64_t tile = (int64_t)BS * D;
    const int64_t blk = s0 / BS;
    const int t0 = (int)(s0 - blk * BS);
    const int np = D >> 6;                // 16-code pieces per column quarter of a token
    const int kper = 16 * (D >> 4);       // K pieces per head: 16 tokens x D/16 runs
    const int vper = 4 * (D >> 3);        // V pieces per head: 4 groups x D/8 runs
    const int k_items = nh * kper, v_items = nh * vper;
    for (int base = 0; base < k_items; base += 4 * kStoreThreads) {
        u32x4 lo[4], hi[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int it = base + u * kStoreThreads + threadIdx.x;
            if (it < k_items) {
                const int hh = it / kper;
                const int r = it - hh * kper;                   // (q, t, j) in this order
                const int h = h0 + hh;
                const int j = r % np, t = (r / np) & 15, q = r / (16 * np);
                const u32x4 *src =
                    reinterpret_cast<const u32x4 *>(a.k + (tok0 + t) * a.k_stride + (int64_t)h * D + q * Q4 + j * 16);
                lo[u] = src[0];
                hi[u] = src[1];
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int it = base + u * kStoreThreads + threadIdx.x;
            if (it < k_items) {
                const int hh = it / kper;
                const int r = it - hh * kper;
                const int h = h0 + hh;
                const int j = r % np, t = (r / np) & 15, q = r / (16 * np);
                const int64_t off = (blk * H + h) * tile + (int64_t)(q * BS + t0 + t) * Q4 + j * 16;
                *reinterpret_cast<u32x4 *>(a.k_pool + off) = encode16(lo[u], hi[u], a.k_inv);
            }
        }
    }
    for (int base = 0; base < v_items; base += 2 * kStoreThreads) {
        u32x4 x[2][4];        // [item][token]: dims 8o..8o+7 of token 4g + k
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int it = base + u * kStoreThreads + threadIdx.x;
            if (it < v_items) {
                const int hh = it / vper;
                const int r = it - hh * vper;                   // (g, o)
                const int h = h0 + hh;
                const int g = r / (D >> 3), o = r - g * (D >> 3);
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    x[u][k] = *reinterpret_cast<const u32x4 *>(a.v + (tok0 + 4 * g + k) * a.v_stride + (int64_t)h * D +
                                                               8 * o);
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int it = base + u * kStoreThreads + threadIdx.x;
            if (it < v_items) {
                const int hh = it / vper;
                const int r = it - hh * vper;
                const int h = h0 + hh;
                const int g = r / (D >> 3), o = r - g * (D >> 3);
                // dim j of the eight: bf16 j/2 of word j/2 ... of each token
                u32x4 out[2];
                uint32_t nan = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                    for (int w = 0; w < 4; ++w) nan |= bf16_nan_halves(x[u][k][w]);
                if (nan == 0) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int w = j >> 1;
                        float f[4];
#pragma unroll
                        for (int k = 0; k < 4; ++k)
                            f[k] = __uint_as_float((j & 1) ? (x[u][k][w] & 0xFFFF0000u) : (x[u][k][w] << 16)) * a.v_inv;
                        out[j >> 2][j & 3] = encode4_finite(f[0], f[1], f[2], f[3]);
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int w = j >> 1, sh = 16 * (j & 1);
                        out[j >> 2][j & 3] = encode4(scaled((x[u][0][w] >> sh) & 0xFFFF, a.v_inv),
                                                     scaled((x[u][1][w] >> sh) & 0xFFFF, a.v_inv),
                                                     scaled((x[u][2][w] >> sh) & 0xFFFF, a.v_inv),
                                                     scaled((x[u][3][w] >> sh) & 0xFFFF, a.v_inv));
                    }
                }
                u32x4 *dst = reinterpret_cast<u32x4 *>(a.v_pool + (blk * H + h) * tile +
                                                       ((int64_t)(t0 / 4 + g) * D + 8 * o) * 4);
                dst[0] = out[0];
                dst[1] = out[1];
            }
        }
    }
}

template <int KB, int VB>
__global__ __launch_bounds__(kStoreThreads) void store_kernel(StoreArgs a) {
    const int64_t tok0 = (int64_t)blockIdx.x * 16;
    // kv-heads [h0, h0 + nh) of the 16 tokens: gridDim.y workgroups share a group's heads
    const int h0 = (int)(((int64_t)blockIdx.y * a.kv_heads) / gridDim.y);
    const int nh = (int)(((int64_t)(blockIdx.y + 1) * a.kv_heads) / gridDim.y) - h0;
    if constexpr (KB == 1 && VB == 1) {
        // the run test: 16 tokens present, slots s0 .. s0+15 with s0 % 16 == 0, inside the pool
        __shared__ int64_t s_first;
        __shared__ int s_run;
        if (threadIdx.x < 64) {
            const int lane = threadIdx.x;
            int64_t s = -1;
            if (lane < 16 && tok0 + lane < a.num_tokens) s = a.slots[tok0 + lane];
            const int64_t s0 = __shfl(s, 0);
            const bool ok = lane >= 16 || (s == s0 + lane && s >= 0 && s < a.pool_slots);
            const bool run = __all(ok) && (s0 & 15) == 0;
            if (lane == 0) {
                s_first = s0;
                s_run = run ? 1 : 0;
            }
        }
        __syncthreads();
        if (s_run) {
            store_run16(a, tok0, s_first, h0, nh);
            return;
        }
    }
    // otherwise wave w stores tokens tok0 + 4w .. + 3, the four waves side by side
    const int64_t quad = tok0 + 4 * (threadIdx.x >> 6);
    if (quad < a.num_tokens) store_quad<KB, VB>(a, quad, threadIdx.x & 63, 64, h0, nh);
}

}  // namespace

hipError_t launch_store(const StoreArgs &a, hipStream_t stream) {
    const int64_t wgs = (a.num_tokens + 15) / 16;
    if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
    // Few tokens (a decode step's one token per sequence) would leave most of
    // the chip idle: the kv-heads of a 16-token group are then split over up
    // to kv_heads workgroups, so that at least ~kMinStoreWgs run.
    int64_t split = (kMinStoreWgs + wgs - 1) / wgs;
    if (split > a.kv_heads) split = a.kv_heads;
    if (split < 1) split = 1;
    const dim3 grid((unsigned)wgs, (unsigned)split);
    if (a.k_eb == 1 && a.v_eb == 1)
        hipLaunchKernelGGL((store_kernel<1, 1>), grid, dim3(kStoreThreads), 0, stream, a);
    else if (a.k_eb == 1)
        hipLaunchKernelGGL((store_kernel<1, 2>), grid, dim3(kStoreThreads), 0, stream, a);
    else if (a.v_eb == 1)
        hipLaunchKernelGGL((store_kernel<2, 1>), grid, dim3(kStoreThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((store_kernel<2, 2>), grid, dim3(kStoreThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kvf8
