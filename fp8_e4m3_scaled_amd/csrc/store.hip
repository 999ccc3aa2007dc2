// kv_store_fp8: quantize new bf16 K/V rows to E4M3 codes and scatter them
// into the paged pools by slot.
//
// [P1, llama-graph.cpp build_attn_scale_kv_inputs]: the cache holds K/s_k and
// V/s_v; here y = fl32(x * fl32(1/s)) and code = saturating RNE E4M3 of y
// [P2, ggml_fp32_to_f8_e4m3].  Negative slots and slots past the pool are
// skipped.
//
// One workgroup handles four consecutive input tokens.  Each thread reads a
// 16-byte-aligned run of bf16 values (coalesced across the workgroup) and
// writes whole 16-byte runs of codes:
//   K: 16 consecutive dims of one token lie inside one column quarter of the
//      tile, which is contiguous in the layout -> one 16-byte store;
//   V: when the four tokens fill one aligned 4-token group of a block (the
//      common case of prefill and fills), four dims x four tokens are 16
//      consecutive bytes -> one 16-byte store.  Otherwise each token's V byte
//      is written on its own (the decode-step case of one token per sequence).
// A bf16 pool gets the input bits at the same element positions (two bytes
// each): 32-byte runs for K and for a V group, two-byte writes otherwise.

#include "fp8_device.hpp"
#include "internal.hpp"

namespace kvf8 {
namespace {

constexpr int kStoreThreads = 256;
constexpr int kGroups = 1;          // four-token groups per workgroup

// KB / VB: element bytes of the K / V pool, 1 (E4M3 codes) or 2 (the bf16
// values as given, at the same element positions).
template <int KB, int VB>
__global__ __launch_bounds__(kStoreThreads) void store_kernel(StoreArgs a) {
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
    const int k_items = 4 * H * runs;   // per group: 4 tokens x H heads x runs
    const int v_items = H * quads;      // per group: H heads x quads, each over the four tokens

#pragma unroll
    for (int grp = 0; grp < kGroups; ++grp) {
        const int64_t tok0 = ((int64_t)blockIdx.x * kGroups + grp) * 4;
        if (tok0 >= a.num_tokens) break;
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
        for (int it = threadIdx.x; it < k_items; it += kStoreThreads) {
            const int k = it / (H * runs);
            const int rem = it - k * (H * runs);
            const int h = rem / runs;
            const int r = rem - h * runs;
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
                const uint32_t w[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                u32x4 out;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t p0 = w[2 * j], p1 = w[2 * j + 1];
                    out[j] = encode4(scaled(p0 & 0xFFFF, a.k_inv), scaled(p0 >> 16, a.k_inv),
                                     scaled(p1 & 0xFFFF, a.k_inv), scaled(p1 >> 16, a.k_inv));
                }
                *reinterpret_cast<u32x4 *>(kout + off) = out;
            } else {
                u32x4 *dst = reinterpret_cast<u32x4 *>(kout + 2 * off);
                dst[0] = lo;
                dst[1] = hi;
            }
        }

        // ---------------- V: an item is four dims of the four tokens
        const bool group = slot[0] >= 0 && (slot[0] & 3) == 0 && slot[1] == slot[0] + 1 &&
                           slot[2] == slot[0] + 2 && slot[3] == slot[0] + 3;
        for (int it = threadIdx.x; it < v_items; it += kStoreThreads) {
            const int h = it / quads;
            const int d4 = it - h * quads;
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
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        out[j] = encode4(scaled(b[0][j], a.v_inv), scaled(b[1][j], a.v_inv),
                                         scaled(b[2][j], a.v_inv), scaled(b[3][j], a.v_inv));
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
}

}  // namespace

hipError_t launch_store(const StoreArgs &a, hipStream_t stream) {
    const int64_t wgs = (a.num_tokens + 4 * kGroups - 1) / (4 * kGroups);
    if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (a.k_eb == 1 && a.v_eb == 1)
        hipLaunchKernelGGL((store_kernel<1, 1>), dim3((unsigned)wgs), dim3(kStoreThreads), 0, stream, a);
    else if (a.k_eb == 1)
        hipLaunchKernelGGL((store_kernel<1, 2>), dim3((unsigned)wgs), dim3(kStoreThreads), 0, stream, a);
    else if (a.v_eb == 1)
        hipLaunchKernelGGL((store_kernel<2, 1>), dim3((unsigned)wgs), dim3(kStoreThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((store_kernel<2, 2>), dim3((unsigned)wgs), dim3(kStoreThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kvf8
