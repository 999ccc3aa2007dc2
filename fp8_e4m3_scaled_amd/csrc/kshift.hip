// kv_shift_rope: move cached K by a RoPE position delta, in place.
//
// [P1, src/llama-kv-cache.cpp build_rope_shift keeps F8_E4M3 out of the
// in-place rope; tests/test-fp8.cpp check_fp8_context_shift expects the cache
// bytes to equal quantize(rope(to_float(bytes), shift)), with no scale.]
//
// For rotary pair i the host passes c_i = fl32(cos a_i), s_i = fl32(sin a_i)
// with a_i = delta * theta^(-2i/rot).  With x0, x1 the pair's decoded E4M3
// values (exact in fp32 and fp64),
//   y0 = fl32(fl64(x0*c) - fl64(x1*s)),   y1 = fl32(fl64(x0*s) + fl64(x1*c)),
// then both are encoded as in the store.  The fp64 products are exact (a
// 4-bit by 24-bit significand), so only the sum and the final narrowing round.
// A pair holding a NaN code becomes the NaN code 0x7F in both places.
//
// Work items.  Run path (NEOX with rot % 32 == 0, NORM with rot % 16 == 0):
// a thread rotates 16 pairs whose bytes are two 16-byte runs of one token's K
// row (both inside a column quarter of the tile, hence contiguous): NEOX runs
// [16r, 16r+16) and [16r + rot/2, ...); NORM one run [16r, 16r+16) holding
// eight (2i, 2i+1) pairs.  Byte path (any other even rot): one pair per thread.

#include "fp8_device.hpp"
#include "internal.hpp"

namespace kvf8 {
namespace {

constexpr int kThreads = 256;

struct Table {
    float c[128];
    float s[128];
};

__device__ __forceinline__ int64_t k_offset(int t, int d, int BS, int D) {
    const int q = D >> 2;
    return ((int64_t)(d / q) * BS + t) * q + d % q;
}

__device__ __forceinline__ void load_table(Table &lds, const KShiftArgs &a) {
    for (int i = threadIdx.x; i < a.rot_dim / 2; i += kThreads) {
        lds.c[i] = a.cos_t[i];
        lds.s[i] = a.sin_t[i];
    }
    __syncthreads();
}

// Rotate one pair of codes; returns the two new codes (c0 in bits 0-7, c1 in 8-15).
__device__ __forceinline__ uint32_t rotate_pair(float x0, float x1, float cf, float sf) {
#pragma clang fp contract(off)
    if (__builtin_isnan(x0) || __builtin_isnan(x1)) return 0x7F7Fu;
    const double c = (double)cf, s = (double)sf;
    const double a = (double)x0, b = (double)x1;
    const double y0 = a * c - b * s;
    const double y1 = a * s + b * c;
    return encode2((float)y0, (float)y1);
}

__global__ __launch_bounds__(kThreads) void kshift_runs(KShiftArgs a) {
    __shared__ Table tab;
    load_table(tab, a);
    const int D = a.head_dim, BS = a.block_size, H = a.kv_heads;
    const int runs = a.neox ? a.rot_dim / 32 : a.rot_dim / 16;
    const int64_t item = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t total = a.n_slots * H * runs;
    if (item >= total) return;
    const int r = (int)(item % runs);
    const int h = (int)((item / runs) % H);
    const int64_t si = item / ((int64_t)runs * H);
    const int64_t slot = a.slots[si];
    if (slot < 0 || slot >= a.pool_slots) return;     // skipped, never written
    const int64_t blk = slot / BS;
    const int t = (int)(slot - blk * BS);
    uint8_t *tile = a.k_pool + (blk * H + h) * (int64_t)BS * D;

    if (a.neox) {
        const int i0 = 16 * r;
        u32x4 *pa = reinterpret_cast<u32x4 *>(tile + k_offset(t, i0, BS, D));
        u32x4 *pb = reinterpret_cast<u32x4 *>(tile + k_offset(t, i0 + a.rot_dim / 2, BS, D));
        const u32x4 wa = *pa, wb = *pb;
        u32x4 oa, ob;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const f32x2 a01 = codes_to_f32x2<false>(wa[w]), a23 = codes_to_f32x2<true>(wa[w]);
            const f32x2 b01 = codes_to_f32x2<false>(wb[w]), b23 = codes_to_f32x2<true>(wb[w]);
            const float xa[4] = {a01[0], a01[1], a23[0], a23[1]};
            const float xb[4] = {b01[0], b01[1], b23[0], b23[1]};
            uint32_t ca = 0, cb = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = i0 + 4 * w + k;
                const uint32_t y = rotate_pair(xa[k], xb[k], tab.c[i], tab.s[i]);
                ca |= (y & 0xFFu) << (8 * k);
                cb |= ((y >> 8) & 0xFFu) << (8 * k);
            }
            oa[w] = ca;
            ob[w] = cb;
        }
        *pa = oa;
        *pb = ob;
    } else {
        const int d0 = 16 * r;           // eight (2i, 2i+1) pairs, i = d0/2 ..
        u32x4 *pa = reinterpret_cast<u32x4 *>(tile + k_offset(t, d0, BS, D));
        const u32x4 wa = *pa;
        u32x4 oa;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const f32x2 a01 = codes_to_f32x2<false>(wa[w]), a23 = codes_to_f32x2<true>(wa[w]);
            const int i = d0 / 2 + 2 * w;
            const uint32_t y0 = rotate_pair(a01[0], a01[1], tab.c[i], tab.s[i]);
            const uint32_t y1 = rotate_pair(a23[0], a23[1], tab.c[i + 1], tab.s[i + 1]);
            oa[w] = (y0 & 0xFFFFu) | (y1 << 16);
        }
        *pa = oa;
    }
}

__global__ __launch_bounds__(kThreads) void kshift_pairs(KShiftArgs a) {
    __shared__ Table tab;
    load_table(tab, a);
    const int D = a.head_dim, BS = a.block_size, H = a.kv_heads;
    const int half = a.rot_dim / 2;
    const int64_t item = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t total = a.n_slots * H * half;
    if (item >= total) return;
    const int p = (int)(item % half);
    const int h = (int)((item / half) % H);
    const int64_t si = item / ((int64_t)half * H);
    const int64_t slot = a.slots[si];
    if (slot < 0 || slot >= a.pool_slots) return;     // skipped, never written
    const int64_t blk = slot / BS;
    const int t = (int)(slot - blk * BS);
    uint8_t *tile = a.k_pool + (blk * H + h) * (int64_t)BS * D;
    const int d0 = a.neox ? p : 2 * p;
    const int d1 = a.neox ? p + half : 2 * p + 1;
    uint8_t *b0 = tile + k_offset(t, d0, BS, D);
    uint8_t *b1 = tile + k_offset(t, d1, BS, D);
    const f32x2 x = codes_to_f32x2<false>((uint32_t)*b0 | ((uint32_t)*b1 << 8));
    const uint32_t y = rotate_pair(x[0], x[1], tab.c[p], tab.s[p]);
    *b0 = (uint8_t)(y & 0xFF);
    *b1 = (uint8_t)(y >> 8);
}

}  // namespace

hipError_t launch_kshift(const KShiftArgs &a, hipStream_t stream) {
    const bool runs = a.neox ? (a.rot_dim % 32 == 0) : (a.rot_dim % 16 == 0);
    const int64_t per_row = runs ? (a.neox ? a.rot_dim / 32 : a.rot_dim / 16) : a.rot_dim / 2;
    const int64_t total = a.n_slots * a.kv_heads * per_row;
    const int64_t wgs = (total + kThreads - 1) / kThreads;
    if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (runs)
        hipLaunchKernelGGL(kshift_runs, dim3((unsigned)wgs), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(kshift_pairs, dim3((unsigned)wgs), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kvf8
