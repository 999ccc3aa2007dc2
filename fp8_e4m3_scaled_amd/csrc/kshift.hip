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
//
// Per-slot deltas (kv_shift_rope_per_slot): each slot names a row of a cos/sin
// table in device memory, built on the host for each distinct delta exactly
// as the single-delta table; the same rotation then runs with that row's
// values.  [P1, tests/test-fp8.cpp check_fp8_context_shift: the shift tensor
// holds one offset per cache cell.]

#include "fp8_device.hpp"
#include "internal.hpp"

namespace kvf8 {
namespace {

constexpr int kThreads = 256;
constexpr int kRunsUnroll = 1;            // (slot, head) items per lane per iteration (2-4 measured slower)
constexpr int64_t kRunsMaxWgs = 4096;     // 16 workgroups per CU

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
__device__ __forceinline__ uint32_t rotate_pair(float x0, float x1, double c, double s) {
#pragma clang fp contract(off)
    if (__builtin_isnan(x0) || __builtin_isnan(x1)) return 0x7F7Fu;
    const double a = (double)x0, b = (double)x1;
    const double y0 = a * c - b * s;
    const double y1 = a * s + b * c;
    return encode2((float)y0, (float)y1);
}

// The same rotation for non-NaN inputs.  x1*s and x1*c are exact in fp64, so
// fma(x0, c, -(x1*s)) rounds x0*c - x1*s once, exactly like the two products
// followed by a rounded subtraction.
__device__ __forceinline__ void rotate_finite(float x0, float x1, double c, double s, float &y0, float &y1) {
#pragma clang fp contract(off)
    const double a = (double)x0, b = (double)x1;
    y0 = (float)__builtin_fma(a, c, -(b * s));
    y1 = (float)__builtin_fma(a, s, b * c);
}

// Rotate the pairs held in one run (NORM: eight (2i, 2i+1) pairs in A) or two
// runs (NEOX: A holds dims of the first half, B the partners) with cos/sin in
// cs/sn; na/nb receive the new codes.
template <bool NEOX, int NP>
__device__ __forceinline__ void rotate_runs(const u32x4 &wa, const u32x4 &wb, const double (&cs)[NP],
                                            const double (&sn)[NP], u32x4 &na, u32x4 &nb) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t A = wa[w], B = NEOX ? wb[w] : 0u;
        const f32x2 a01 = codes_to_f32x2<false>(A), a23 = codes_to_f32x2<true>(A);
        if (NEOX) {
            const f32x2 b01 = codes_to_f32x2<false>(B), b23 = codes_to_f32x2<true>(B);
            const float xa[4] = {a01[0], a01[1], a23[0], a23[1]};
            const float xb[4] = {b01[0], b01[1], b23[0], b23[1]};
            if (!(has_nan4(A) || has_nan4(B))) {
                float y0[4], y1[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) rotate_finite(xa[k], xb[k], cs[4 * w + k], sn[4 * w + k], y0[k], y1[k]);
                na[w] = encode4_finite(y0[0], y0[1], y0[2], y0[3]);
                nb[w] = encode4_finite(y1[0], y1[1], y1[2], y1[3]);
            } else {
                uint32_t ca = 0, cb = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t y = rotate_pair(xa[k], xb[k], cs[4 * w + k], sn[4 * w + k]);
                    ca |= (y & 0xFFu) << (8 * k);
                    cb |= ((y >> 8) & 0xFFu) << (8 * k);
                }
                na[w] = ca;
                nb[w] = cb;
            }
        } else {
            if (!has_nan4(A)) {
                float p0, q0, p1, q1;
                rotate_finite(a01[0], a01[1], cs[2 * w], sn[2 * w], p0, q0);
                rotate_finite(a23[0], a23[1], cs[2 * w + 1], sn[2 * w + 1], p1, q1);
                na[w] = encode4_finite(p0, q0, p1, q1);
            } else {
                const uint32_t y0 = rotate_pair(a01[0], a01[1], cs[2 * w], sn[2 * w]);
                const uint32_t y1 = rotate_pair(a23[0], a23[1], cs[2 * w + 1], sn[2 * w + 1]);
                na[w] = (y0 & 0xFFFFu) | (y1 << 16);
            }
        }
    }
}

// Run path.  Thread g works on run r = g mod RP (RP: runs per row rounded up to
// a power of two; lanes with r >= runs idle) of the (slot, head) items
// j = g / RP, g / RP + J, ... with J = grid threads / RP, so its rotary pairs
// never change: their cos/sin are held in registers.  U items are loaded per
// iteration (U = 1: more loads in flight per lane measured slower, as in the
// streaming-read probe).
template <bool NEOX, int U>
__global__ __launch_bounds__(kThreads) void kshift_runs(KShiftArgs a, int rp_log2) {
    constexpr int NP = NEOX ? 16 : 8;      // rotary pairs per run
    const int D = a.head_dim, H = a.kv_heads;
    const int bs_log2 = a.block_size == 32 ? 5 : 4;
    const int runs = NEOX ? a.rot_dim / 32 : a.rot_dim / 16;
    const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int r = (int)(g & ((1 << rp_log2) - 1));
    const int64_t nj = a.n_slots * H;
    int64_t j = g >> rp_log2;
    if (r >= runs || j >= nj) return;
    const int64_t jstep = ((int64_t)gridDim.x * kThreads) >> rp_log2;
    const bool small = nj <= 0x7FFFFFFF;

    double cs[NP], sn[NP];
    const int p0 = NEOX ? 16 * r : 8 * r;
#pragma unroll
    for (int k = 0; k < NP; ++k) {
        cs[k] = (double)a.cos_t[p0 + k];
        sn[k] = (double)a.sin_t[p0 + k];
    }
    const int da = 16 * r;                      // first byte run: dims [16r, 16r+16)
    const int db = da + a.rot_dim / 2;          // NEOX partner run

    for (; j < nj; j += U * jstep) {
        int64_t oa[U], ob[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t jj = j + u * jstep;
            oa[u] = -1;
            if (jj < nj) {
                int64_t si;
                int h;
                if (small) {
                    si = (uint32_t)jj / (uint32_t)H;
                    h = (int)((uint32_t)jj - (uint32_t)si * (uint32_t)H);
                } else {
                    si = jj / H;
                    h = (int)(jj - si * H);
                }
                const int64_t slot = a.slots[si];
                if (slot >= 0 && slot < a.pool_slots) {   // others are skipped, never written
                    const int64_t blk = slot >> bs_log2;
                    const int t = (int)(slot - (blk << bs_log2));
                    const int64_t tile = ((blk * H + h) << bs_log2) * D;
                    oa[u] = tile + k_offset(t, da, a.block_size, D);
                    ob[u] = tile + k_offset(t, db, a.block_size, D);
                }
            }
        }
        u32x4 wa[U], wb[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (oa[u] >= 0) {
                wa[u] = *reinterpret_cast<const u32x4 *>(a.k_pool + oa[u]);
                if (NEOX) wb[u] = *reinterpret_cast<const u32x4 *>(a.k_pool + ob[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (oa[u] < 0) continue;
            u32x4 na, nb;
            rotate_runs<NEOX, NP>(wa[u], wb[u], cs, sn, na, nb);
            *reinterpret_cast<u32x4 *>(a.k_pool + oa[u]) = na;
            if (NEOX) *reinterpret_cast<u32x4 *>(a.k_pool + ob[u]) = nb;
        }
    }
}

// Per-slot path, runs.  Every slot carries its own row of the cos/sin table
// (a.rows[si] into a.table, [row][pair][cos, sin] fp32).  Lane l of a wave
// works on run r = l mod RP of the wave's span of slots, 64 / RP slots per
// iteration; it loads its run's cos/sin (16-byte loads of the interleaved row)
// only when the slot's row differs from the previous slot's, and rotates that
// run in every kv-head, one head after the other (two heads in flight, or
// (slot, head) items with a table load each, measured slower).
template <bool NEOX>
__global__ __launch_bounds__(kThreads) void kshift_slot_runs(KShiftArgs a, int rp_log2) {
    constexpr int NP = NEOX ? 16 : 8;
    const int D = a.head_dim, H = a.kv_heads;
    const int bs_log2 = a.block_size == 32 ? 5 : 4;
    const int runs = NEOX ? a.rot_dim / 32 : a.rot_dim / 16;
    const int half = a.rot_dim / 2;
    const int lane = threadIdx.x & 63;
    const int r = lane & ((1 << rp_log2) - 1);
    if (r >= runs) return;
    // Each wave walks one contiguous span of the slot list, 64 / RP slots per
    // iteration (its lanes cover those slots' runs, so accesses stay as
    // coalesced as a grid stride).  A lane's successive slots are then close in
    // the list, where neighbouring slots usually share a delta: the lane keeps
    // its row's cos/sin (widened to fp64) until the row index changes.
    const int spw = 64 >> rp_log2;
    const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
    const int64_t wave_id = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
    const int64_t per_wave = (a.n_slots + nwaves - 1) / nwaves;
    const int64_t span = (per_wave + spw - 1) / spw * spw;
    const int64_t s_end = min(a.n_slots, (wave_id + 1) * span);
    const int p0 = NEOX ? 16 * r : 8 * r;
    const int da = 16 * r;
    const int db = da + half;
    double cs[NP], sn[NP];
    int32_t cached = -1;
    for (int64_t si = wave_id * span + (lane >> rp_log2); si < s_end; si += spw) {
        const int64_t slot = a.slots[si];
        const int32_t row = a.rows[si];
        if (slot < 0 || slot >= a.pool_slots || row < 0 || row >= a.n_rows) continue;
        if (row != cached) {
            const f32x4 *tp = reinterpret_cast<const f32x4 *>(a.table + ((int64_t)row * half + p0) * 2);
#pragma unroll
            for (int k = 0; k < NP / 2; ++k) {
                const f32x4 v = tp[k];
                cs[2 * k] = (double)v[0];
                sn[2 * k] = (double)v[1];
                cs[2 * k + 1] = (double)v[2];
                sn[2 * k + 1] = (double)v[3];
            }
            cached = row;
        }
        const int64_t blk = slot >> bs_log2;
        const int t = (int)(slot - (blk << bs_log2));
        const int64_t oa0 = k_offset(t, da, a.block_size, D), ob0 = k_offset(t, db, a.block_size, D);
        const int64_t head_bytes = ((int64_t)1 << bs_log2) * D;
        uint8_t *base = a.k_pool + blk * H * head_bytes;
        for (int h = 0; h < H; ++h) {
            uint8_t *t0 = base + h * head_bytes;
            const u32x4 wa = *reinterpret_cast<const u32x4 *>(t0 + oa0);
            u32x4 wb = {0u, 0u, 0u, 0u};
            if (NEOX) wb = *reinterpret_cast<const u32x4 *>(t0 + ob0);
            u32x4 na, nb;
            rotate_runs<NEOX, NP>(wa, wb, cs, sn, na, nb);
            *reinterpret_cast<u32x4 *>(t0 + oa0) = na;
            if (NEOX) *reinterpret_cast<u32x4 *>(t0 + ob0) = nb;
        }
    }
}

// Per-slot path, one pair per thread (rotary widths the run path does not cover).
__global__ __launch_bounds__(kThreads) void kshift_slot_pairs(KShiftArgs a) {
    const int D = a.head_dim, BS = a.block_size, H = a.kv_heads;
    const int half = a.rot_dim / 2;
    const int64_t item = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t total = a.n_slots * H * half;
    if (item >= total) return;
    const int p = (int)(item % half);
    const int h = (int)((item / half) % H);
    const int64_t si = item / ((int64_t)half * H);
    const int64_t slot = a.slots[si];
    const int32_t row = a.rows[si];
    if (slot < 0 || slot >= a.pool_slots || row < 0 || row >= a.n_rows) return;
    const f32x2 cs = *reinterpret_cast<const f32x2 *>(a.table + ((int64_t)row * half + p) * 2);
    const int64_t blk = slot / BS;
    const int t = (int)(slot - blk * BS);
    uint8_t *tile = a.k_pool + (blk * H + h) * (int64_t)BS * D;
    const int d0 = a.neox ? p : 2 * p;
    const int d1 = a.neox ? p + half : 2 * p + 1;
    uint8_t *b0 = tile + k_offset(t, d0, BS, D);
    uint8_t *b1 = tile + k_offset(t, d1, BS, D);
    const f32x2 x = codes_to_f32x2<false>((uint32_t)*b0 | ((uint32_t)*b1 << 8));
    const uint32_t y = rotate_pair(x[0], x[1], (double)cs[0], (double)cs[1]);
    *b0 = (uint8_t)(y & 0xFF);
    *b1 = (uint8_t)(y >> 8);
}

// ---------------------------------------------------------------- bf16 K pools
// The bf16 twin of the cache keeps K as bf16 values at the same element
// positions.  A pair rotates as above (fp64, products exact: 8-bit by 24-bit
// significands) and each result is rounded to fp32, then to the nearest bf16;
// a pair holding a NaN becomes the quiet NaN 0x7FC0 in both places.

__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two bf16 values (x0 in bits 0-15, x1 in 16-31 of the result) from a pair.
__device__ __forceinline__ uint32_t rotate_bf16(uint32_t b0, uint32_t b1, double c, double s) {
#pragma clang fp contract(off)
    const float x0 = __uint_as_float(b0 << 16), x1 = __uint_as_float(b1 << 16);
    if (__builtin_isnan(x0) || __builtin_isnan(x1)) return 0x7FC07FC0u;
    const double a = (double)x0, b = (double)x1;
    const float y0 = (float)__builtin_fma(a, c, -(b * s));
    const float y1 = (float)__builtin_fma(a, s, b * c);
    return bf16_rne(y0) | (bf16_rne(y1) << 16);
}

// Run path for bf16: a thread rotates the pairs of one 16-byte run (eight
// elements; NEOX: eight pairs with the partner run rot/2 further, NORM: four
// (2i, 2i+1) pairs) in every (slot, head) item j = g / RP, g / RP + J, ...
// With one delta its cos/sin stay in registers; with a table row per slot
// they are loaded per item.
template <bool NEOX, bool PER_SLOT>
__global__ __launch_bounds__(kThreads) void kshift_bf16_runs(KShiftArgs a, int rp_log2) {
    constexpr int NP = NEOX ? 8 : 4;
    const int D = a.head_dim, H = a.kv_heads;
    const int half = a.rot_dim / 2;
    const int runs = NEOX ? a.rot_dim / 16 : a.rot_dim / 8;
    const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int r = (int)(g & ((1 << rp_log2) - 1));
    const int64_t nj = a.n_slots * H;
    int64_t j = g >> rp_log2;
    if (r >= runs || j >= nj) return;
    const int64_t jstep = ((int64_t)gridDim.x * kThreads) >> rp_log2;
    const int p0 = NEOX ? 8 * r : 4 * r;
    const int da = 8 * r, db = da + half;
    double cs[NP], sn[NP];
    if (!PER_SLOT) {
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            cs[k] = (double)a.cos_t[p0 + k];
            sn[k] = (double)a.sin_t[p0 + k];
        }
    }
    uint16_t *kp = reinterpret_cast<uint16_t *>(a.k_pool);
    for (; j < nj; j += jstep) {
        const int64_t si = j / H;
        const int h = (int)(j - si * H);
        const int64_t slot = a.slots[si];
        if (slot < 0 || slot >= a.pool_slots) continue;
        if (PER_SLOT) {
            const int32_t row = a.rows[si];
            if (row < 0 || row >= a.n_rows) continue;
            const f32x4 *tp = reinterpret_cast<const f32x4 *>(a.table + ((int64_t)row * half + p0) * 2);
#pragma unroll
            for (int k = 0; k < NP / 2; ++k) {
                const f32x4 v = tp[k];
                cs[2 * k] = (double)v[0];
                sn[2 * k] = (double)v[1];
                cs[2 * k + 1] = (double)v[2];
                sn[2 * k + 1] = (double)v[3];
            }
        }
        const int64_t blk = slot / a.block_size;
        const int t = (int)(slot - blk * a.block_size);
        uint16_t *tile = kp + (blk * H + h) * (int64_t)a.block_size * D;
        u32x4 *pa = reinterpret_cast<u32x4 *>(tile + k_offset(t, da, a.block_size, D));
        const u32x4 A = *pa;
        if (NEOX) {
            u32x4 *pb = reinterpret_cast<u32x4 *>(tile + k_offset(t, db, a.block_size, D));
            const u32x4 B = *pb;
            u32x4 na, nb;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t y0 = rotate_bf16(A[w] & 0xFFFFu, B[w] & 0xFFFFu, cs[2 * w], sn[2 * w]);
                const uint32_t y1 = rotate_bf16(A[w] >> 16, B[w] >> 16, cs[2 * w + 1], sn[2 * w + 1]);
                na[w] = (y0 & 0xFFFFu) | (y1 << 16);
                nb[w] = (y0 >> 16) | (y1 & 0xFFFF0000u);
            }
            *pa = na;
            *pb = nb;
        } else {
            u32x4 na;
#pragma unroll
            for (int w = 0; w < 4; ++w) na[w] = rotate_bf16(A[w] & 0xFFFFu, A[w] >> 16, cs[w], sn[w]);
            *pa = na;
        }
    }
}

// One pair per thread for bf16 (rotary widths the run path does not cover).
template <bool PER_SLOT>
__global__ __launch_bounds__(kThreads) void kshift_bf16_pairs(KShiftArgs a) {
    const int D = a.head_dim, BS = a.block_size, H = a.kv_heads;
    const int half = a.rot_dim / 2;
    const int64_t item = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t total = a.n_slots * H * half;
    if (item >= total) return;
    const int p = (int)(item % half);
    const int h = (int)((item / half) % H);
    const int64_t si = item / ((int64_t)half * H);
    const int64_t slot = a.slots[si];
    if (slot < 0 || slot >= a.pool_slots) return;
    float c, s;
    if (PER_SLOT) {
        const int32_t row = a.rows[si];
        if (row < 0 || row >= a.n_rows) return;
        const f32x2 v = *reinterpret_cast<const f32x2 *>(a.table + ((int64_t)row * half + p) * 2);
        c = v[0];
        s = v[1];
    } else {
        c = a.cos_t[p];
        s = a.sin_t[p];
    }
    const int64_t blk = slot / BS;
    const int t = (int)(slot - blk * BS);
    uint16_t *tile = reinterpret_cast<uint16_t *>(a.k_pool) + (blk * H + h) * (int64_t)BS * D;
    uint16_t *e0 = tile + k_offset(t, a.neox ? p : 2 * p, BS, D);
    uint16_t *e1 = tile + k_offset(t, a.neox ? p + half : 2 * p + 1, BS, D);
    const uint32_t y = rotate_bf16(*e0, *e1, (double)c, (double)s);
    *e0 = (uint16_t)(y & 0xFFFFu);
    *e1 = (uint16_t)(y >> 16);
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
    const uint32_t y = rotate_pair(x[0], x[1], (double)tab.c[p], (double)tab.s[p]);
    *b0 = (uint8_t)(y & 0xFF);
    *b1 = (uint8_t)(y >> 8);
}

}  // namespace

static hipError_t launch_kshift_bf16(const KShiftArgs &a, hipStream_t stream) {
    const bool per_slot = a.rows != nullptr;
    const bool runs = a.neox ? (a.rot_dim % 16 == 0) : (a.rot_dim % 8 == 0);
    if (runs) {
        const int per_row = a.neox ? a.rot_dim / 16 : a.rot_dim / 8;
        int rp_log2 = 0;
        while ((1 << rp_log2) < per_row) ++rp_log2;
        int64_t wgs = (((a.n_slots * a.kv_heads) << rp_log2) + kThreads - 1) / kThreads;
        if (wgs > kRunsMaxWgs) wgs = kRunsMaxWgs;
        if (wgs < 1) wgs = 1;
        const dim3 grid((unsigned)wgs), block(kThreads);
        if (a.neox && per_slot) hipLaunchKernelGGL((kshift_bf16_runs<true, true>), grid, block, 0, stream, a, rp_log2);
        else if (a.neox) hipLaunchKernelGGL((kshift_bf16_runs<true, false>), grid, block, 0, stream, a, rp_log2);
        else if (per_slot) hipLaunchKernelGGL((kshift_bf16_runs<false, true>), grid, block, 0, stream, a, rp_log2);
        else hipLaunchKernelGGL((kshift_bf16_runs<false, false>), grid, block, 0, stream, a, rp_log2);
        return hipGetLastError();
    }
    const int64_t total = a.n_slots * a.kv_heads * (a.rot_dim / 2);
    const int64_t wgs = (total + kThreads - 1) / kThreads;
    if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (per_slot) hipLaunchKernelGGL(kshift_bf16_pairs<true>, dim3((unsigned)wgs), dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL(kshift_bf16_pairs<false>, dim3((unsigned)wgs), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_kshift(const KShiftArgs &a, hipStream_t stream) {
    if (a.k_eb == 2) return launch_kshift_bf16(a, stream);
    const bool runs = a.neox ? (a.rot_dim % 32 == 0) : (a.rot_dim % 16 == 0);
    if (a.rows) {
        if (runs) {
            const int per_row = a.neox ? a.rot_dim / 32 : a.rot_dim / 16;
            int rp_log2 = 0;
            while ((1 << rp_log2) < per_row) ++rp_log2;
            int64_t wgs = ((a.n_slots << rp_log2) + kThreads - 1) / kThreads;
            if (wgs > kRunsMaxWgs) wgs = kRunsMaxWgs;
            if (wgs < 1) wgs = 1;
            if (a.neox)
                hipLaunchKernelGGL(kshift_slot_runs<true>, dim3((unsigned)wgs), dim3(kThreads), 0, stream, a,
                                   rp_log2);
            else
                hipLaunchKernelGGL(kshift_slot_runs<false>, dim3((unsigned)wgs), dim3(kThreads), 0, stream, a,
                                   rp_log2);
            return hipGetLastError();
        }
        const int64_t total = a.n_slots * a.kv_heads * (a.rot_dim / 2);
        const int64_t wgs = (total + kThreads - 1) / kThreads;
        if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
        hipLaunchKernelGGL(kshift_slot_pairs, dim3((unsigned)wgs), dim3(kThreads), 0, stream, a);
        return hipGetLastError();
    }
    if (runs) {
        const int per_row = a.neox ? a.rot_dim / 32 : a.rot_dim / 16;
        int rp_log2 = 0;
        while ((1 << rp_log2) < per_row) ++rp_log2;
        const int64_t threads = (a.n_slots * a.kv_heads) << rp_log2;
        int64_t wgs = (threads + kThreads - 1) / kThreads;
        if (wgs > kRunsMaxWgs) wgs = kRunsMaxWgs;     // then each thread loops
        if (wgs < 1) wgs = 1;
        if (a.neox)
            hipLaunchKernelGGL((kshift_runs<true, kRunsUnroll>), dim3((unsigned)wgs), dim3(kThreads), 0, stream,
                               a, rp_log2);
        else
            hipLaunchKernelGGL((kshift_runs<false, kRunsUnroll>), dim3((unsigned)wgs), dim3(kThreads), 0, stream,
                               a, rp_log2);
        return hipGetLastError();
    }
    const int64_t total = a.n_slots * a.kv_heads * (a.rot_dim / 2);
    const int64_t wgs = (total + kThreads - 1) / kThreads;
    if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kshift_pairs, dim3((unsigned)wgs), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kvf8
