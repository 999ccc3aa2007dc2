// kvf8_probe_read: a plain streaming read of a device buffer, the achievable
// read-bandwidth ceiling that the cache kernels are measured beside.
//
// Every workgroup walks the buffer's 16-byte words grid-stride (one load per
// lane per iteration: more in flight measured slower), XORs everything it
// read into one 32-bit word and
// writes it to out[blockIdx.x]; the XOR of all out words is the XOR of every
// 32-bit word of the buffer, so the result can be checked and the loads
// cannot be dropped.
//
// kvf8_probe_gather: the same plain read, but of exactly the tiles a paged
// decode reads: workgroup (sequence, kv-head) walks its sequence's K and V
// tiles through the block table (block ids staged in LDS, four 16-byte loads
// in flight per lane, K tiles then V tiles) and writes their XOR.  Its rate
// is the ceiling of the decode's access pattern (scattered tiles), as
// opposed to a linear stream.  kvf8_probe_gather_split gives each chunk of
// a row's table entries a workgroup of its own, as a split-K decode does.
//
// kvf8_probe_rmw: the K-shift's memory traffic with no arithmetic.  The same
// work items as the run path of the NEOX K-shift (a (slot, head) item and a
// 16-byte run r: dims [16r, 16r + 16) and their partners rot/2 further, both
// read and written in place), the same grid-stride launch, but each byte is
// only XORed with 1.  Its rate is the ceiling of the K-shift's access pattern
// through a given slot list.
//
// kvf8_probe_store_copy: the cache fill's memory traffic with no arithmetic.
// The same workgroups, pieces and loads as the store's 16-token run path
// (one workgroup per 16 input tokens bound for one aligned run of 16 slots;
// K pieces of 16 dims of a token, V pieces of 8 dims x 4 tokens), but each
// bf16 value's high byte is written where the store writes its code.  Its
// rate is the ceiling of the fill's access pattern through a given slot list.
// Measurement aids of the benchmark only, built into their own library
// (libkvf8probe.so), not into the cache library.

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "readprobe.h"

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kThreads = 256;

struct GatherArgs {
    const void *k_pool;
    const void *v_pool;
    const int32_t *block_tables;
    const int32_t *seq_lens;
    uint32_t *out;
    int64_t num_blocks;
    int32_t max_blocks;
    int32_t num_seqs;
    int32_t kv_heads;
    int32_t block_size;
    int32_t k_words_log2;    // log2 of the 16-byte words of one (block, head) tile
    int32_t v_words_log2;
    int32_t chunk_blocks;    // table entries per unit (a unit reads one chunk of one pair's row)
    int32_t chunks;          // chunks per row: ceil(max_blocks / chunk_blocks)
};

__global__ __launch_bounds__(kThreads) void read_probe(const u32x4 *buf, int64_t n16, uint32_t *out) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) acc ^= buf[i];
    uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    for (int o = 32; o > 0; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o);
    __shared__ uint32_t part[kThreads / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int w = 0; w < kThreads / 64; ++w) r ^= part[w];
        out[blockIdx.x] = r;
    }
}

constexpr int kGatherIds = 4096;   // block ids staged in LDS per pass
constexpr int kGatherUnroll = 4;   // 16-byte loads in flight per lane

// XOR of the 16-byte words of tiles ids[0..nb) of one kv-head in one pool.
__device__ __forceinline__ u32x4 gather_words(const u32x4 *pool, const int32_t *ids, int nb, int wl, int head,
                                              int heads) {
    const int64_t words = (int64_t)nb << wl;
    const int64_t mask = ((int64_t)1 << wl) - 1;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t w = threadIdx.x; w < words; w += kGatherUnroll * kThreads) {
        u32x4 x[kGatherUnroll];
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) {
            const int64_t ww = w + u * kThreads;
            x[u] = u32x4{0u, 0u, 0u, 0u};
            if (ww < words) {
                const int64_t tile = (int64_t)ids[ww >> wl] * heads + head;
                x[u] = pool[(tile << wl) + (ww & mask)];
            }
        }
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) acc ^= x[u];
    }
    return acc;
}

__global__ __launch_bounds__(kThreads) void gather_probe(GatherArgs a) {
    __shared__ int32_t ids[kGatherIds];
    const int unit = blockIdx.x;
    const int npairs = a.num_seqs * a.kv_heads;
    const int pair = unit % npairs, chunk = unit / npairs;   // chunk-major: neighbouring units, other pairs
    const int seq = pair / a.kv_heads, head = pair - seq * a.kv_heads;
    const int len = a.seq_lens[seq];
    int64_t nblk = len > 0 ? (len + a.block_size - 1) / a.block_size : 0;
    if (nblk > a.max_blocks) nblk = a.max_blocks;            // as the decode: never past the table row
    const int64_t first = (int64_t)chunk * a.chunk_blocks;
    nblk = nblk > first ? nblk - first : 0;
    if (nblk > a.chunk_blocks) nblk = a.chunk_blocks;
    const int32_t *table = a.block_tables + (int64_t)seq * a.max_blocks + first;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t b0 = 0; b0 < nblk; b0 += kGatherIds) {
        const int nb = (int)(nblk - b0 < kGatherIds ? nblk - b0 : kGatherIds);
        __syncthreads();
        for (int i = threadIdx.x; i < nb; i += kThreads) {
            const uint32_t id = (uint32_t)table[b0 + i];          // out-of-pool ids read the last block
            ids[i] = (int32_t)(id < a.num_blocks ? id : (uint32_t)(a.num_blocks - 1));
        }
        __syncthreads();
        acc ^= gather_words(reinterpret_cast<const u32x4 *>(a.k_pool), ids, nb, a.k_words_log2, head, a.kv_heads);
        acc ^= gather_words(reinterpret_cast<const u32x4 *>(a.v_pool), ids, nb, a.v_words_log2, head, a.kv_heads);
    }
    uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    for (int o = 32; o > 0; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o);
    __shared__ uint32_t part[kThreads / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int w = 0; w < kThreads / 64; ++w) r ^= part[w];
        a.out[unit] = r;
    }
}

constexpr int64_t kRmwMaxWgs = 4096;     // as the K-shift's run path: 16 workgroups per CU, then a grid stride

struct RmwArgs {
    uint8_t *k_pool;
    const int64_t *slots;
    int64_t n_slots;
    int64_t pool_slots;
    int32_t kv_heads;
    int32_t head_dim;
    int32_t block_size;
    int32_t runs;            // 16-byte runs of the rotated first half: rot_dim / 32
    int32_t half;            // rot_dim / 2: byte distance of a run's partner
    int32_t rp_log2;         // runs rounded up to a power of two
};

__device__ __forceinline__ int64_t k_byte(int t, int d, int BS, int D) {
    const int q = D >> 2;
    return ((int64_t)(d / q) * BS + t) * q + d % q;
}

__global__ __launch_bounds__(kThreads) void rmw_probe(RmwArgs a) {
    const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int r = (int)(g & ((1 << a.rp_log2) - 1));
    const int64_t nj = a.n_slots * a.kv_heads;
    if (r >= a.runs) return;
    const int bs_log2 = a.block_size == 32 ? 5 : 4;
    const int64_t jstep = ((int64_t)gridDim.x * kThreads) >> a.rp_log2;
    for (int64_t j = g >> a.rp_log2; j < nj; j += jstep) {
        int64_t si;
        int h;
        if (nj <= 0x7FFFFFFF) {                 // 32-bit division, as the K-shift
            si = (uint32_t)j / (uint32_t)a.kv_heads;
            h = (int)((uint32_t)j - (uint32_t)si * (uint32_t)a.kv_heads);
        } else {
            si = j / a.kv_heads;
            h = (int)(j - si * a.kv_heads);
        }
        const int64_t slot = a.slots[si];
        if (slot < 0 || slot >= a.pool_slots) continue;
        const int64_t blk = slot >> bs_log2;
        const int t = (int)(slot - (blk << bs_log2));
        uint8_t *tile = a.k_pool + ((blk * a.kv_heads + h) << bs_log2) * a.head_dim;
        u32x4 *pa = reinterpret_cast<u32x4 *>(tile + k_byte(t, 16 * r, a.block_size, a.head_dim));
        u32x4 *pb = reinterpret_cast<u32x4 *>(tile + k_byte(t, 16 * r + a.half, a.block_size, a.head_dim));
        const u32x4 va = *pa, vb = *pb;
        *pa = va ^ 0x01010101u;
        *pb = vb ^ 0x01010101u;
    }
}

struct CopyArgs {
    const uint16_t *k;
    const uint16_t *v;
    int64_t k_stride;        // elements between consecutive tokens' rows
    int64_t v_stride;
    const int64_t *slots;
    int64_t num_tokens;
    int64_t pool_slots;
    uint8_t *k_pool;
    uint8_t *v_pool;
    int32_t kv_heads;
    int32_t head_dim;
    int32_t block_size;
};

// High bytes of four bf16 values (two words): bytes 1, 3 of p0, then of p1.
__device__ __forceinline__ uint32_t hi_bytes(uint32_t p0, uint32_t p1) {
    return __builtin_amdgcn_perm(p1, p0, 0x07050301u);
}

__global__ __launch_bounds__(kThreads) void store_copy_probe(CopyArgs a) {
    const int64_t tok0 = (int64_t)blockIdx.x * 16;
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
    if (!s_run) return;                          // only whole aligned 16-token runs are copied
    const int D = a.head_dim, H = a.kv_heads, BS = a.block_size;
    const int Q4 = D >> 2;
    const int64_t tile = (int64_t)BS * D;
    const int64_t blk = s_first / BS;
    const int t0 = (int)(s_first - blk * BS);
    const int np = D >> 6;
    const int kper = 16 * (D >> 4);
    const int vper = 4 * (D >> 3);
    const int k_items = H * kper, v_items = H * vper;
    for (int base = 0; base < k_items; base += 4 * kThreads) {
        u32x4 lo[4], hi[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int it = base + u * kThreads + threadIdx.x;
            if (it < k_items) {
                const int h = it / kper;
                const int r = it - h * kper;
                const int j = r % np, t = (r / np) & 15, q = r / (16 * np);
                const u32x4 *src =
                    reinterpret_cast<const u32x4 *>(a.k + (tok0 + t) * a.k_stride + (int64_t)h * D + q * Q4 + j * 16);
                lo[u] = src[0];
                hi[u] = src[1];
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int it = base + u * kThreads + threadIdx.x;
            if (it < k_items) {
                const int h = it / kper;
                const int r = it - h * kper;
                const int j = r % np, t = (r / np) & 15, q = r / (16 * np);
                const int64_t off = (blk * H + h) * tile + (int64_t)(q * BS + t0 + t) * Q4 + j * 16;
                const u32x4 c = {hi_bytes(lo[u][0], lo[u][1]), hi_bytes(lo[u][2], lo[u][3]),
                                 hi_bytes(hi[u][0], hi[u][1]), hi_bytes(hi[u][2], hi[u][3])};
                *reinterpret_cast<u32x4 *>(a.k_pool + off) = c;
            }
        }
    }
    for (int base = 0; base < v_items; base += 2 * kThreads) {
        u32x4 x[2][4];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int it = base + u * kThreads + threadIdx.x;
            if (it < v_items) {
                const int h = it / vper;
                const int r = it - h * vper;
                const int g = r / (D >> 3), o = r - g * (D >> 3);
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    x[u][k] = *reinterpret_cast<const u32x4 *>(a.v + (tok0 + 4 * g + k) * a.v_stride + (int64_t)h * D +
                                                               8 * o);
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int it = base + u * kThreads + threadIdx.x;
            if (it < v_items) {
                const int h = it / vper;
                const int r = it - h * vper;
                const int g = r / (D >> 3), o = r - g * (D >> 3);
                u32x4 out[2];
#pragma unroll
                for (int j = 0; j < 8; ++j) {           // dim 8o + j: four tokens' high bytes
                    const int w = j >> 1;
                    const uint32_t sel = (j & 1) ? 0x07030703u : 0x05010501u;
                    const uint32_t lo = __builtin_amdgcn_perm(x[u][1][w], x[u][0][w], sel);
                    const uint32_t hi = __builtin_amdgcn_perm(x[u][3][w], x[u][2][w], sel);
                    out[j >> 2][j & 3] = (lo & 0xFFFFu) | (hi << 16);
                }
                u32x4 *dst = reinterpret_cast<u32x4 *>(a.v_pool + (blk * H + h) * tile +
                                                       ((int64_t)(t0 / 4 + g) * D + 8 * o) * 4);
                dst[0] = out[0];
                dst[1] = out[1];
            }
        }
    }
}

thread_local std::string g_last_error;

int fail(const char *fmt, ...) {
    char buf[256];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return 1;
}

int launched(const char *what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        fail("%s: %s", what, hipGetErrorString(e));
        return 6;
    }
    g_last_error.clear();
    return 0;
}

}  // namespace

extern "C" {

const char *kvf8_probe_last_error(void) { return g_last_error.c_str(); }

int kvf8_probe_read(const void *buf, size_t bytes, uint32_t *out_words, int32_t n_out, void *stream) {
    if (bytes == 0) {
        g_last_error.clear();
        return 0;
    }
    if (!buf || !out_words) return fail("buf and out_words must be non-NULL");
    if ((reinterpret_cast<uintptr_t>(buf) % 16) != 0 || bytes % 16 != 0)
        return fail("buf must be 16-byte aligned and bytes a multiple of 16");
    if (n_out < 1 || n_out > (1 << 20)) return fail("n_out must be in [1, 2^20]");
    hipLaunchKernelGGL(read_probe, dim3((unsigned)n_out), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4 *>(buf), (int64_t)(bytes / 16), out_words);
    return launched("kvf8_probe_read launch");
}

int kvf8_probe_gather_split(const void *k_pool, const void *v_pool, int64_t num_blocks, int32_t num_kv_heads,
                            int32_t block_size, int32_t head_dim, int32_t k_elem_bytes, int32_t v_elem_bytes,
                            const int32_t *block_tables, int32_t max_blocks, const int32_t *seq_lens, int32_t num_seqs,
                            int32_t chunk_blocks, uint32_t *out_words, void *stream) {
    if (chunk_blocks <= 0) return fail("chunk_blocks must be positive");
    if (num_seqs < 0 || max_blocks < 0) return fail("num_seqs and max_blocks must be >= 0");
    if (num_blocks <= 0 || num_kv_heads <= 0) return fail("num_blocks and num_kv_heads must be positive");
    if ((block_size != 16 && block_size != 32) || (head_dim != 64 && head_dim != 128 && head_dim != 256))
        return fail("block_size must be 16 or 32 and head_dim 64, 128 or 256");
    if ((k_elem_bytes != 1 && k_elem_bytes != 2) || (v_elem_bytes != 1 && v_elem_bytes != 2))
        return fail("element bytes must be 1 or 2");
    if (num_seqs == 0) {
        g_last_error.clear();
        return 0;
    }
    if (!k_pool || !v_pool || !block_tables || !seq_lens || !out_words)
        return fail("pools, block_tables, seq_lens and out_words must be non-NULL");
    const int64_t chunks = max_blocks > 0 ? ((int64_t)max_blocks + chunk_blocks - 1) / chunk_blocks : 1;
    if ((int64_t)num_seqs * num_kv_heads * chunks > 0x7FFFFFFF) return fail("too many units");
    auto words_log2 = [&](int eb) {
        const int64_t words = (int64_t)block_size * head_dim * eb / 16;
        int l = 0;
        while ((int64_t(1) << l) < words) ++l;
        return l;
    };
    GatherArgs a{};
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.out = out_words;
    a.num_blocks = num_blocks;
    a.max_blocks = max_blocks;
    a.num_seqs = num_seqs;
    a.kv_heads = num_kv_heads;
    a.block_size = block_size;
    a.k_words_log2 = words_log2(k_elem_bytes);
    a.v_words_log2 = words_log2(v_elem_bytes);
    a.chunk_blocks = chunk_blocks;
    a.chunks = (int32_t)chunks;
    hipLaunchKernelGGL(gather_probe, dim3((unsigned)((int64_t)num_seqs * num_kv_heads * chunks)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), a);
    return launched("kvf8_probe_gather launch");
}

int kvf8_probe_gather(const void *k_pool, const void *v_pool, int64_t num_blocks, int32_t num_kv_heads,
                      int32_t block_size, int32_t head_dim, int32_t k_elem_bytes, int32_t v_elem_bytes,
                      const int32_t *block_tables, int32_t max_blocks, const int32_t *seq_lens, int32_t num_seqs,
                      uint32_t *out_words, void *stream) {
    return kvf8_probe_gather_split(k_pool, v_pool, num_blocks, num_kv_heads, block_size, head_dim, k_elem_bytes,
                                   v_elem_bytes, block_tables, max_blocks, seq_lens, num_seqs,
                                   max_blocks > 0 ? max_blocks : 1, out_words, stream);
}

int kvf8_probe_rmw(void *k_pool, int64_t num_blocks, int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                   int32_t rot_dim, const int64_t *slots, int64_t n_slots, void *stream) {
    if (num_blocks <= 0 || num_kv_heads <= 0) return fail("num_blocks and num_kv_heads must be positive");
    if ((block_size != 16 && block_size != 32) || (head_dim != 64 && head_dim != 128 && head_dim != 256))
        return fail("block_size must be 16 or 32 and head_dim 64, 128 or 256");
    if (rot_dim < 32 || rot_dim > head_dim || rot_dim % 32 != 0)
        return fail("rot_dim must be a multiple of 32 in [32, head_dim]");
    if (n_slots < 0) return fail("n_slots must be >= 0");
    if (n_slots == 0) {
        g_last_error.clear();
        return 0;
    }
    if (!k_pool || !slots) return fail("k_pool and slots must be non-NULL");
    if (n_slots > (int64_t(1) << 40) / num_kv_heads) return fail("too many slots");
    RmwArgs a{};
    a.k_pool = static_cast<uint8_t *>(k_pool);
    a.slots = slots;
    a.n_slots = n_slots;
    a.pool_slots = num_blocks * block_size;
    a.kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.block_size = block_size;
    a.runs = rot_dim / 32;
    a.half = rot_dim / 2;
    while ((1 << a.rp_log2) < a.runs) ++a.rp_log2;
    int64_t wgs = (((n_slots * num_kv_heads) << a.rp_log2) + kThreads - 1) / kThreads;
    if (wgs > kRmwMaxWgs) wgs = kRmwMaxWgs;
    hipLaunchKernelGGL(rmw_probe, dim3((unsigned)wgs), dim3(kThreads), 0, static_cast<hipStream_t>(stream), a);
    return launched("kvf8_probe_rmw launch");
}

int kvf8_probe_store_copy(const uint16_t *k, const uint16_t *v, int64_t k_stride, int64_t v_stride,
                          const int64_t *slots, int64_t num_tokens, void *k_pool, void *v_pool, int64_t num_blocks,
                          int32_t num_kv_heads, int32_t block_size, int32_t head_dim, void *stream) {
    if (num_blocks <= 0 || num_kv_heads <= 0) return fail("num_blocks and num_kv_heads must be positive");
    if ((block_size != 16 && block_size != 32) || (head_dim != 64 && head_dim != 128 && head_dim != 256))
        return fail("block_size must be 16 or 32 and head_dim 64, 128 or 256");
    if (num_tokens < 0) return fail("num_tokens must be >= 0");
    const int64_t row = (int64_t)num_kv_heads * head_dim;
    if (k_stride < row || v_stride < row) return fail("token strides must be >= num_kv_heads * head_dim");
    if (k_stride % 8 != 0 || v_stride % 8 != 0) return fail("token strides must be multiples of 8 elements");
    if (num_tokens == 0) {
        g_last_error.clear();
        return 0;
    }
    if (!k || !v || !slots || !k_pool || !v_pool) return fail("k, v, slots and pools must be non-NULL");
    if ((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(k_pool) |
         reinterpret_cast<uintptr_t>(v_pool)) % 16 != 0)
        return fail("k, v and the pools must be 16-byte aligned");
    const int64_t wgs = (num_tokens + 15) / 16;
    if (wgs > 0x7FFFFFFF) return fail("too many tokens");
    CopyArgs a{};
    a.k = k;
    a.v = v;
    a.k_stride = k_stride;
    a.v_stride = v_stride;
    a.slots = slots;
    a.num_tokens = num_tokens;
    a.pool_slots = num_blocks * block_size;
    a.k_pool = static_cast<uint8_t *>(k_pool);
    a.v_pool = static_cast<uint8_t *>(v_pool);
    a.kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.block_size = block_size;
    hipLaunchKernelGGL(store_copy_probe, dim3((unsigned)wgs), dim3(kThreads), 0, static_cast<hipStream_t>(stream), a);
    return launched("kvf8_probe_store_copy launch");
}

}  // extern "C"
