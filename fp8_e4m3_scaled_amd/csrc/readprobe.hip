// kvf8_read_probe: a plain streaming read of a device buffer, the achievable
// read-bandwidth ceiling that the cache kernels are measured beside.
//
// Every workgroup walks the buffer's 16-byte words grid-stride (one load per
// lane per iteration: more in flight measured slower), XORs everything it
// read into one 32-bit word and
// writes it to out[blockIdx.x]; the XOR of all out words is the XOR of every
// 32-bit word of the buffer, so the result can be checked and the loads
// cannot be dropped.
//
// kvf8_gather_probe: the same plain read, but of exactly the tiles a paged
// decode reads: workgroup (sequence, kv-head) walks its sequence's K and V
// tiles through the block table (block ids staged in LDS, four 16-byte loads
// in flight per lane, K tiles then V tiles) and writes their XOR.  Its rate is the ceiling of the decode's
// access pattern (scattered tiles), as opposed to a linear stream.

#include "fp8_device.hpp"
#include "internal.hpp"

namespace kvf8 {
namespace {

constexpr int kThreads = 256;

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

__global__ __launch_bounds__(kThreads) void gather_probe(GatherProbeArgs a) {
    __shared__ int32_t ids[kGatherIds];
    const int unit = blockIdx.x;
    const int seq = unit / a.kv_heads, head = unit - seq * a.kv_heads;
    const int len = a.seq_lens[seq];
    int64_t nblk = len > 0 ? (len + a.block_size - 1) / a.block_size : 0;
    if (nblk > a.max_blocks) nblk = a.max_blocks;            // as the decode: never past the table row
    const int32_t *table = a.block_tables + (int64_t)seq * a.max_blocks;
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

}  // namespace

hipError_t launch_gather_probe(const GatherProbeArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL(gather_probe, dim3((unsigned)(a.num_seqs * a.kv_heads)), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_read_probe(const void *buf, int64_t bytes, uint32_t *out, int32_t n_out, hipStream_t stream) {
    hipLaunchKernelGGL(read_probe, dim3((unsigned)n_out), dim3(kThreads), 0, stream,
                       static_cast<const u32x4 *>(buf), bytes / 16, out);
    return hipGetLastError();
}

}  // namespace kvf8
