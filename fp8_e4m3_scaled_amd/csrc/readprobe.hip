// kvf8_read_probe: a plain streaming read of a device buffer, the achievable
// read-bandwidth ceiling that the cache kernels are measured beside.
//
// Every workgroup walks the buffer's 16-byte words grid-stride (one load per
// lane per iteration: more in flight measured slower), XORs everything it
// read into one 32-bit word and
// writes it to out[blockIdx.x]; the XOR of all out words is the XOR of every
// 32-bit word of the buffer, so the result can be checked and the loads
// cannot be dropped.

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

}  // namespace

hipError_t launch_read_probe(const void *buf, int64_t bytes, uint32_t *out, int32_t n_out, hipStream_t stream) {
    hipLaunchKernelGGL(read_probe, dim3((unsigned)n_out), dim3(kThreads), 0, stream,
                       static_cast<const u32x4 *>(buf), bytes / 16, out);
    return hipGetLastError();
}

}  // namespace kvf8
