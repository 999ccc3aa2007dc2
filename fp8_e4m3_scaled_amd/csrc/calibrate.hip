// kv_calibrate_scales: per-tensor scales from the data.  A running absolute
// maximum of bf16 K and V tensors, then s = amax / 448 in fp32 (correctly
// rounded) or rounded on to the nearest-even bf16, so that the largest
// magnitude lands on E4M3's largest finite value.  The pages use this
// amax / 448 rule for their benchmark tensors and leave calibration at run
// time unbuilt (vllm.cpp PR #1641, "Unreached and owed"); 448 is the
// saturation bound of ggml_fp32_to_f8_e4m3 (git.wylab.me osimons/ocp_fp8_kv).
//
// amax pass: HBM-bound, 2 bytes read per element.  Every lane walks 16-byte
// runs (8 elements) of its tensor grid-stride, one load in flight per lane as
// in the streaming-read probe.  A bf16 magnitude, its bits with the sign
// cleared, orders like an unsigned 15-bit integer for every finite and
// infinite value, and every NaN pattern sorts above infinity; so the lane
// keeps a packed 16-bit integer maximum (four v_pk_max_u16 per run) and the
// workgroup's result, widened to fp32 bits (NaN made the quiet 0x7FC00000),
// goes to the running maximum with one unsigned atomic max: for non-negative
// fp32 bit patterns, unsigned order is value order and the quiet NaN sorts
// above +inf.
//
// scale pass: one wave; lanes 0 and 1 turn the K and V maxima into scales.

#include "fp8_device.hpp"
#include "internal.hpp"

namespace kvf8 {
namespace {

constexpr int kThreads = 256;
constexpr uint32_t kQuietNaN = 0x7FC00000u;

typedef __attribute__((ext_vector_type(8))) uint16_t u16x8;

__global__ __launch_bounds__(kThreads) void amax_kernel(CalibArgs a) {
    const int side = a.side[blockIdx.y];
    const uint16_t *x = a.x[side];
    const int64_t row_stride = a.stride[side];
    const int64_t cpr = a.runs_per_row;
    // (row, run) of this lane's first run, and the grid stride split the same way
    const int64_t first = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t step = (int64_t)gridDim.x * kThreads;
    int64_t row = first / cpr, col = first % cpr;
    const int64_t step_rows = step / cpr, step_cols = step % cpr;

    u16x8 acc = {0, 0, 0, 0, 0, 0, 0, 0};
    const u32x4 mask = {0x7FFF7FFFu, 0x7FFF7FFFu, 0x7FFF7FFFu, 0x7FFF7FFFu};
    while (row < a.rows) {
        const u32x4 w = *reinterpret_cast<const u32x4 *>(x + row * row_stride + col * 8);
        acc = __builtin_elementwise_max(acc, __builtin_bit_cast(u16x8, w & mask));
        row += step_rows;
        col += step_cols;
        if (col >= cpr) {
            col -= cpr;
            ++row;
        }
    }
    uint32_t m = acc[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) m = m > acc[i] ? m : (uint32_t)acc[i];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t n = (uint32_t)__shfl_xor((int)m, o);
        m = m > n ? m : n;
    }
    __shared__ uint32_t part[kThreads / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = part[0];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) r = r > part[w] ? r : part[w];
        if (r != 0) atomicMax(a.amax + side, r > 0x7F80u ? kQuietNaN : r << 16);
    }
}

__global__ __launch_bounds__(64) void scale_kernel(const uint32_t *amax, void *out, int32_t out_bf16) {
    const int side = threadIdx.x;
    if (side >= 2) return;
    const uint32_t bits = amax[side];
    uint32_t s;
    if (bits > 0x7F800000u) {
        s = kQuietNaN;
    } else {
        s = __builtin_bit_cast(uint32_t, __fdiv_rn(__builtin_bit_cast(float, bits), 448.0f));
    }
    if (out_bf16) {
        // nearest-even bf16 of a non-NaN fp32 (the carry into the exponent
        // is the round-up, up to infinity); NaN stays the quiet NaN
        const uint16_t h = s == kQuietNaN ? (uint16_t)0x7FC0u
                                          : (uint16_t)((s + 0x7FFFu + ((s >> 16) & 1u)) >> 16);
        static_cast<uint16_t *>(out)[side] = h;
    } else {
        static_cast<uint32_t *>(out)[side] = s;
    }
}

}  // namespace

hipError_t launch_calibrate(const CalibArgs &a, int32_t sides, void *scales_out, int32_t out_bf16,
                            hipStream_t stream) {
    if (sides > 0 && a.rows > 0) {
        const int64_t runs = a.rows * a.runs_per_row;
        const int64_t want = (runs + kThreads - 1) / kThreads;
        const int64_t cap = kCalibWorkgroups / sides;
        const unsigned wgs = (unsigned)(want < cap ? want : cap);
        hipLaunchKernelGGL(amax_kernel, dim3(wgs, (unsigned)sides), dim3(kThreads), 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (scales_out) {
        hipLaunchKernelGGL(scale_kernel, dim3(1), dim3(64), 0, stream,
                           a.amax, scales_out, out_bf16);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace kvf8
