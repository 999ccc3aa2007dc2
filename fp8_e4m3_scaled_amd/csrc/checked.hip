// Checked mode (kv_cache_set_checked): device-side validation of the index
// inputs that the fast kernels take on trust, run before the real launch.
//
// State: word 0 holds problem flags, words 1.. a bitmap with one bit per
// cache slot.  check_slots marks each in-pool slot with an atomic OR and
// flags a repeat; check_tables walks every sequence's lengths and the table
// entries those lengths use.  The host clears the state, launches a check,
// reads word 0 back and synchronizes, so a call that fails its check has
// launched nothing that writes the cache.

#include "internal.hpp"

namespace kvf8 {
namespace {

constexpr int kThreads = 256;
constexpr int64_t kMaxWgs = 4096;

__global__ __launch_bounds__(kThreads) void check_clear(uint32_t *w, int64_t n) {
    const int64_t step = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += step) w[i] = 0u;
}

__global__ __launch_bounds__(kThreads) void check_slots(const int64_t *slots, int64_t n, int64_t pool_slots,
                                                        uint32_t *w) {
    const int64_t step = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += step) {
        const int64_t s = slots[i];
        if (s < 0 || s >= pool_slots) continue;       // skipped by the operations, not an error
        const uint32_t bit = 1u << (s & 31);
        const uint32_t old = atomicOr(w + 1 + (s >> 5), bit);
        if (old & bit) atomicOr(w, kCheckRepeatedSlot);
    }
}

// One thread per sequence; entries of long rows are walked by that thread.
__global__ __launch_bounds__(kThreads) void check_tables(CheckTablesArgs a, uint32_t *w) {
    const int b = blockIdx.x * kThreads + threadIdx.x;
    if (b >= a.num_seqs) return;
    int64_t len;
    uint32_t flags = 0;
    if (a.cu_q_lens) {                                  // prefill: context + chunk
        const int32_t q0 = a.cu_q_lens[b], q1 = a.cu_q_lens[b + 1];
        const int32_t ctx = a.context_lens[b];
        if (q1 < q0 || q1 - q0 > a.max_q_len || ctx < 0 || ctx > a.max_ctx_len) flags |= kCheckLength;
        if (b == a.num_seqs - 1 && q1 != a.total_q) flags |= kCheckLength;
        len = (int64_t)ctx + (q1 - q0);
    } else {                                            // decode
        len = a.seq_lens[b];
        if (len > a.max_len) flags |= kCheckLength;
    }
    if (len > (int64_t)a.max_blocks * a.block_size) {
        flags |= kCheckLength;
        len = (int64_t)a.max_blocks * a.block_size;
    }
    const int64_t nblk = len > 0 ? (len + a.block_size - 1) / a.block_size : 0;
    const int32_t *row = a.block_tables + (int64_t)b * a.max_blocks;
    for (int64_t j = 0; j < nblk; ++j) {
        const int32_t id = row[j];
        if (id < 0 || id >= a.num_blocks) {
            flags |= kCheckBlockId;
            break;
        }
    }
    if (flags) atomicOr(w, flags);
}

unsigned grid_for(int64_t n) {
    int64_t g = (n + kThreads - 1) / kThreads;
    if (g > kMaxWgs) g = kMaxWgs;
    return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_check_slots(uint32_t *w, int64_t bitmap_words, const int64_t *slots, int64_t n,
                              int64_t pool_slots, hipStream_t stream) {
    hipLaunchKernelGGL(check_clear, dim3(grid_for(bitmap_words + 1)), dim3(kThreads), 0, stream, w,
                       bitmap_words + 1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(check_slots, dim3(grid_for(n)), dim3(kThreads), 0, stream, slots, n, pool_slots, w);
    return hipGetLastError();
}

hipError_t launch_check_tables(uint32_t *w, const CheckTablesArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL(check_clear, dim3(1), dim3(kThreads), 0, stream, w, (int64_t)1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned g = (unsigned)((a.num_seqs + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(check_tables, dim3(g < 1 ? 1 : g), dim3(kThreads), 0, stream, a, w);
    return hipGetLastError();
}

}  // namespace kvf8
