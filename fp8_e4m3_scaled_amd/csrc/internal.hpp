// Internal declarations shared by the host library and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <vector>

#include "decode_args.hpp"

struct kvf8_cache {
    int32_t layers = 0;
    int64_t num_blocks = 0;
    int32_t block_size = 0;
    int32_t kv_heads = 0;
    int32_t head_dim = 0;
    int32_t k_eb = 1;               // element bytes of the K pool: 1 (E4M3) or 2 (bf16)
    int32_t v_eb = 1;
    size_t k_pool_bytes = 0;        // bytes of one layer's K pool
    size_t v_pool_bytes = 0;
    uint8_t *k_base = nullptr;      // [layers][pool_bytes]
    uint8_t *v_base = nullptr;
    bool owned = false;
    int device = 0;
    std::vector<float> k_scale, v_scale, k_inv, v_inv;
    std::vector<int32_t> free_list;  // LIFO: back() is handed out next
    std::vector<uint8_t> allocated;
    // checked mode: device state of the index checks (word 0 flags, then one bit per slot)
    bool checked = false;
    uint32_t *check_state = nullptr;
    int64_t check_bitmap_words = 0;
};

namespace kvf8 {

// ---------------------------------------------------------------- store
struct StoreArgs {
    const uint16_t *k;
    const uint16_t *v;
    int64_t k_stride;        // elements between token rows
    int64_t v_stride;
    const int64_t *slots;
    int64_t num_tokens;
    int64_t pool_slots;      // num_blocks * block_size: slots at or past it are skipped
    uint8_t *k_pool;         // this layer
    uint8_t *v_pool;
    float k_inv;
    float v_inv;
    int32_t kv_heads;
    int32_t head_dim;
    int32_t block_size;
    int32_t k_eb;            // element bytes of the K pool: 1 (E4M3 codes) or 2 (bf16 as given)
    int32_t v_eb;
};
hipError_t launch_store(const StoreArgs &a, hipStream_t stream);

// ---------------------------------------------------------------- no-allocation decode
// Bytes of the fixed device array that holds paged_attn_decode_noalloc's
// split-K partials (one per device, for the life of the process).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
// Device address of that array on `device`; looked up on the first call for
// each device (with that device current), then kept.
hipError_t noalloc_scratch(int device, void **ptr);

// ---------------------------------------------------------------- prefill constants
constexpr int kPrefillThreads = 256;  // threads per prefill workgroup (4 waves)
constexpr int kPrefillRows = 128;     // (query token, head) rows per prefill workgroup


// ---------------------------------------------------------------- K-shift
struct KShiftArgs {
    uint8_t *k_pool;
    const int64_t *slots;
    int64_t n_slots;
    int64_t pool_slots;      // num_blocks * block_size: slots at or past it are skipped
    int32_t kv_heads;
    int32_t head_dim;
    int32_t block_size;
    int32_t rot_dim;
    int32_t neox;
    float cos_t[128];        // one delta for every slot (rows == nullptr) ...
    float sin_t[128];
    const int32_t *rows;     // ... or a row of `table` per slot: [n_rows][rot_dim/2][cos, sin]
    const float *table;
    int32_t n_rows;
    int32_t k_eb;            // element bytes of the K pool: 1 (E4M3 codes) or 2 (bf16 values)
};
hipError_t launch_kshift(const KShiftArgs &a, hipStream_t stream);

// ---------------------------------------------------------------- prefill
struct PrefillArgs {
    const uint16_t *q;
    const uint8_t *k_pool;
    const uint8_t *v_pool;
    const int32_t *cu_q_lens;
    const int32_t *context_lens;
    const int32_t *block_tables;
    void *out;
    int64_t num_blocks;
    int32_t max_blocks;
    int32_t num_seqs;
    int32_t q_heads;
    int32_t kv_heads;
    int32_t head_dim;
    int32_t block_size;
    int32_t max_q_len;
    int32_t q_tiles;         // query-row tiles per (sequence, kv head), set by the launcher
    float qk_scale;          // k_scale * sm_scale * log2(e)
    float v_scale;
    int32_t out_bf16;
    int32_t k_eb;            // element bytes of the K / V pools: 1 (E4M3) or 2 (bf16)
    int32_t v_eb;
};
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);

// ---------------------------------------------------------------- calibration
struct CalibArgs {
    const uint16_t *x[2];    // K, V bf16 rows (a side may be null when not launched)
    int64_t stride[2];       // elements between rows
    int32_t side[2];         // tensor of grid row y: side[y] in {0 (K), 1 (V)}
    int64_t rows;            // tokens
    int64_t runs_per_row;    // 16-byte runs (8 elements) per row
    uint32_t *amax;          // [2] running maxima as fp32 bit patterns
};
constexpr int64_t kCalibWorkgroups = 2048;   // amax workgroups per launch, over both tensors (512-8192 swept)
// amax over the sides present (sides = 0, 1 or 2), then, when scales_out is
// non-null, the two scales from the maxima (fp32 or bf16 bit patterns).
hipError_t launch_calibrate(const CalibArgs &a, int32_t sides, void *scales_out, int32_t out_bf16,
                            hipStream_t stream);

// ---------------------------------------------------------------- checked mode
constexpr uint32_t kCheckRepeatedSlot = 1u;   // a slot appears twice in one call
constexpr uint32_t kCheckLength = 2u;         // a length outside its stated bound or the table row
constexpr uint32_t kCheckBlockId = 4u;        // a used table entry outside [0, num_blocks)
struct CheckTablesArgs {
    const int32_t *block_tables;
    const int32_t *seq_lens;      // decode lengths, or
    const int32_t *cu_q_lens;     // prefill: chunk offsets [num_seqs + 1] with
    const int32_t *context_lens;  //   context lengths [num_seqs]
    int64_t num_blocks;
    int64_t total_q;
    int32_t max_blocks;
    int32_t num_seqs;
    int32_t block_size;
    int32_t max_len;              // decode: max_seq_len
    int32_t max_q_len;            // prefill bounds
    int32_t max_ctx_len;
};
hipError_t launch_check_slots(uint32_t *w, int64_t bitmap_words, const int64_t *slots, int64_t n,
                              int64_t pool_slots, hipStream_t stream);
hipError_t launch_check_tables(uint32_t *w, const CheckTablesArgs &a, hipStream_t stream);


}  // namespace kvf8
