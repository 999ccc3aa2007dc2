// The paged decode's launch arguments, shared by the host library and the
// decode kernels (kept apart from the other operations' declarations).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace kvf8 {

// ---------------------------------------------------------------- decode
struct DecodeArgs {
    const uint16_t *q;
    const uint8_t *k_pool;
    const uint8_t *v_pool;
    const int32_t *block_tables;
    const int32_t *seq_lens;
    void *out;
    float *partials;         // [num_seqs][q_heads][splits][head_dim + 2] or null
    int64_t num_blocks;      // pool blocks; table entries are clamped below it
    int32_t max_blocks;
    int32_t num_seqs;
    int32_t q_heads;
    int32_t kv_heads;
    int32_t head_dim;
    int32_t block_size;
    int32_t splits;          // chunks per (seq, kv-head)
    int32_t chunk_tokens;    // tokens per chunk (multiple of the block size)
    float qk_scale;          // k_scale * sm_scale * log2(e)
    float v_scale;
    int32_t out_bf16;
    int32_t k_eb;            // element bytes of the K / V pools: 1 (E4M3) or 2 (bf16)
    int32_t v_eb;
};
constexpr int kDecodeThreads = 256;   // threads per decode workgroup (4 waves)
// Number of splits and chunk length the decode uses for this shape.
void decode_plan(int32_t num_seqs, int32_t kv_heads, int32_t head_dim, int32_t block_size,
                 int32_t max_seq_len, int32_t *splits, int32_t *chunk_tokens);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);

}  // namespace kvf8
