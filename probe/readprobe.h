/*
 * Measurement aids for the benchmark, not steps of the cache and not part of
 * the kvfp8 library: a plain streaming read of a device buffer (the part's
 * practical read-bandwidth ceiling), a plain read of exactly the K/V tiles a
 * paged decode reads (the ceiling of its scattered access pattern), and the
 * K-shift's and the cache fill's traffic with no arithmetic (the ceilings of
 * their access patterns).  Built into libkvf8probe.so.  Every call checks its arguments on
 * the host and launches nothing when one is wrong; it returns 0 on success, 1
 * for an invalid argument (message in kvf8_probe_last_error) and 6 for a HIP
 * error.
 */
#ifndef KVF8_PROBE_H
#define KVF8_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Message of the calling thread's last failed call ("" after a success). */
const char *kvf8_probe_last_error(void);

/*
 * Streaming read of `bytes` of device memory at `buf` (16-byte aligned, bytes
 * a multiple of 16) by n_out workgroups (1 <= n_out <= 2^20), grid-stride;
 * workgroup i writes the XOR of every 32-bit word it read to out_words[i]
 * (device, caller-owned), so the XOR of all out_words equals the XOR of the
 * buffer's 32-bit words.  bytes == 0 is a no-op.  Asynchronous on `stream`.
 */
int kvf8_probe_read(const void *buf, size_t bytes, uint32_t *out_words, int32_t n_out, void *stream);

/*
 * Read of every K and V tile of blocks 0 .. ceil(seq_lens[b] / block_size) - 1
 * of block_tables[b] (never past max_blocks entries), for every kv-head: the
 * tiles paged_attn_decode reads.  k_pool / v_pool (device): one layer's pools,
 * [num_blocks][num_kv_heads][block_size * head_dim] elements of k_elem_bytes /
 * v_elem_bytes (1 or 2) bytes.  Block ids at or past num_blocks read the last
 * block.  Workgroup (b, h) writes the XOR of every 32-bit word of its tiles to
 * out_words[b * num_kv_heads + h] (device, caller-owned).  block_size in
 * {16, 32}, head_dim in {64, 128, 256}.  Asynchronous on `stream`.
 */
int kvf8_probe_gather(const void *k_pool, const void *v_pool, int64_t num_blocks, int32_t num_kv_heads,
                      int32_t block_size, int32_t head_dim, int32_t k_elem_bytes, int32_t v_elem_bytes,
                      const int32_t *block_tables, int32_t max_blocks, const int32_t *seq_lens, int32_t num_seqs,
                      uint32_t *out_words, void *stream);

/*
 * The same read split the way a split-K decode reads: unit (c, b, h) reads
 * table entries [c * chunk_blocks, (c + 1) * chunk_blocks) of sequence b's
 * blocks (as limited above) for kv-head h and writes their XOR to
 * out_words[(c * num_seqs + b) * num_kv_heads + h], for c < ceil(max_blocks /
 * chunk_blocks) (units past a sequence's blocks write 0).  chunk_blocks > 0.
 * kvf8_probe_gather is this call with one chunk per row.
 */
int kvf8_probe_gather_split(const void *k_pool, const void *v_pool, int64_t num_blocks, int32_t num_kv_heads,
                            int32_t block_size, int32_t head_dim, int32_t k_elem_bytes, int32_t v_elem_bytes,
                            const int32_t *block_tables, int32_t max_blocks, const int32_t *seq_lens, int32_t num_seqs,
                            int32_t chunk_blocks, uint32_t *out_words, void *stream);

/*
 * The memory traffic of kv_shift_rope's run path (NEOX pairing) with no
 * arithmetic: for every slot of `slots` (device, n_slots int64 entries;
 * entries < 0 or >= num_blocks * block_size are skipped, as by the K-shift)
 * and every kv-head, the bytes of dims [0, rot_dim/2) and their partners
 * [rot_dim/2, rot_dim) of the slot's K row are read and written back XORed
 * with 0x01, in place, 16 bytes per access, through the same work items and
 * grid-stride launch as the K-shift.  Applying it twice restores the pool.
 * k_pool (device): [num_blocks][num_kv_heads][block_size * head_dim] E4M3
 * codes.  block_size in {16, 32}, head_dim in {64, 128, 256}, rot_dim a
 * multiple of 32 in [32, head_dim].  n_slots == 0 is a no-op.  Calls that
 * name the same slot twice, or overlap on one pool, race.  Asynchronous on
 * `stream`.
 */
int kvf8_probe_rmw(void *k_pool, int64_t num_blocks, int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                   int32_t rot_dim, const int64_t *slots, int64_t n_slots, void *stream);

/*
 * The memory traffic of kv_store_fp8's 16-token run path with no arithmetic:
 * every group of 16 consecutive input tokens (token 16i .. 16i + 15) whose
 * slots are 16 consecutive slots s0 .. s0 + 15 with s0 a multiple of 16,
 * inside the pool (num_blocks * block_size slots), is read and written with
 * the store's workgroups, pieces and loads, but the byte written where the
 * store writes a value's code is the high byte of the value's bf16 bits.
 * Other groups (and a last partial one) are left alone.  k / v (device):
 * [num_tokens][*_stride] bf16 bits, rows of num_kv_heads * head_dim values,
 * strides multiples of 8 elements and >= that row; slots (device):
 * num_tokens int64; k_pool / v_pool (device): [num_blocks][num_kv_heads]
 * [block_size * head_dim] bytes in the cache's E4M3 layout.  k, v and the
 * pools 16-byte aligned; block_size in {16, 32}, head_dim in {64, 128, 256}.
 * num_tokens == 0 is a no-op.  Asynchronous on `stream`.
 */
int kvf8_probe_store_copy(const uint16_t *k, const uint16_t *v, int64_t k_stride, int64_t v_stride,
                          const int64_t *slots, int64_t num_tokens, void *k_pool, void *v_pool, int64_t num_blocks,
                          int32_t num_kv_heads, int32_t block_size, int32_t head_dim, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVF8_PROBE_H */
