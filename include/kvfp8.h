/*
 * kvfp8.h -- C ABI of an FP8-E4M3 paged KV cache with per-layer scalar
 * scales, for AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages, cited by title and section):
 *   [P1] "llama : Add FP8 KV-cache support (#28392)", llama.cpp commit
 *        202c1a229 (gitnews mirror).
 *   [P2] git.wylab.me compare view, branch osimons/ocp_fp8_kv (the E4M3
 *        codec in ggml).
 *   [P3] vllm.cpp PR #1641, "feat(KV-FP8): W3 -- half-sized KV blocks the
 *        runner actually serves ...".
 *
 * Conventions
 *   - Every call checks its arguments on the host before it launches
 *     anything; a call that fails launches nothing and leaves the cache as
 *     it was.  Failure is reported by the returned status; kvf8_last_error()
 *     then describes it.  No C++ exception crosses this interface.
 *   - Pointers documented as "device" are HIP device (or managed) memory of
 *     the device that was current at kv_cache_alloc; "host" pointers are
 *     ordinary host memory read before the call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Kernels are enqueued on it and the call returns without waiting.
 *     Only kv_cache_alloc (when it allocates the pools), kv_cache_free and
 *     kv_cache_set_checked allocate, set or synchronize device memory, and
 *     calls in checked mode wait for their stream; every other call only
 *     launches kernels, so it can be recorded into a HIP graph.
 *   - bf16 tensors are passed as their raw 16-bit patterns (uint16_t).
 *   - A cache handle is not thread-safe; callers serialize calls on one
 *     handle.  Calls that overlap on a stream ordering basis follow normal
 *     HIP stream semantics.
 *
 * Cache layout.  Per layer a K pool and a V pool, each
 *   [num_blocks][num_kv_heads][block_size * head_dim] bytes,
 * one OCP E4M3 code per element (or, in a pool created as bf16 by
 * kv_cache_alloc_typed, one bf16 value per element at the same index).  Slot s is token s % block_size of block
 * s / block_size.  Inside one (block, kv-head) tile of block_size*head_dim
 * bytes the order is chosen for the matrix cores:
 *   K byte (t, d) at ((d / (D/4)) * BS + t) * (D/4) + d % (D/4)
 *   V byte (t, d) at ((t / 4) * D + d) * 4 + t % 4
 * (K: four column quarters, each [BS][D/4]; V: d-major inside groups of four
 * tokens).  kv_cache_pools() exposes the pools for copy-out.
 */
#ifndef KVFP8_H
#define KVFP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvf8_status {
    KVF8_OK = 0,
    KVF8_E_INVALID = 1,      /* bad argument: shape, pointer, layer, range       */
    KVF8_E_SCALE = 2,        /* a scale is zero, not finite, or has no finite    */
                             /* fp32 reciprocal                                  */
    KVF8_E_NOMEM = 3,        /* device or host allocation failed                 */
    KVF8_E_NOBLOCKS = 4,     /* the block allocator cannot satisfy the request   */
    KVF8_E_UNSUPPORTED = 5,  /* valid request outside the supported shapes       */
    KVF8_E_HIP = 6           /* a HIP runtime call failed                        */
} kvf8_status;

typedef enum kvf8_dtype {
    KVF8_DTYPE_F32 = 0,
    KVF8_DTYPE_BF16 = 1
} kvf8_dtype;

/* Element type of one pool.  E4M3 is the scaled FP8 cache; BF16 stores the
 * given bf16 values as they are (the two-byte twin) [P3, "What turning it
 * on costs": the fp8-vs-bf16 exchange rate; P1, tests/test-fp8.cpp and
 * test-backend-ops.cpp choose the K and V cache types independently]. */
typedef enum kvf8_elem {
    KVF8_ELEM_E4M3 = 0,
    KVF8_ELEM_BF16 = 1
} kvf8_elem;

typedef enum kvf8_rope {
    KVF8_ROPE_NORM = 0,      /* rotary pairs (2i, 2i+1)                          */
    KVF8_ROPE_NEOX = 1       /* rotary pairs (i, i + rot_dim/2)                  */
} kvf8_rope;

typedef struct kvf8_cache kvf8_cache;

/* Library version string, e.g. "kvfp8 0.1.0 gfx950".  Library-owned. */
const char *kvf8_version(void);

/* Description of the last failure on the calling thread.  Library-owned,
 * valid until the next call on this thread. */
const char *kvf8_last_error(void);

/*
 * Bytes of one KV block of one layer, K and V together:
 *   2 * block_size * num_kv_heads * head_dim * elem_bytes.
 * For one-byte E4M3 elements this is exactly half the bf16 figure
 * [P3, W3 summary: KVBytesPerBlock exactly halved; "What the SECOND fresh
 * review found": with a byte budget the block count doubles].
 * Returns 0 when an argument is not positive.  Pure; no device access.
 */
size_t kv_bytes_per_block(int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                          int32_t elem_bytes);

/*
 * Create a cache of num_layers layers with num_blocks blocks per layer.
 *
 * block_size in {16, 32}; head_dim in {64, 128, 256}; num_kv_heads >= 1.
 * k_scales / v_scales (host): num_layers scales each, given as fp32 values
 *   (scale_dtype KVF8_DTYPE_F32) or bf16 bit patterns (KVF8_DTYPE_BF16),
 *   widened exactly to fp32 and stored per layer [P1, conversion/base.py
 *   _prepare_kv_cache_scales accepts BF16 or FP32 scalars and stores F32].
 *   NULL means scale 1.0 for every layer (a missing scale means no scaling,
 *   [P1, llama-graph.cpp build_attn_scale_kv_inputs]).  Every scale must be
 *   finite and nonzero [P1, llama_init_from_model] and have a finite,
 *   nonzero fp32 reciprocal (the store multiplies by it); otherwise
 *   KVF8_E_SCALE names the layer and K or V.
 * k_pool / v_pool (device): both NULL -> the library allocates the pools
 *   (num_layers * num_blocks * kv_bytes_per_block/2 bytes each), zero-fills
 *   them (synchronously) and frees them in kv_cache_free.  Both non-NULL ->
 *   borrowed caller memory of that size, [num_layers][num_blocks][...] in
 *   the layout above; the library neither clears nor frees it.  Mixed ->
 *   KVF8_E_INVALID.
 * The block allocator starts with every block free.
 * *out is written only on KVF8_OK.
 */
kvf8_status kv_cache_alloc(int32_t num_layers, int64_t num_blocks, int32_t block_size,
                           int32_t num_kv_heads, int32_t head_dim,
                           const void *k_scales, const void *v_scales, kvf8_dtype scale_dtype,
                           void *k_pool, void *v_pool, kvf8_cache **out);

/*
 * kv_cache_alloc with an element type per pool: k_elem / v_elem in
 * {KVF8_ELEM_E4M3, KVF8_ELEM_BF16} (kv_cache_alloc is E4M3 / E4M3).  A BF16
 * pool holds num_layers * num_blocks * block_size * num_kv_heads * head_dim
 * bf16 values in the same tile order as above (element (t, d) at the same
 * index, two bytes each) and stores the given values unchanged, so its scale
 * must be 1.0 for every layer (NULL scales give 1.0; any other value ->
 * KVF8_E_SCALE).  BF16 pools support head_dim 64 and 128 (256 ->
 * KVF8_E_UNSUPPORTED).  Store, decode and prefill read each pool with its
 * own element type.  kv_shift_rope on a BF16 K pool rounds each
 * rotated value to fp32 and then to the nearest bf16 (a pair holding a NaN
 * becomes the quiet NaN 0x7FC0 in both places).
 */
kvf8_status kv_cache_alloc_typed(int32_t num_layers, int64_t num_blocks, int32_t block_size,
                                 int32_t num_kv_heads, int32_t head_dim, kvf8_elem k_elem,
                                 kvf8_elem v_elem, const void *k_scales, const void *v_scales,
                                 kvf8_dtype scale_dtype, void *k_pool, void *v_pool,
                                 kvf8_cache **out);

/* The element types of a cache's K and V pools (host outputs; either may be NULL). */
kvf8_status kv_cache_elem_types(const kvf8_cache *cache, kvf8_elem *k_elem, kvf8_elem *v_elem);

/* Destroy a cache; frees what kv_cache_alloc allocated.  NULL -> KVF8_OK. */
kvf8_status kv_cache_free(kvf8_cache *cache);

/*
 * Checked mode, off by default (a debugging aid for callers that build slot
 * lists and block tables themselves).  When on, the index inputs the kernels
 * otherwise take on trust are verified on the device before the real launch,
 * and a call that fails launches nothing that writes the cache:
 *   kv_store_fp8, kv_shift_rope, kv_shift_rope_per_slot: a slot that appears
 *     twice in one call (whose result is otherwise undefined) -> KVF8_E_INVALID;
 *   paged_attn_decode / paged_attn_prefill_chunk: a length above its stated
 *     bound (max_seq_len; max_q_len, max_ctx_len, total_q) or past the table
 *     row, or a table entry in use outside [0, num_blocks) -> KVF8_E_INVALID.
 * Each check waits for `stream`, so calls in checked mode synchronize and
 * cannot be recorded into a HIP graph.  Turning it on allocates one bit per
 * cache slot (plus a word) of device memory on the current device (make the
 * cache's device current); turning it off frees it.  on: nonzero / zero.
 */
kvf8_status kv_cache_set_checked(kvf8_cache *cache, int32_t on);

/* Replace one layer's scales (host values, as in kv_cache_alloc; NULL keeps
 * that side unchanged).  Checked like kv_cache_alloc; on error nothing
 * changes.  Bytes already stored are not rewritten. */
kvf8_status kv_cache_set_scales(kvf8_cache *cache, int32_t layer, const void *k_scale,
                                const void *v_scale, kvf8_dtype scale_dtype);

/* Read one layer's fp32 scales (host outputs; either may be NULL). */
kvf8_status kv_cache_get_scales(const kvf8_cache *cache, int32_t layer, float *k_scale,
                                float *v_scale);

/* Borrowed device views of one layer's pools and the size in bytes of the K
 * pool (outputs may be NULL; the V pool's size is the same times its element
 * size over K's). */
kvf8_status kv_cache_pools(const kvf8_cache *cache, int32_t layer, uint8_t **k_pool,
                           uint8_t **v_pool, size_t *pool_bytes);

/*
 * Host block allocator of the cache (one free list shared by all layers:
 * a block id names the same block in every layer).
 *   kv_block_alloc: take n block ids, written to ids_out (host, n entries).
 *     All or nothing: KVF8_E_NOBLOCKS when fewer than n are free.
 *   kv_block_free: return n ids (host).  KVF8_E_INVALID, with nothing
 *     returned, when an id is out of range, not allocated, or repeated.
 *   kv_blocks_free: number of free blocks (-1 for a NULL cache).
 *   kv_block_shuffle: permute the free list with a seeded generator, so that
 *     later allocations come back scattered over the pool.
 * Ids are handed out last-freed-first; a fresh cache hands out 0, 1, 2, ...
 */
kvf8_status kv_block_alloc(kvf8_cache *cache, int32_t n, int32_t *ids_out);
kvf8_status kv_block_free(kvf8_cache *cache, const int32_t *ids, int32_t n);
int64_t kv_blocks_free(const kvf8_cache *cache);
kvf8_status kv_block_shuffle(kvf8_cache *cache, uint64_t seed);

/*
 * Store new K/V rows into one layer as E4M3 codes.
 *
 * For token i, kv-head h, dim d with slot = slot_mapping[i] >= 0:
 *   x    = bf16 value widened to fp32,
 *   y    = fl32(x * fl32(1 / scale))      (scale of this layer, K or V),
 *   code = saturating round-half-even E4M3 of y,
 * written at the slot's position in the layout above.  Saturation, NaN and
 * signed zero follow [P2, ggml_fp32_to_f8_e4m3]: NaN -> sign|0x7F with the
 * input's sign, +-Inf and |y| >= 448 -> sign|0x7E, zero keeps its sign.
 * The division of [P1, build_attn_scale_kv_inputs] (store K/s, V/s) is done
 * as a multiply by the reciprocal.  A BF16 pool (kv_cache_alloc_typed)
 * receives the bf16 bit patterns unchanged instead.
 *
 * k_bf16, v_bf16 (device): [num_tokens][num_kv_heads][head_dim] bf16 rows;
 *   row i starts at element i * k_tok_stride (resp. v_tok_stride), heads and
 *   dims are contiguous inside a row; stride >= num_kv_heads*head_dim.
 * slot_mapping (device): int64 [num_tokens].  Slots < 0 and slots >=
 *   num_blocks * block_size are skipped (nothing is written for them).  No
 *   slot may repeat in one call: the bytes of a repeated slot are undefined.
 * num_tokens == 0 is a no-op.
 */
kvf8_status kv_store_fp8(kvf8_cache *cache, int32_t layer, const uint16_t *k_bf16,
                         const uint16_t *v_bf16, int64_t k_tok_stride, int64_t v_tok_stride,
                         const int64_t *slot_mapping, int64_t num_tokens, void *stream);

/*
 * Workspace bytes paged_attn_decode needs for this shape (0 when it needs
 * none).  max_seq_len is the host upper bound later passed to the call.
 */
size_t paged_attn_decode_workspace(const kvf8_cache *cache, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t max_seq_len);

/*
 * Paged decode attention over one layer's cache, dequantizing in flight.
 *
 * For sequence b and query head h (kv-head h / (num_q_heads/num_kv_heads)):
 *   s_t = (q . K_t) * k_scale * sm_scale      over t < seq_lens[b],
 *   o   = v_scale * sum_t softmax(s)_t V_t,
 * where K_t, V_t are the stored elements' values (E4M3 codes' values, or
 * bf16 values in a bf16 pool, whose scale is 1); this equals attention
 * over the dequantized cache [P1, build_attn_scale_kv_inputs /
 * build_attn_scale_kv_output: (Q*s)(K/s) = QK, P(V/s)s = PV].
 * seq_lens[b] <= 0 gives a zero row.
 *
 * q_bf16 (device): [num_seqs][num_q_heads][head_dim] bf16.
 * block_tables (device): int32 [num_seqs][max_blocks_per_seq]; entries
 *   0 .. ceil(seq_lens[b]/block_size)-1 of row b must be valid block ids.
 * seq_lens (device): int32 [num_seqs], each at most max_seq_len and at most
 *   max_blocks_per_seq * block_size.  A longer length is out of contract: the
 *   call still reads only the row's table entries and the pools, but that
 *   row's result is unspecified.
 * max_seq_len (host): upper bound of seq_lens, sizes the launch.
 * sm_scale: softmax scale, finite and > 0 (usually 1/sqrt(head_dim)); the
 *   fp32 factor k_scale * sm_scale * log2(e) must be finite and nonzero
 *   (else KVF8_E_SCALE).
 * out (device): [num_seqs][num_q_heads][head_dim], fp32 or bf16 (out_dtype).
 * workspace (device): at least paged_attn_decode_workspace(...) bytes,
 *   used as scratch by this call only; may be NULL when that is 0.
 * num_q_heads must be a multiple of num_kv_heads with a group size <= 16.
 */
kvf8_status paged_attn_decode(kvf8_cache *cache, int32_t layer, const uint16_t *q_bf16,
                              int32_t num_q_heads, const int32_t *block_tables,
                              int32_t max_blocks_per_seq, const int32_t *seq_lens,
                              int32_t num_seqs, int32_t max_seq_len, float sm_scale, void *out,
                              kvf8_dtype out_dtype, void *workspace, size_t workspace_bytes,
                              void *stream);

/*
 * paged_attn_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, arguments and results, without the
 * workspace arguments.  The split-K partials go into a fixed device array of
 * 64 MiB that the library holds on each GPU it runs on until the process
 * ends; its device address is looked up once per device (at kv_cache_alloc
 * with library-owned pools, else on the first call on that device) and the
 * call itself allocates nothing.
 *   - A shape whose workspace (paged_attn_decode_workspace) exceeds 64 MiB
 *     -> KVF8_E_UNSUPPORTED, before anything is launched.
 *   - Every call on one GPU uses that GPU's array, which keeps the last
 *     call's contents (nothing in it needs to start at zero): calls that
 *     overlap on one GPU (concurrent streams, threads) race and give
 *     undefined results; calls ordered on one stream do not.
 *   - The device is the stream's (the current device for a NULL stream).
 */
kvf8_status paged_attn_decode_noalloc(kvf8_cache *cache, int32_t layer, const uint16_t *q_bf16,
                                      int32_t num_q_heads, const int32_t *block_tables,
                                      int32_t max_blocks_per_seq, const int32_t *seq_lens,
                                      int32_t num_seqs, int32_t max_seq_len, float sm_scale,
                                      void *out, kvf8_dtype out_dtype, void *stream);

/*
 * Causal attention of a chunk of new query tokens over one layer's cache
 * (chunked prefill).  Sequence b has context_lens[b] tokens cached before
 * its chunk of cu_q_lens[b+1] - cu_q_lens[b] query tokens; query token i of
 * the chunk sits at position context_lens[b] + i and attends to positions
 * 0 .. context_lens[b] + i [P1, tests/test-fp8.cpp check_fp8_attention,
 * causal "past <= token"].  Scales and GQA as in paged_attn_decode.
 * Precondition: the chunk's own K/V are already stored (kv_store_fp8) at
 * positions context_lens[b] .. context_lens[b] + q_len - 1, so that every key
 * is read from the E4M3 cache [P1, build_attn: store first, then read the
 * cache views].
 *
 * q_bf16 (device): [total_q][num_q_heads][head_dim] bf16, sequences
 *   back to back.  cu_q_lens (device): int32 [num_seqs+1], cu_q_lens[0] = 0,
 *   non-decreasing, cu_q_lens[num_seqs] = total_q.  context_lens (device):
 *   int32 [num_seqs].  block_tables (device): as in paged_attn_decode,
 *   covering context + chunk: context_lens[b] + q_len_b must not exceed
 *   max_blocks_per_seq * block_size (keys past the table row are never
 *   read).  max_q_len / max_ctx_len (host): upper bounds of the chunk lengths
 *   and context lengths, size the launch.
 * sm_scale: as in paged_attn_decode (KVF8_E_SCALE when k_scale * sm_scale *
 *   log2(e) is 0 or not finite in fp32).
 * out (device): [total_q][num_q_heads][head_dim], fp32 or bf16.
 */
kvf8_status paged_attn_prefill_chunk(kvf8_cache *cache, int32_t layer, const uint16_t *q_bf16,
                                     int32_t num_q_heads, const int32_t *cu_q_lens,
                                     const int32_t *context_lens, const int32_t *block_tables,
                                     int32_t max_blocks_per_seq, int32_t num_seqs,
                                     int64_t total_q, int32_t max_q_len, int32_t max_ctx_len,
                                     float sm_scale, void *out, kvf8_dtype out_dtype,
                                     void *stream);

/*
 * Shift cached K by a RoPE position delta, in place: dequantize -> rotate ->
 * requantize [P1, src/llama-kv-cache.cpp build_rope_shift keeps F8_E4M3 out
 * of the in-place rope; tests/test-fp8.cpp check_fp8_context_shift expects
 * quantize(rope(to_float(bytes))) with no scale].  The rotation works on the
 * stored codes' values without the layer scale (rotation is linear, so
 * rot(K)/s = rot(K/s)).
 *
 * Rotary pair i (0 <= i < rot_dim/2) turns by angle a_i = delta *
 * theta_base^(-2i/rot_dim); the library computes cos a_i and sin a_i in
 * double on the host and rounds them to fp32.  With x0, x1 the pair's
 * decoded values, y0 = fl32(x0*c - x1*s) and y1 = fl32(x0*s + x1*c) computed
 * in fp64, then encoded as in kv_store_fp8.  A pair holding a NaN code
 * becomes 0x7F in both places.  Dims >= rot_dim are not touched.
 *
 * slots (device): int64 [n_slots] cache slots to shift (< 0 and >=
 *   num_blocks * block_size skipped; no repeats).  rot_dim even, 2 <= rot_dim <= head_dim.  theta_base finite
 *   and > 0.
 */
kvf8_status kv_shift_rope(kvf8_cache *cache, int32_t layer, const int64_t *slots,
                          int64_t n_slots, int32_t delta, float theta_base, int32_t rot_dim,
                          kvf8_rope style, void *stream);

/*
 * Position deltas per slot [P1, tests/test-fp8.cpp check_fp8_context_shift:
 * the shift tensor holds one offset per cache cell, so one pass moves cells
 * by different amounts].  Two calls:
 *
 * kv_rope_table (host only): table[j][i] = (cos a, sin a) as fp32, with
 *   a = deltas[j] * theta_base^(-2i/rot_dim) for 0 <= i < rot_dim/2, the
 *   same values kv_shift_rope computes for a single delta.  deltas: host
 *   int32 [n_deltas]; table: host float [n_deltas][rot_dim/2][2],
 *   caller-owned.  rot_dim even in [2, 256]; theta_base finite and > 0.
 *
 * kv_shift_rope_per_slot: slot slots[k] turns by the angles of table row
 *   table_rows[k], exactly as kv_shift_rope turns it for that row's delta.
 *   slots (device): int64 [n_slots], no repeats; negative slots, slots at or
 *   past num_blocks * block_size, and rows outside [0, n_rows) are skipped.
 *   table_rows (device): int32 [n_slots].  table (device, 16-byte aligned,
 *   caller-owned): the kv_rope_table output for n_rows deltas, copied to the
 *   device.  rot_dim and style as in kv_shift_rope (the table must have been
 *   built for the same rot_dim).  Asynchronous on `stream`.  E4M3 and bf16
 *   K pools, each as in kv_shift_rope.
 */
kvf8_status kv_rope_table(const int32_t *deltas, int32_t n_deltas, float theta_base, int32_t rot_dim,
                          float *table);
kvf8_status kv_shift_rope_per_slot(kvf8_cache *cache, int32_t layer, const int64_t *slots,
                                   const int32_t *table_rows, int64_t n_slots, const float *table,
                                   int32_t n_rows, int32_t rot_dim, kvf8_rope style, void *stream);

/*
 * Per-tensor scale calibration on the device: a running absolute maximum of
 * bf16 K and V tensors and the scales s = amax / 448, which put each
 * tensor's largest magnitude on E4M3's largest finite value (the amax / 448
 * rule of vllm.cpp PR #1641, whose "Unreached and owed" list leaves run-time
 * calibration unbuilt; 448 from ggml_fp32_to_f8_e4m3, git.wylab.me
 * osimons/ocp_fp8_kv).  The scales are meant for kv_cache_alloc /
 * kv_cache_set_scales, which take host values: copy scales_out to the host
 * once the stream has finished.
 *
 * k_bf16, v_bf16 (device): [num_tokens][row_elems] bf16 rows, row i at
 *   element i * k_tok_stride (resp. v_tok_stride); either may be NULL, which
 *   leaves that side's maximum unchanged.  Rows 16-byte aligned (pointer
 *   16-byte aligned, stride a multiple of 8 and >= row_elems); row_elems a
 *   positive multiple of 8, at most 2^31.
 * amax (device, caller-owned, 4-byte aligned): float [2], the running K and
 *   V maxima.  Start each at +0.0; every call raises amax[0] (amax[1]) to the
 *   largest |x| of the K (V) rows it reads, so calls over parts of a tensor
 *   accumulate.  A NaN element makes that maximum the quiet NaN 0x7FC00000
 *   (it stays NaN); infinities count as the largest values.
 * scales_out (device, may be NULL): [2] scales (K, V) from the maxima after
 *   this call, as fp32 bit patterns (scale_dtype KVF8_DTYPE_F32: the
 *   correctly rounded quotient amax / 448) or bf16 bit patterns
 *   (KVF8_DTYPE_BF16: that fp32 value rounded to the nearest bf16, ties to
 *   even).  A NaN maximum gives the quiet NaN.  A zero or infinite maximum
 *   gives a scale of 0 or infinity, which kv_cache_alloc and
 *   kv_cache_set_scales refuse with KVF8_E_SCALE.
 * num_tokens == 0 only computes the scales.  Asynchronous on `stream`; calls
 * that share an amax buffer must be ordered on one stream.
 */
kvf8_status kv_calibrate_scales(const uint16_t *k_bf16, const uint16_t *v_bf16, int64_t k_tok_stride,
                                int64_t v_tok_stride, int64_t num_tokens, int64_t row_elems, float *amax,
                                void *scales_out, kvf8_dtype scale_dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVFP8_H */
