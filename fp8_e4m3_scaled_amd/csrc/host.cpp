// Host side of the kvfp8 C ABI: argument checks, scale intake, pool
// ownership, the block allocator and kernel launch configuration.
// Sources are cited by web-page title and section (see kvfp8.h).

#include "kvfp8.h"
#include "internal.hpp"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

namespace {

thread_local std::string g_last_error;

kvf8_status fail(kvf8_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

kvf8_status ok() {
    g_last_error.clear();
    return KVF8_OK;
}

kvf8_status hip_fail(hipError_t e, const char *what) {
    return fail(KVF8_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Checked mode: read back the flag word of a check launched on `stream` and
// wait for it (the only synchronizing step besides allocation).
kvf8_status check_result(const kvf8_cache *c, hipError_t launched, hipStream_t stream, uint32_t *flags) {
    if (launched != hipSuccess) return hip_fail(launched, "checked mode: check launch");
    uint32_t h = 0;
    hipError_t e = hipMemcpyAsync(&h, c->check_state, sizeof h, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "checked mode: read-back");
    *flags = h;
    return KVF8_OK;
}

// Checked mode: a slot list must not repeat an in-pool slot.
kvf8_status check_slot_list(const kvf8_cache *c, const int64_t *slots, int64_t n, hipStream_t stream) {
    if (!c->checked || n == 0) return KVF8_OK;
    uint32_t flags = 0;
    kvf8_status st = check_result(c, kvf8::launch_check_slots(c->check_state, c->check_bitmap_words, slots, n,
                                                              c->num_blocks * c->block_size, stream),
                                  stream, &flags);
    if (st != KVF8_OK) return st;
    if (flags & kvf8::kCheckRepeatedSlot)
        return fail(KVF8_E_INVALID, "checked mode: a slot appears more than once in this call");
    return KVF8_OK;
}

// Checked mode: lengths within their stated bounds and the table row; every
// table entry a sequence uses inside the pool.
kvf8_status check_table_args(const kvf8_cache *c, const kvf8::CheckTablesArgs &a, hipStream_t stream) {
    if (!c->checked || a.num_seqs == 0) return KVF8_OK;
    uint32_t flags = 0;
    kvf8_status st = check_result(c, kvf8::launch_check_tables(c->check_state, a, stream), stream, &flags);
    if (st != KVF8_OK) return st;
    if (flags & kvf8::kCheckLength)
        return fail(KVF8_E_INVALID, "checked mode: a sequence length exceeds its stated bound or its table row");
    if (flags & kvf8::kCheckBlockId)
        return fail(KVF8_E_INVALID, "checked mode: a block table entry in use lies outside the pool");
    return KVF8_OK;
}

// Scale intake: bf16 bit patterns widen exactly to fp32 (the top 16 bits).
float read_scale(const void *p, int32_t i, kvf8_dtype dt) {
    if (dt == KVF8_DTYPE_F32) {
        float f;
        std::memcpy(&f, static_cast<const float *>(p) + i, sizeof f);
        return f;
    }
    uint16_t b;
    std::memcpy(&b, static_cast<const uint16_t *>(p) + i, sizeof b);
    uint32_t u = static_cast<uint32_t>(b) << 16;
    float f;
    std::memcpy(&f, &u, sizeof f);
    return f;
}

// A usable scale is finite and nonzero [P1, llama_init_from_model] and has a
// finite, nonzero fp32 reciprocal, because the store multiplies by it.
bool scale_usable(float s) {
    if (!std::isfinite(s) || s == 0.0f) return false;
    volatile float inv = 1.0f / s;
    return std::isfinite(inv) && inv != 0.0f;
}

bool shape_supported(int32_t bs, int32_t d) {
    return (bs == 16 || bs == 32) && (d == 64 || d == 128 || d == 256);
}

kvf8_status check_layer(const kvf8_cache *c, int32_t layer) {
    if (!c) return fail(KVF8_E_INVALID, "cache is NULL");
    if (layer < 0 || layer >= c->layers)
        return fail(KVF8_E_INVALID, "layer %d out of range [0, %d)", layer, c->layers);
    return KVF8_OK;
}

uint8_t *k_pool_of(const kvf8_cache *c, int32_t layer) { return c->k_base + (size_t)layer * c->k_pool_bytes; }
uint8_t *v_pool_of(const kvf8_cache *c, int32_t layer) { return c->v_base + (size_t)layer * c->v_pool_bytes; }

int32_t elem_bytes(kvf8_elem e) { return e == KVF8_ELEM_BF16 ? 2 : 1; }

// splitmix64: the seeded generator behind kv_block_shuffle.
uint64_t splitmix64(uint64_t &x) {
    uint64_t z = (x += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

}  // namespace

extern "C" {

const char *kvf8_version(void) { return "kvfp8 0.1.0 gfx950"; }

const char *kvf8_last_error(void) { return g_last_error.c_str(); }

size_t kv_bytes_per_block(int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                          int32_t elem_bytes) {
    if (block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0 || elem_bytes <= 0) return 0;
    return 2ull * (size_t)block_size * (size_t)num_kv_heads * (size_t)head_dim * (size_t)elem_bytes;
}

kvf8_status kv_cache_alloc(int32_t num_layers, int64_t num_blocks, int32_t block_size,
                           int32_t num_kv_heads, int32_t head_dim, const void *k_scales,
                           const void *v_scales, kvf8_dtype scale_dtype, void *k_pool,
                           void *v_pool, kvf8_cache **out) {
    return kv_cache_alloc_typed(num_layers, num_blocks, block_size, num_kv_heads, head_dim, KVF8_ELEM_E4M3,
                                KVF8_ELEM_E4M3, k_scales, v_scales, scale_dtype, k_pool, v_pool, out);
}

kvf8_status kv_cache_alloc_typed(int32_t num_layers, int64_t num_blocks, int32_t block_size,
                                 int32_t num_kv_heads, int32_t head_dim, kvf8_elem k_elem,
                                 kvf8_elem v_elem, const void *k_scales, const void *v_scales,
                                 kvf8_dtype scale_dtype, void *k_pool, void *v_pool, kvf8_cache **out) {
    if (!out) return fail(KVF8_E_INVALID, "out is NULL");
    if ((k_elem != KVF8_ELEM_E4M3 && k_elem != KVF8_ELEM_BF16) || (v_elem != KVF8_ELEM_E4M3 && v_elem != KVF8_ELEM_BF16))
        return fail(KVF8_E_INVALID, "k_elem and v_elem must be KVF8_ELEM_E4M3 or KVF8_ELEM_BF16");
    if (num_layers <= 0 || num_blocks <= 0 || num_kv_heads <= 0 || block_size <= 0 || head_dim <= 0)
        return fail(KVF8_E_INVALID, "num_layers, num_blocks, block_size, num_kv_heads and head_dim must be positive");
    if (num_blocks > INT32_MAX)
        return fail(KVF8_E_INVALID, "num_blocks %lld exceeds the int32 block-id range", (long long)num_blocks);
    if (!shape_supported(block_size, head_dim))
        return fail(KVF8_E_INVALID, "unsupported block_size %d / head_dim %d (block_size 16 or 32, head_dim 64, 128 or 256)",
                    block_size, head_dim);
    if (scale_dtype != KVF8_DTYPE_F32 && scale_dtype != KVF8_DTYPE_BF16)
        return fail(KVF8_E_INVALID, "scale_dtype must be KVF8_DTYPE_F32 or KVF8_DTYPE_BF16");
    if ((k_pool == nullptr) != (v_pool == nullptr))
        return fail(KVF8_E_INVALID, "k_pool and v_pool must both be NULL or both be given");
    if ((k_elem == KVF8_ELEM_BF16 || v_elem == KVF8_ELEM_BF16) && head_dim > 128)
        return fail(KVF8_E_UNSUPPORTED, "bf16 pools support head_dim 64 and 128, got %d", head_dim);

    std::vector<float> ks(num_layers, 1.0f), vs(num_layers, 1.0f);
    for (int32_t l = 0; l < num_layers; ++l) {
        if (k_scales) ks[l] = read_scale(k_scales, l, scale_dtype);
        if (v_scales) vs[l] = read_scale(v_scales, l, scale_dtype);
        if (!scale_usable(ks[l]))
            return fail(KVF8_E_SCALE, "FP8 cache scale of layer %d (K) must be finite and nonzero with a finite reciprocal, got %g",
                        l, (double)ks[l]);
        if (!scale_usable(vs[l]))
            return fail(KVF8_E_SCALE, "FP8 cache scale of layer %d (V) must be finite and nonzero with a finite reciprocal, got %g",
                        l, (double)vs[l]);
        if (k_elem == KVF8_ELEM_BF16 && ks[l] != 1.0f)
            return fail(KVF8_E_SCALE, "the bf16 K pool stores values as given: its scale (layer %d) must be 1, got %g",
                        l, (double)ks[l]);
        if (v_elem == KVF8_ELEM_BF16 && vs[l] != 1.0f)
            return fail(KVF8_E_SCALE, "the bf16 V pool stores values as given: its scale (layer %d) must be 1, got %g",
                        l, (double)vs[l]);
    }

    const size_t tile = (size_t)block_size * (size_t)head_dim;
    const size_t pool_elems = (size_t)num_blocks * (size_t)num_kv_heads * tile;
    if (pool_elems / tile / (size_t)num_kv_heads != (size_t)num_blocks)
        return fail(KVF8_E_INVALID, "pool size overflows");

    kvf8_cache *c = new (std::nothrow) kvf8_cache();
    if (!c) return fail(KVF8_E_NOMEM, "host allocation of the cache handle failed");
    c->layers = num_layers;
    c->num_blocks = num_blocks;
    c->block_size = block_size;
    c->kv_heads = num_kv_heads;
    c->head_dim = head_dim;
    c->k_eb = elem_bytes(k_elem);
    c->v_eb = elem_bytes(v_elem);
    c->k_pool_bytes = pool_elems * (size_t)c->k_eb;
    c->v_pool_bytes = pool_elems * (size_t)c->v_eb;
    c->k_scale = ks;
    c->v_scale = vs;
    c->k_inv.resize(num_layers);
    c->v_inv.resize(num_layers);
    for (int32_t l = 0; l < num_layers; ++l) {
        c->k_inv[l] = 1.0f / ks[l];
        c->v_inv[l] = 1.0f / vs[l];
    }
    try {
        c->free_list.resize((size_t)num_blocks);
        c->allocated.assign((size_t)num_blocks, 0);
    } catch (...) {
        delete c;
        return fail(KVF8_E_NOMEM, "host allocation of the block free list failed");
    }
    for (int64_t i = 0; i < num_blocks; ++i) c->free_list[(size_t)i] = (int32_t)(num_blocks - 1 - i);

    if (k_pool) {
        c->k_base = static_cast<uint8_t *>(k_pool);
        c->v_base = static_cast<uint8_t *>(v_pool);
        c->owned = false;
        *out = c;
        return ok();
    }
    hipError_t e = hipGetDevice(&c->device);
    if (e != hipSuccess) {
        delete c;
        return hip_fail(e, "hipGetDevice");
    }
    const size_t k_total = c->k_pool_bytes * (size_t)num_layers;
    const size_t v_total = c->v_pool_bytes * (size_t)num_layers;
    e = hipMalloc(reinterpret_cast<void **>(&c->k_base), k_total);
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&c->v_base), v_total);
    if (e == hipSuccess) e = hipMemset(c->k_base, 0, k_total);
    if (e == hipSuccess) e = hipMemset(c->v_base, 0, v_total);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        const bool oom = e == hipErrorOutOfMemory;
        if (c->k_base) (void)hipFree(c->k_base);
        if (c->v_base) (void)hipFree(c->v_base);
        delete c;
        if (oom) return fail(KVF8_E_NOMEM, "device allocation of %zu + %zu pool bytes failed", k_total, v_total);
        return hip_fail(e, "allocating and clearing the pools");
    }
    c->owned = true;
    {   // set up the no-allocation decode's scratch on this device now (its
        // first call would otherwise); a failure here is reported by that call
        void *ws = nullptr;
        (void)kvf8::noalloc_scratch(c->device, &ws);
    }
    *out = c;
    return ok();
}

kvf8_status kv_cache_free(kvf8_cache *c) {
    if (!c) return ok();
    hipError_t e = hipSuccess;
    if (c->owned) {
        hipError_t e1 = hipFree(c->k_base);
        hipError_t e2 = hipFree(c->v_base);
        e = e1 != hipSuccess ? e1 : e2;
    }
    if (c->check_state) {
        hipError_t e3 = hipFree(c->check_state);
        if (e == hipSuccess) e = e3;
    }
    delete c;
    if (e != hipSuccess) return hip_fail(e, "hipFree");
    return ok();
}

kvf8_status kv_cache_set_checked(kvf8_cache *c, int32_t on) {
    if (!c) return fail(KVF8_E_INVALID, "cache is NULL");
    if (on) {
        if (!c->check_state) {
            const int64_t words = (c->num_blocks * c->block_size + 31) / 32;
            hipError_t e = hipMalloc(reinterpret_cast<void **>(&c->check_state), (size_t)(words + 1) * sizeof(uint32_t));
            if (e != hipSuccess) {
                c->check_state = nullptr;
                (void)hipGetLastError();
                return fail(KVF8_E_NOMEM, "checked mode: %lld bytes of check state: %s",
                            (long long)((words + 1) * 4), hipGetErrorString(e));
            }
            c->check_bitmap_words = words;
        }
        c->checked = true;
        return ok();
    }
    c->checked = false;
    if (c->check_state) {
        hipError_t e = hipFree(c->check_state);
        c->check_state = nullptr;
        c->check_bitmap_words = 0;
        if (e != hipSuccess) return hip_fail(e, "hipFree");
    }
    return ok();
}

kvf8_status kv_cache_set_scales(kvf8_cache *c, int32_t layer, const void *k_scale,
                                const void *v_scale, kvf8_dtype scale_dtype) {
    kvf8_status st = check_layer(c, layer);
    if (st != KVF8_OK) return st;
    if (scale_dtype != KVF8_DTYPE_F32 && scale_dtype != KVF8_DTYPE_BF16)
        return fail(KVF8_E_INVALID, "scale_dtype must be KVF8_DTYPE_F32 or KVF8_DTYPE_BF16");
    float ks = c->k_scale[layer], vs = c->v_scale[layer];
    if (k_scale) ks = read_scale(k_scale, 0, scale_dtype);
    if (v_scale) vs = read_scale(v_scale, 0, scale_dtype);
    if (!scale_usable(ks))
        return fail(KVF8_E_SCALE, "FP8 cache scale of layer %d (K) must be finite and nonzero with a finite reciprocal, got %g",
                    layer, (double)ks);
    if (!scale_usable(vs))
        return fail(KVF8_E_SCALE, "FP8 cache scale of layer %d (V) must be finite and nonzero with a finite reciprocal, got %g",
                    layer, (double)vs);
    if (c->k_eb == 2 && ks != 1.0f)
        return fail(KVF8_E_SCALE, "the bf16 K pool stores values as given: its scale must be 1, got %g", (double)ks);
    if (c->v_eb == 2 && vs != 1.0f)
        return fail(KVF8_E_SCALE, "the bf16 V pool stores values as given: its scale must be 1, got %g", (double)vs);
    c->k_scale[layer] = ks;
    c->v_scale[layer] = vs;
    c->k_inv[layer] = 1.0f / ks;
    c->v_inv[layer] = 1.0f / vs;
    return ok();
}

kvf8_status kv_cache_get_scales(const kvf8_cache *c, int32_t layer, float *k_scale, float *v_scale) {
    kvf8_status st = check_layer(c, layer);
    if (st != KVF8_OK) return st;
    if (k_scale) *k_scale = c->k_scale[layer];
    if (v_scale) *v_scale = c->v_scale[layer];
    return ok();
}

kvf8_status kv_cache_pools(const kvf8_cache *c, int32_t layer, uint8_t **k_pool, uint8_t **v_pool,
                           size_t *pool_bytes) {
    kvf8_status st = check_layer(c, layer);
    if (st != KVF8_OK) return st;
    if (k_pool) *k_pool = k_pool_of(c, layer);
    if (v_pool) *v_pool = v_pool_of(c, layer);
    if (pool_bytes) *pool_bytes = c->k_pool_bytes;
    return ok();
}

kvf8_status kv_cache_elem_types(const kvf8_cache *c, kvf8_elem *k_elem, kvf8_elem *v_elem) {
    if (!c) return fail(KVF8_E_INVALID, "cache is NULL");
    if (k_elem) *k_elem = c->k_eb == 2 ? KVF8_ELEM_BF16 : KVF8_ELEM_E4M3;
    if (v_elem) *v_elem = c->v_eb == 2 ? KVF8_ELEM_BF16 : KVF8_ELEM_E4M3;
    return ok();
}

kvf8_status kv_block_alloc(kvf8_cache *c, int32_t n, int32_t *ids_out) {
    if (!c) return fail(KVF8_E_INVALID, "cache is NULL");
    if (n < 0) return fail(KVF8_E_INVALID, "n must be >= 0");
    if (n > 0 && !ids_out) return fail(KVF8_E_INVALID, "ids_out is NULL");
    if ((size_t)n > c->free_list.size())
        return fail(KVF8_E_NOBLOCKS, "requested %d blocks, %zu free", n, c->free_list.size());
    for (int32_t i = 0; i < n; ++i) {
        int32_t id = c->free_list.back();
        c->free_list.pop_back();
        c->allocated[(size_t)id] = 1;
        ids_out[i] = id;
    }
    return ok();
}

kvf8_status kv_block_free(kvf8_cache *c, const int32_t *ids, int32_t n) {
    if (!c) return fail(KVF8_E_INVALID, "cache is NULL");
    if (n < 0) return fail(KVF8_E_INVALID, "n must be >= 0");
    if (n > 0 && !ids) return fail(KVF8_E_INVALID, "ids is NULL");
    // validate everything first so that a failed call returns nothing
    std::vector<uint8_t> seen;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t id = ids[i];
        if (id < 0 || (int64_t)id >= c->num_blocks)
            return fail(KVF8_E_INVALID, "block id %d out of range [0, %lld)", id, (long long)c->num_blocks);
        if (!c->allocated[(size_t)id])
            return fail(KVF8_E_INVALID, "block id %d is not allocated (double free?)", id);
    }
    if (n > 1) {
        seen.assign((size_t)c->num_blocks, 0);
        for (int32_t i = 0; i < n; ++i) {
            if (seen[(size_t)ids[i]]) return fail(KVF8_E_INVALID, "block id %d repeated in one free", ids[i]);
            seen[(size_t)ids[i]] = 1;
        }
    }
    for (int32_t i = 0; i < n; ++i) {
        c->allocated[(size_t)ids[i]] = 0;
        c->free_list.push_back(ids[i]);
    }
    return ok();
}

int64_t kv_blocks_free(const kvf8_cache *c) {
    if (!c) return -1;
    return (int64_t)c->free_list.size();
}

kvf8_status kv_block_shuffle(kvf8_cache *c, uint64_t seed) {
    if (!c) return fail(KVF8_E_INVALID, "cache is NULL");
    uint64_t st = seed;
    for (size_t i = c->free_list.size(); i > 1; --i) {
        const size_t j = (size_t)(splitmix64(st) % i);
        std::swap(c->free_list[i - 1], c->free_list[j]);
    }
    return ok();
}

kvf8_status kv_store_fp8(kvf8_cache *c, int32_t layer, const uint16_t *k_bf16,
                         const uint16_t *v_bf16, int64_t k_tok_stride, int64_t v_tok_stride,
                         const int64_t *slot_mapping, int64_t num_tokens, void *stream) {
    kvf8_status st = check_layer(c, layer);
    if (st != KVF8_OK) return st;
    if (num_tokens < 0) return fail(KVF8_E_INVALID, "num_tokens must be >= 0");
    if (num_tokens == 0) return ok();
    if (!k_bf16 || !v_bf16 || !slot_mapping)
        return fail(KVF8_E_INVALID, "k, v and slot_mapping must be non-NULL");
    const int64_t row = (int64_t)c->kv_heads * c->head_dim;
    if (k_tok_stride < row || v_tok_stride < row)
        return fail(KVF8_E_INVALID, "token strides (%lld, %lld) must be >= num_kv_heads*head_dim = %lld",
                    (long long)k_tok_stride, (long long)v_tok_stride, (long long)row);
    if ((k_tok_stride % 8) != 0 || (v_tok_stride % 8) != 0 ||
        (reinterpret_cast<uintptr_t>(k_bf16) % 16) != 0 || (reinterpret_cast<uintptr_t>(v_bf16) % 16) != 0)
        return fail(KVF8_E_INVALID, "K/V rows must be 16-byte aligned (pointers 16-byte aligned, strides multiples of 8 elements)");
    kvf8::StoreArgs a{};
    a.k = k_bf16;
    a.v = v_bf16;
    a.k_stride = k_tok_stride;
    a.v_stride = v_tok_stride;
    a.slots = slot_mapping;
    a.num_tokens = num_tokens;
    a.pool_slots = c->num_blocks * c->block_size;
    a.k_pool = k_pool_of(c, layer);
    a.v_pool = v_pool_of(c, layer);
    a.k_inv = c->k_inv[layer];
    a.v_inv = c->v_inv[layer];
    a.k_eb = c->k_eb;
    a.v_eb = c->v_eb;
    a.kv_heads = c->kv_heads;
    a.head_dim = c->head_dim;
    a.block_size = c->block_size;
    st = check_slot_list(c, slot_mapping, num_tokens, static_cast<hipStream_t>(stream));
    if (st != KVF8_OK) return st;
    hipError_t e = kvf8::launch_store(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "kv_store_fp8 launch");
    return ok();
}

size_t paged_attn_decode_workspace(const kvf8_cache *c, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t max_seq_len) {
    if (!c || num_seqs <= 0 || num_q_heads <= 0 || max_seq_len < 0) return 0;
    int32_t splits = 1, chunk = 0;
    kvf8::decode_plan(num_seqs, c->kv_heads, c->head_dim, c->block_size, max_seq_len, &splits, &chunk);
    if (splits <= 1) return 0;
    return (size_t)num_seqs * (size_t)num_q_heads * (size_t)splits * (size_t)(c->head_dim + 2) * sizeof(float);
}

namespace {

kvf8_status decode_call(kvf8_cache *c, int32_t layer, const uint16_t *q_bf16, int32_t num_q_heads,
                        const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *seq_lens,
                        int32_t num_seqs, int32_t max_seq_len, float sm_scale, void *out, kvf8_dtype out_dtype,
                        void *workspace, size_t workspace_bytes, void *stream) {
    kvf8_status st = check_layer(c, layer);
    if (st != KVF8_OK) return st;
    if (num_seqs < 0 || max_seq_len < 0 || max_blocks_per_seq < 0)
        return fail(KVF8_E_INVALID, "num_seqs, max_seq_len and max_blocks_per_seq must be >= 0");
    if (num_q_heads <= 0 || num_q_heads % c->kv_heads != 0)
        return fail(KVF8_E_INVALID, "num_q_heads %d must be a positive multiple of num_kv_heads %d",
                    num_q_heads, c->kv_heads);
    if (num_q_heads / c->kv_heads > 16)
        return fail(KVF8_E_UNSUPPORTED, "query-group size %d exceeds 16", num_q_heads / c->kv_heads);
    if (!(std::isfinite(sm_scale) && sm_scale > 0.0f))
        return fail(KVF8_E_INVALID, "sm_scale must be finite and > 0");
    if (out_dtype != KVF8_DTYPE_F32 && out_dtype != KVF8_DTYPE_BF16)
        return fail(KVF8_E_INVALID, "out_dtype must be KVF8_DTYPE_F32 or KVF8_DTYPE_BF16");
    if ((int64_t)max_seq_len > (int64_t)max_blocks_per_seq * c->block_size)
        return fail(KVF8_E_INVALID, "max_seq_len %d exceeds max_blocks_per_seq * block_size", max_seq_len);
    if (num_seqs == 0) return ok();
    if (!q_bf16 || !block_tables || !seq_lens || !out)
        return fail(KVF8_E_INVALID, "q, block_tables, seq_lens and out must be non-NULL");
    if ((reinterpret_cast<uintptr_t>(q_bf16) % 16) != 0)
        return fail(KVF8_E_INVALID, "q must be 16-byte aligned");
    int32_t splits = 1, chunk = 0;
    kvf8::decode_plan(num_seqs, c->kv_heads, c->head_dim, c->block_size, max_seq_len, &splits, &chunk);
    // one workgroup per (sequence, kv head, split), pairs padded to a multiple of 8
    const int64_t units = (int64_t)splits * ((((int64_t)num_seqs * c->kv_heads) + 7) / 8 * 8);
    if (units * kvf8::kDecodeThreads >= ((int64_t)1 << 32))
        return fail(KVF8_E_UNSUPPORTED, "%lld decode workgroups exceed one launch", (long long)units);
    const size_t need = paged_attn_decode_workspace(c, num_seqs, num_q_heads, max_seq_len);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(KVF8_E_INVALID, "workspace of %zu bytes is too small, %zu needed", workspace_bytes, need);
    kvf8::DecodeArgs a{};
    a.q = q_bf16;
    a.k_pool = k_pool_of(c, layer);
    a.v_pool = v_pool_of(c, layer);
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.out = out;
    a.partials = need > 0 ? static_cast<float *>(workspace) : nullptr;
    a.num_blocks = c->num_blocks;
    a.max_blocks = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.q_heads = num_q_heads;
    a.kv_heads = c->kv_heads;
    a.head_dim = c->head_dim;
    a.block_size = c->block_size;
    a.splits = splits;
    a.chunk_tokens = chunk;
    a.qk_scale = c->k_scale[layer] * sm_scale * 1.4426950408889634f;
    if (!(std::isfinite(a.qk_scale) && a.qk_scale != 0.0f))
        return fail(KVF8_E_SCALE, "k_scale * sm_scale * log2(e) = %g is not a finite nonzero fp32 factor",
                    (double)a.qk_scale);
    a.v_scale = c->v_scale[layer];
    a.out_bf16 = out_dtype == KVF8_DTYPE_BF16;
    a.k_eb = c->k_eb;
    a.v_eb = c->v_eb;
    {
        kvf8::CheckTablesArgs ca{};
        ca.block_tables = block_tables;
        ca.seq_lens = seq_lens;
        ca.num_blocks = c->num_blocks;
        ca.max_blocks = max_blocks_per_seq;
        ca.num_seqs = num_seqs;
        ca.block_size = c->block_size;
        ca.max_len = max_seq_len;
        st = check_table_args(c, ca, static_cast<hipStream_t>(stream));
        if (st != KVF8_OK) return st;
    }
    hipError_t e = kvf8::launch_decode(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "paged_attn_decode launch");
    return ok();
}

}  // namespace

kvf8_status paged_attn_decode(kvf8_cache *c, int32_t layer, const uint16_t *q_bf16,
                              int32_t num_q_heads, const int32_t *block_tables,
                              int32_t max_blocks_per_seq, const int32_t *seq_lens,
                              int32_t num_seqs, int32_t max_seq_len, float sm_scale, void *out,
                              kvf8_dtype out_dtype, void *workspace, size_t workspace_bytes,
                              void *stream) {
    return decode_call(c, layer, q_bf16, num_q_heads, block_tables, max_blocks_per_seq, seq_lens, num_seqs,
                       max_seq_len, sm_scale, out, out_dtype, workspace, workspace_bytes, stream);
}

kvf8_status paged_attn_decode_noalloc(kvf8_cache *c, int32_t layer, const uint16_t *q_bf16,
                                      int32_t num_q_heads, const int32_t *block_tables,
                                      int32_t max_blocks_per_seq, const int32_t *seq_lens,
                                      int32_t num_seqs, int32_t max_seq_len, float sm_scale, void *out,
                                      kvf8_dtype out_dtype, void *stream) {
    kvf8_status st = check_layer(c, layer);
    if (st != KVF8_OK) return st;
    // 0 for shapes that need no workspace and for invalid arguments, which
    // decode_call then rejects with their own message
    const size_t need = paged_attn_decode_workspace(c, num_seqs, num_q_heads, max_seq_len);
    if (need > kvf8::kNoAllocScratchBytes)
        return fail(KVF8_E_UNSUPPORTED,
                    "this decode needs %zu bytes of split-K workspace; paged_attn_decode_noalloc holds %zu "
                    "(use paged_attn_decode with a workspace)",
                    need, kvf8::kNoAllocScratchBytes);
    void *ws = nullptr;
    if (need > 0) {
        int dev = 0;
        hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
        if (e == hipSuccess) e = kvf8::noalloc_scratch(dev, &ws);
        if (e != hipSuccess) return hip_fail(e, "device scratch of paged_attn_decode_noalloc");
    }
    return decode_call(c, layer, q_bf16, num_q_heads, block_tables, max_blocks_per_seq, seq_lens, num_seqs,
                       max_seq_len, sm_scale, out, out_dtype, ws, need, stream);
}

kvf8_status paged_attn_prefill_chunk(kvf8_cache *c, int32_t layer, const uint16_t *q_bf16,
                                     int32_t num_q_heads, const int32_t *cu_q_lens,
                                     const int32_t *context_lens, const int32_t *block_tables,
                                     int32_t max_blocks_per_seq, int32_t num_seqs, int64_t total_q,
                                     int32_t max_q_len, int32_t max_ctx_len, float sm_scale,
                                     void *out, kvf8_dtype out_dtype, void *stream) {
    kvf8_status st = check_layer(c, layer);
    if (st != KVF8_OK) return st;
    if (num_seqs < 0 || total_q < 0 || max_q_len < 0 || max_ctx_len < 0 || max_blocks_per_seq < 0)
        return fail(KVF8_E_INVALID, "sizes must be >= 0");
    if (num_q_heads <= 0 || num_q_heads % c->kv_heads != 0)
        return fail(KVF8_E_INVALID, "num_q_heads %d must be a positive multiple of num_kv_heads %d",
                    num_q_heads, c->kv_heads);
    if (num_q_heads / c->kv_heads > 16)
        return fail(KVF8_E_UNSUPPORTED, "query-group size %d exceeds 16", num_q_heads / c->kv_heads);
    if (!(std::isfinite(sm_scale) && sm_scale > 0.0f))
        return fail(KVF8_E_INVALID, "sm_scale must be finite and > 0");
    if (out_dtype != KVF8_DTYPE_F32 && out_dtype != KVF8_DTYPE_BF16)
        return fail(KVF8_E_INVALID, "out_dtype must be KVF8_DTYPE_F32 or KVF8_DTYPE_BF16");
    if ((int64_t)max_q_len > (int64_t)max_blocks_per_seq * c->block_size)
        return fail(KVF8_E_INVALID, "max_q_len exceeds max_blocks_per_seq * block_size");
    if (num_seqs == 0 || total_q == 0) return ok();
    if (!q_bf16 || !cu_q_lens || !context_lens || !block_tables || !out)
        return fail(KVF8_E_INVALID, "q, cu_q_lens, context_lens, block_tables and out must be non-NULL");
    if ((reinterpret_cast<uintptr_t>(q_bf16) % 16) != 0)
        return fail(KVF8_E_INVALID, "q must be 16-byte aligned");
    {   // one workgroup per (sequence, kv head, 128-row query tile), pairs padded to a multiple of 8
        const int64_t tok_per_tile = kvf8::kPrefillRows / (num_q_heads / c->kv_heads);
        const int64_t units = ((int64_t)max_q_len + tok_per_tile - 1) / tok_per_tile *
                              ((((int64_t)num_seqs * c->kv_heads) + 7) / 8 * 8);
        if (units * kvf8::kPrefillThreads >= ((int64_t)1 << 32))
            return fail(KVF8_E_UNSUPPORTED, "%lld prefill workgroups exceed one launch", (long long)units);
    }
    kvf8::PrefillArgs a{};
    a.q = q_bf16;
    a.k_pool = k_pool_of(c, layer);
    a.v_pool = v_pool_of(c, layer);
    a.cu_q_lens = cu_q_lens;
    a.context_lens = context_lens;
    a.block_tables = block_tables;
    a.out = out;
    a.num_blocks = c->num_blocks;
    a.max_blocks = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.q_heads = num_q_heads;
    a.kv_heads = c->kv_heads;
    a.head_dim = c->head_dim;
    a.block_size = c->block_size;
    a.max_q_len = max_q_len;
    a.qk_scale = c->k_scale[layer] * sm_scale * 1.4426950408889634f;
    if (!(std::isfinite(a.qk_scale) && a.qk_scale != 0.0f))
        return fail(KVF8_E_SCALE, "k_scale * sm_scale * log2(e) = %g is not a finite nonzero fp32 factor",
                    (double)a.qk_scale);
    a.v_scale = c->v_scale[layer];
    a.out_bf16 = out_dtype == KVF8_DTYPE_BF16;
    a.k_eb = c->k_eb;
    a.v_eb = c->v_eb;
    {
        kvf8::CheckTablesArgs ca{};
        ca.block_tables = block_tables;
        ca.cu_q_lens = cu_q_lens;
        ca.context_lens = context_lens;
        ca.num_blocks = c->num_blocks;
        ca.total_q = total_q;
        ca.max_blocks = max_blocks_per_seq;
        ca.num_seqs = num_seqs;
        ca.block_size = c->block_size;
        ca.max_q_len = max_q_len;
        ca.max_ctx_len = max_ctx_len;
        st = check_table_args(c, ca, static_cast<hipStream_t>(stream));
        if (st != KVF8_OK) return st;
    }
    hipError_t e = kvf8::launch_prefill(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "paged_attn_prefill_chunk launch");
    return ok();
}

}  // extern "C"

namespace {
// Angle of rotary pair i for a position delta: a_i = delta * theta^(-2i/rot),
// cos/sin in double rounded to fp32 (the contract stated in kvfp8.h).
void rope_angle(int32_t delta, float theta_base, int32_t rot_dim, int32_t i, float &c, float &s) {
    const double omega = std::pow((double)theta_base, -2.0 * (double)i / (double)rot_dim);
    const double ang = (double)delta * omega;
    c = (float)std::cos(ang);
    s = (float)std::sin(ang);
}

kvf8_status check_rope(const kvf8_cache *c, float theta_base, int32_t rot_dim, kvf8_rope style) {
    if (rot_dim < 2 || (rot_dim % 2) != 0 || rot_dim > c->head_dim)
        return fail(KVF8_E_INVALID, "rot_dim %d must be even and in [2, head_dim=%d]", rot_dim, c->head_dim);
    if (!(std::isfinite(theta_base) && theta_base > 0.0f))
        return fail(KVF8_E_INVALID, "theta_base must be finite and > 0");
    if (style != KVF8_ROPE_NORM && style != KVF8_ROPE_NEOX)
        return fail(KVF8_E_INVALID, "style must be KVF8_ROPE_NORM or KVF8_ROPE_NEOX");
    return KVF8_OK;
}
}  // namespace

extern "C" {

kvf8_status kv_shift_rope(kvf8_cache *c, int32_t layer, const int64_t *slots, int64_t n_slots,
                          int32_t delta, float theta_base, int32_t rot_dim, kvf8_rope style,
                          void *stream) {
    kvf8_status st = check_layer(c, layer);
    if (st != KVF8_OK) return st;
    if (n_slots < 0) return fail(KVF8_E_INVALID, "n_slots must be >= 0");
    st = check_rope(c, theta_base, rot_dim, style);
    if (st != KVF8_OK) return st;
    if (n_slots == 0) return ok();
    if (!slots) return fail(KVF8_E_INVALID, "slots is NULL");
    kvf8::KShiftArgs a{};
    a.k_pool = k_pool_of(c, layer);
    a.slots = slots;
    a.n_slots = n_slots;
    a.pool_slots = c->num_blocks * c->block_size;
    a.kv_heads = c->kv_heads;
    a.head_dim = c->head_dim;
    a.block_size = c->block_size;
    a.rot_dim = rot_dim;
    a.neox = style == KVF8_ROPE_NEOX;
    a.k_eb = c->k_eb;
    for (int32_t i = 0; i < rot_dim / 2; ++i) rope_angle(delta, theta_base, rot_dim, i, a.cos_t[i], a.sin_t[i]);
    st = check_slot_list(c, slots, n_slots, static_cast<hipStream_t>(stream));
    if (st != KVF8_OK) return st;
    hipError_t e = kvf8::launch_kshift(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "kv_shift_rope launch");
    return ok();
}

kvf8_status kv_rope_table(const int32_t *deltas, int32_t n_deltas, float theta_base, int32_t rot_dim,
                          float *table) {
    if (n_deltas < 0) return fail(KVF8_E_INVALID, "n_deltas must be >= 0");
    if (rot_dim < 2 || (rot_dim % 2) != 0 || rot_dim > 256)
        return fail(KVF8_E_INVALID, "rot_dim %d must be even and in [2, 256]", rot_dim);
    if (!(std::isfinite(theta_base) && theta_base > 0.0f))
        return fail(KVF8_E_INVALID, "theta_base must be finite and > 0");
    if (n_deltas == 0) return ok();
    if (!deltas || !table) return fail(KVF8_E_INVALID, "deltas and table must be non-NULL");
    const int32_t half = rot_dim / 2;
    for (int32_t j = 0; j < n_deltas; ++j)
        for (int32_t i = 0; i < half; ++i)
            rope_angle(deltas[j], theta_base, rot_dim, i, table[((int64_t)j * half + i) * 2],
                       table[((int64_t)j * half + i) * 2 + 1]);
    return ok();
}

kvf8_status kv_shift_rope_per_slot(kvf8_cache *c, int32_t layer, const int64_t *slots, const int32_t *table_rows,
                                   int64_t n_slots, const float *table, int32_t n_rows, int32_t rot_dim,
                                   kvf8_rope style, void *stream) {
    kvf8_status st = check_layer(c, layer);
    if (st != KVF8_OK) return st;
    if (n_slots < 0) return fail(KVF8_E_INVALID, "n_slots must be >= 0");
    st = check_rope(c, 1.0f, rot_dim, style);
    if (st != KVF8_OK) return st;
    if (n_rows < 1) return fail(KVF8_E_INVALID, "n_rows must be >= 1");
    if (n_slots == 0) return ok();
    if (!slots || !table_rows || !table) return fail(KVF8_E_INVALID, "slots, table_rows and table must be non-NULL");
    if ((reinterpret_cast<uintptr_t>(table) % 16) != 0) return fail(KVF8_E_INVALID, "table must be 16-byte aligned");
    kvf8::KShiftArgs a{};
    a.k_pool = k_pool_of(c, layer);
    a.slots = slots;
    a.n_slots = n_slots;
    a.pool_slots = c->num_blocks * c->block_size;
    a.kv_heads = c->kv_heads;
    a.head_dim = c->head_dim;
    a.block_size = c->block_size;
    a.rot_dim = rot_dim;
    a.neox = style == KVF8_ROPE_NEOX;
    a.rows = table_rows;
    a.table = table;
    a.n_rows = n_rows;
    a.k_eb = c->k_eb;
    st = check_slot_list(c, slots, n_slots, static_cast<hipStream_t>(stream));
    if (st != KVF8_OK) return st;
    hipError_t e = kvf8::launch_kshift(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "kv_shift_rope_per_slot launch");
    return ok();
}

kvf8_status kv_calibrate_scales(const uint16_t *k_bf16, const uint16_t *v_bf16, int64_t k_tok_stride,
                                int64_t v_tok_stride, int64_t num_tokens, int64_t row_elems, float *amax,
                                void *scales_out, kvf8_dtype scale_dtype, void *stream) {
    if (!amax) return fail(KVF8_E_INVALID, "amax must be non-NULL");
    if ((reinterpret_cast<uintptr_t>(amax) % 4) != 0) return fail(KVF8_E_INVALID, "amax must be 4-byte aligned");
    if (num_tokens < 0) return fail(KVF8_E_INVALID, "num_tokens must be >= 0");
    if (row_elems <= 0 || row_elems % 8 != 0 || row_elems > (int64_t(1) << 31))
        return fail(KVF8_E_INVALID, "row_elems (%lld) must be a positive multiple of 8, at most 2^31",
                    (long long)row_elems);
    const uint16_t *xs[2] = {k_bf16, v_bf16};
    const int64_t strides[2] = {k_tok_stride, v_tok_stride};
    kvf8::CalibArgs a{};
    int32_t sides = 0;
    for (int t = 0; t < 2; ++t) {
        a.x[t] = xs[t];
        a.stride[t] = strides[t];
        if (!xs[t]) continue;
        if (strides[t] < row_elems || strides[t] % 8 != 0 || (reinterpret_cast<uintptr_t>(xs[t]) % 16) != 0)
            return fail(KVF8_E_INVALID,
                        "%s rows must be 16-byte aligned: pointer 16-byte aligned, stride (%lld) a multiple of 8 "
                        "and >= row_elems (%lld)", t ? "V" : "K", (long long)strides[t], (long long)row_elems);
        if (num_tokens > (int64_t(1) << 62) / strides[t])
            return fail(KVF8_E_INVALID, "num_tokens * stride must stay below 2^62");
        a.side[sides++] = t;
    }
    if (scales_out) {
        if (scale_dtype != KVF8_DTYPE_F32 && scale_dtype != KVF8_DTYPE_BF16)
            return fail(KVF8_E_INVALID, "scale_dtype must be KVF8_DTYPE_F32 or KVF8_DTYPE_BF16");
        const uintptr_t al = scale_dtype == KVF8_DTYPE_F32 ? 4 : 2;
        if ((reinterpret_cast<uintptr_t>(scales_out) % al) != 0)
            return fail(KVF8_E_INVALID, "scales_out must be aligned to its element size");
    }
    a.rows = num_tokens;
    a.runs_per_row = row_elems / 8;
    a.amax = reinterpret_cast<uint32_t *>(amax);
    hipError_t e = kvf8::launch_calibrate(a, num_tokens > 0 ? sides : 0, scales_out,
                                          scale_dtype == KVF8_DTYPE_BF16 ? 1 : 0, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "kv_calibrate_scales launch");
    return ok();
}

}  // extern "C"
