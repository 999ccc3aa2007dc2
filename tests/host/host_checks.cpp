// Host-side checks of the kvfp8 C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host side and run without a GPU: every
// path here stays in the library's host code (argument checks, scale intake,
// the block allocator, the angle table, error strings), using placeholder
// device addresses that are never dereferenced.
#include "kvfp8.h"

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

static int g_fail = 0;
#define EXPECT(cond)                                                          \
    do {                                                                      \
        if (!(cond)) {                                                        \
            std::fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond); \
            ++g_fail;                                                         \
        }                                                                     \
    } while (0)

static void *fake(uint64_t a) { return reinterpret_cast<void *>(a); }

static void allocator_and_scales() {
    const float ks[2] = {0.5f, 0.25f}, vs[2] = {0.125f, 2.0f};
    kvf8_cache *c = nullptr;
    EXPECT(kv_cache_alloc(2, 64, 16, 2, 64, ks, vs, KVF8_DTYPE_F32, fake(1ull << 40), fake(2ull << 40), &c) == KVF8_OK);
    EXPECT(c != nullptr);
    EXPECT(kv_blocks_free(c) == 64);
    std::vector<int32_t> ids(64);
    EXPECT(kv_block_alloc(c, 40, ids.data()) == KVF8_OK);
    EXPECT(kv_blocks_free(c) == 24);
    EXPECT(kv_block_alloc(c, 25, ids.data() + 40) == KVF8_E_NOBLOCKS);     // all or nothing
    EXPECT(kv_blocks_free(c) == 24);
    EXPECT(kv_block_free(c, ids.data(), 10) == KVF8_OK);
    EXPECT(kv_block_free(c, ids.data(), 1) == KVF8_E_INVALID);              // double free
    const int32_t bad = 64;
    EXPECT(kv_block_free(c, &bad, 1) == KVF8_E_INVALID);
    EXPECT(kv_block_shuffle(c, 12345) == KVF8_OK);
    EXPECT(kv_block_alloc(c, 34, ids.data()) == KVF8_OK);
    EXPECT(kv_blocks_free(c) == 0);
    float k = 0, v = 0;
    EXPECT(kv_cache_get_scales(c, 1, &k, &v) == KVF8_OK && k == 0.25f && v == 2.0f);
    const float zero = 0.0f, inf = INFINITY, nan_ = NAN, tiny = 1e-45f;
    EXPECT(kv_cache_set_scales(c, 0, &zero, nullptr, KVF8_DTYPE_F32) == KVF8_E_SCALE);
    EXPECT(kv_cache_set_scales(c, 0, &inf, nullptr, KVF8_DTYPE_F32) == KVF8_E_SCALE);
    EXPECT(kv_cache_set_scales(c, 0, nullptr, &nan_, KVF8_DTYPE_F32) == KVF8_E_SCALE);
    EXPECT(kv_cache_set_scales(c, 0, &tiny, nullptr, KVF8_DTYPE_F32) == KVF8_E_SCALE);   // 1/s overflows
    const uint16_t bf = 0x3F00;                                                           // bf16 0.5
    EXPECT(kv_cache_set_scales(c, 1, &bf, &bf, KVF8_DTYPE_BF16) == KVF8_OK);
    EXPECT(kv_cache_get_scales(c, 1, &k, &v) == KVF8_OK && k == 0.5f && v == 0.5f);
    EXPECT(kv_cache_set_scales(c, 2, &bf, &bf, KVF8_DTYPE_BF16) == KVF8_E_INVALID);       // layer
    uint8_t *kp = nullptr, *vp = nullptr;
    size_t bytes = 0;
    EXPECT(kv_cache_pools(c, 1, &kp, &vp, &bytes) == KVF8_OK && bytes == 64u * 2 * 16 * 64);
    EXPECT(kv_cache_free(c) == KVF8_OK);
    EXPECT(kv_bytes_per_block(16, 8, 128, 1) * 2 == kv_bytes_per_block(16, 8, 128, 2));
    EXPECT(kv_bytes_per_block(0, 8, 128, 1) == 0);
    // shapes and scales refused at allocation
    EXPECT(kv_cache_alloc(1, 8, 24, 2, 64, ks, vs, KVF8_DTYPE_F32, fake(1ull << 40), fake(2ull << 40), &c) != KVF8_OK);
    EXPECT(kv_cache_alloc(1, 8, 16, 2, 96, ks, vs, KVF8_DTYPE_F32, fake(1ull << 40), fake(2ull << 40), &c) != KVF8_OK);
    EXPECT(kv_cache_alloc(1, 8, 16, 2, 64, &zero, vs, KVF8_DTYPE_F32, fake(1ull << 40), fake(2ull << 40), &c) == KVF8_E_SCALE);
}

static void call_checks() {
    const float ks = 0.5f, vs = 0.5f;
    kvf8_cache *c = nullptr;
    EXPECT(kv_cache_alloc(1, 8, 16, 2, 64, &ks, &vs, KVF8_DTYPE_F32, fake(1ull << 40), fake(2ull << 40), &c) == KVF8_OK);
    const uint16_t *kb = static_cast<const uint16_t *>(fake(3ull << 40));
    const int64_t *sl = static_cast<const int64_t *>(fake(4ull << 40));
    EXPECT(kv_store_fp8(c, 0, kb, kb, 100, 128, sl, 4, nullptr) == KVF8_E_INVALID);     // stride below the row
    EXPECT(kv_store_fp8(c, 1, kb, kb, 128, 128, sl, 4, nullptr) == KVF8_E_INVALID);     // layer
    EXPECT(kv_store_fp8(c, 0, kb, kb, 128, 128, sl, 0, nullptr) == KVF8_OK);            // nothing to do
    EXPECT(kv_store_fp8(c, 0, nullptr, kb, 128, 128, sl, 4, nullptr) == KVF8_E_INVALID);
    const int32_t *t32 = static_cast<const int32_t *>(fake(5ull << 40));
    float *out = static_cast<float *>(fake(6ull << 40));
    EXPECT(paged_attn_decode(c, 0, kb, 3, t32, 4, t32, 2, 64, 0.125f, out, KVF8_DTYPE_F32, nullptr, 0, nullptr) ==
           KVF8_E_INVALID);                                                                  // 3 % 2 != 0
    EXPECT(paged_attn_decode(c, 0, kb, 4, t32, 4, t32, 2, 64, -1.0f, out, KVF8_DTYPE_F32, nullptr, 0, nullptr) !=
           KVF8_OK);                                                                         // sm_scale
    EXPECT(kv_shift_rope(c, 0, sl, 4, 1, 1e4f, 63, KVF8_ROPE_NEOX, nullptr) == KVF8_E_INVALID);
    EXPECT(kv_shift_rope(c, 0, sl, 4, 1, 0.0f, 64, KVF8_ROPE_NEOX, nullptr) == KVF8_E_INVALID);
    EXPECT(kv_cache_set_checked(nullptr, 1) == KVF8_E_INVALID);
    EXPECT(kv_calibrate_scales(kb, kb, 128, 128, 4, 12, static_cast<float *>(fake(7ull << 40)), nullptr,
                               KVF8_DTYPE_F32, nullptr) == KVF8_E_INVALID);            // row_elems % 8
    EXPECT(kv_cache_free(c) == KVF8_OK);
    EXPECT(kv_cache_free(nullptr) == KVF8_OK);
}

static void rope_table() {
    const int32_t deltas[3] = {-4096, 0, 7};
    std::vector<float> t(3 * 32 * 2);
    EXPECT(kv_rope_table(deltas, 3, 1e4f, 64, t.data()) == KVF8_OK);
    EXPECT(t[(1 * 32 + 5) * 2] == 1.0f && t[(1 * 32 + 5) * 2 + 1] == 0.0f);           // delta 0
    EXPECT(t[0] == (float)std::cos(-4096.0) && t[1] == (float)std::sin(-4096.0));      // pair 0 turns by delta
    EXPECT(kv_rope_table(deltas, 3, 1e4f, 258, t.data()) == KVF8_E_INVALID);
    EXPECT(kv_rope_table(deltas, 3, NAN, 64, t.data()) == KVF8_E_INVALID);
    EXPECT(kv_rope_table(nullptr, 0, 1e4f, 64, nullptr) == KVF8_OK);
}

static void thread_local_errors() {
    std::string a, b;
    std::thread t1([&] {
        (void)kv_block_alloc(nullptr, 1, nullptr);
        a = kvf8_last_error();
    });
    std::thread t2([&] {
        (void)kv_rope_table(nullptr, 1, 1e4f, 64, nullptr);
        b = kvf8_last_error();
    });
    t1.join();
    t2.join();
    EXPECT(!a.empty() && !b.empty() && a != b);
    EXPECT(std::strlen(kvf8_version()) > 0);
}

int main() {
    allocator_and_scales();
    call_checks();
    rope_table();
    thread_local_errors();
    if (g_fail) {
        std::fprintf(stderr, "%d host checks failed\n", g_fail);
        return 1;
    }
    std::printf("host checks passed\n");
    return 0;
}
