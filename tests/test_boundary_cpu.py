"""Host-side tests of the C ABI: the library loads, exports every declared
symbol, and every host-only path (scale intake, shape checks, the block
allocator, argument checks that fail before any launch) behaves as
include/kvfp8.h states.  No call here touches a GPU: pools are borrowed
placeholder addresses that are never dereferenced, and every compute call
made is one that fails its host-side checks.
"""
import ctypes
import math
import os
import re
import struct

import pytest

import fp8_e4m3_scaled_amd as kv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvfp8.h")
FAKE_K, FAKE_V = 1 << 40, 2 << 40      # borrowed placeholder "device" addresses


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_0-9]+)\s*\(", text)) - {"sizeof"})


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 17
    lib = ctypes.CDLL(kv.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(kv.SIGNATURES), "binding and header disagree"


def test_version_string():
    assert "gfx950" in kv.kvf8_version()


@pytest.mark.parametrize("bs,h,d", [(16, 2, 64), (16, 8, 128), (32, 2, 256), (32, 8, 128)])
def test_bytes_per_block_halved(bs, h, d):
    fp8 = kv.kv_bytes_per_block(bs, h, d, 1)
    assert fp8 == 2 * bs * h * d
    assert 2 * fp8 == kv.kv_bytes_per_block(bs, h, d, 2)
    assert kv.kv_bytes_per_block(0, h, d, 1) == 0 and kv.kv_bytes_per_block(bs, h, d, -1) == 0


def _cache(layers=2, nb=64, bs=16, h=2, d=64, ks=None, vs=None, dtype=kv.DTYPE_F32):
    return kv.kv_cache_alloc(layers, nb, bs, h, d, ks, vs, dtype, FAKE_K, FAKE_V)


def test_scales_default_to_one_and_pools_are_borrowed():
    c = _cache()
    try:
        assert kv.kv_cache_get_scales(c, 0) == (1.0, 1.0)
        k, v, n = kv.kv_cache_pools(c, 1)
        assert n == 64 * 2 * 16 * 64
        assert k == FAKE_K + n and v == FAKE_V + n
    finally:
        kv.kv_cache_free(c)


def test_bf16_scales_widen_exactly():
    # 0x3CA3 is bf16(0.02) = 0.019958...; 0x3C75 ~ 0.01495
    c = _cache(ks=[0x3CA3, 0x4000], vs=[0x3C75, 0xBE00], dtype=kv.DTYPE_BF16)
    try:
        k0, v0 = kv.kv_cache_get_scales(c, 0)
        assert struct.unpack("<I", struct.pack("<f", k0))[0] == 0x3CA30000
        assert struct.unpack("<I", struct.pack("<f", v0))[0] == 0x3C750000
        assert kv.kv_cache_get_scales(c, 1) == (2.0, -0.125)   # negative scales are allowed
    finally:
        kv.kv_cache_free(c)


@pytest.mark.parametrize("bad", [0.0, -0.0, math.inf, -math.inf, math.nan, 1e-45, 2.0 ** -129])
def test_bad_scales_rejected(bad):
    with pytest.raises(kv.KvF8Error) as ei:
        _cache(ks=[0.5, bad], vs=[0.5, 0.5])
    assert ei.value.status == kv.E_SCALE
    assert "layer 1 (K)" in str(ei.value)
    with pytest.raises(kv.KvF8Error) as ei:
        _cache(ks=[0.5, 0.5], vs=[bad, 0.5])
    assert ei.value.status == kv.E_SCALE and "layer 0 (V)" in str(ei.value)


def test_bad_bf16_scale_patterns_rejected():
    for bits in [0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0x0001]:   # 0, -0, inf, -inf, nan, subnormal
        with pytest.raises(kv.KvF8Error) as ei:
            _cache(ks=[0x3F80, bits], vs=[0x3F80, 0x3F80], dtype=kv.DTYPE_BF16)
        assert ei.value.status == kv.E_SCALE


def test_set_scales_checks_and_keeps_old_on_error():
    c = _cache(ks=[0.5, 0.5], vs=[0.25, 0.25])
    try:
        kv.kv_cache_set_scales(c, 1, 0.03, None)
        assert kv.kv_cache_get_scales(c, 1) == (pytest.approx(0.03), 0.25)
        with pytest.raises(kv.KvF8Error) as ei:
            kv.kv_cache_set_scales(c, 1, 0.125, math.nan)
        assert ei.value.status == kv.E_SCALE
        assert kv.kv_cache_get_scales(c, 1) == (pytest.approx(0.03), 0.25)
        with pytest.raises(kv.KvF8Error) as ei:
            kv.kv_cache_set_scales(c, 2, 0.1, 0.1)
        assert ei.value.status == kv.E_INVALID
    finally:
        kv.kv_cache_free(c)


@pytest.mark.parametrize("args", [
    (0, 64, 16, 2, 64), (1, 0, 16, 2, 64), (1, 64, 16, 0, 64), (1, 64, 8, 2, 64),
    (1, 64, 64, 2, 64), (1, 64, 16, 2, 96), (1, 64, 16, 2, 512), (1, 1 << 31, 16, 2, 64)])
def test_bad_shapes_rejected(args):
    with pytest.raises(kv.KvF8Error) as ei:
        kv.kv_cache_alloc(*args, None, None, kv.DTYPE_F32, FAKE_K, FAKE_V)
    assert ei.value.status == kv.E_INVALID


def test_mixed_pool_ownership_rejected():
    with pytest.raises(kv.KvF8Error) as ei:
        kv.kv_cache_alloc(1, 64, 16, 2, 64, None, None, kv.DTYPE_F32, FAKE_K, None)
    assert ei.value.status == kv.E_INVALID


def test_allocator_lifo_all_or_nothing_and_double_free():
    c = _cache(nb=8)
    try:
        assert kv.kv_blocks_free(c) == 8
        a = kv.kv_block_alloc(c, 3)
        assert a == [0, 1, 2]
        with pytest.raises(kv.KvF8Error) as ei:
            kv.kv_block_alloc(c, 6)
        assert ei.value.status == kv.E_NOBLOCKS
        assert kv.kv_blocks_free(c) == 5          # nothing taken by the failed call
        kv.kv_block_free(c, [1])
        assert kv.kv_block_alloc(c, 1) == [1]     # last freed, first out
        for bad in ([1, 1], [7], [-1], [8]):
            with pytest.raises(kv.KvF8Error) as ei:
                kv.kv_block_free(c, bad)
            assert ei.value.status == kv.E_INVALID
        assert kv.kv_blocks_free(c) == 5          # failed frees returned nothing
        kv.kv_block_free(c, a)
        assert kv.kv_blocks_free(c) == 8
    finally:
        kv.kv_cache_free(c)


def test_allocator_shuffle_is_seeded_permutation():
    outs = []
    for seed in (7, 7, 8):
        c = _cache(nb=1000)
        kv.kv_block_shuffle(c, seed)
        outs.append(kv.kv_block_alloc(c, 1000))
        kv.kv_cache_free(c)
    assert outs[0] == outs[1] != outs[2]
    assert sorted(outs[0]) == list(range(1000)) and outs[0] != list(range(1000))


def test_compute_calls_fail_their_host_checks():
    c = _cache(h=2, d=64)
    try:
        def dec(**kw):
            a = dict(cache=c, layer=0, q_bf16=1 << 30, num_q_heads=4, block_tables=1 << 30,
                     max_blocks_per_seq=4, seq_lens=1 << 30, num_seqs=2, max_seq_len=64,
                     sm_scale=0.125, out=1 << 30, out_dtype=kv.DTYPE_F32, stream=0)
            a.update(kw)
            with pytest.raises(kv.KvF8Error) as ei:
                kv.paged_attn_decode(**a)
            return ei.value.status
        assert dec(num_q_heads=3) == kv.E_INVALID                  # Hq % Hkv
        assert dec(num_q_heads=34) == kv.E_UNSUPPORTED              # group of 17
        assert dec(sm_scale=0.0) == kv.E_INVALID
        assert dec(sm_scale=math.nan) == kv.E_INVALID
        assert dec(layer=2) == kv.E_INVALID
        assert dec(max_seq_len=65) == kv.E_INVALID                 # beyond the table
        assert dec(out_dtype=7) == kv.E_INVALID
        assert dec(q_bf16=(1 << 30) + 2) == kv.E_INVALID            # misaligned q
        with pytest.raises(kv.KvF8Error) as ei:
            kv.kv_store_fp8(c, 0, 1 << 30, 1 << 30, 64, 128, 1 << 30, 4, 0)   # stride < H*D
        assert ei.value.status == kv.E_INVALID
        with pytest.raises(kv.KvF8Error) as ei:
            kv.kv_store_fp8(c, 0, None, 1 << 30, 128, 128, 1 << 30, 4, 0)
        assert ei.value.status == kv.E_INVALID
        kv.kv_store_fp8(c, 0, None, None, 128, 128, None, 0, 0)     # zero tokens: no-op
        for rot in (0, 3, 66):
            with pytest.raises(kv.KvF8Error) as ei:
                kv.kv_shift_rope(c, 0, 1 << 30, 4, -1, 1e4, rot, kv.ROPE_NEOX, 0)
            assert ei.value.status == kv.E_INVALID
        with pytest.raises(kv.KvF8Error) as ei:
            kv.kv_shift_rope(c, 0, 1 << 30, 4, -1, -1.0, 64, kv.ROPE_NEOX, 0)
        assert ei.value.status == kv.E_INVALID
        with pytest.raises(kv.KvF8Error) as ei:
            kv.paged_attn_prefill_chunk(c, 0, 1 << 30, 5, 1 << 30, 1 << 30, 1 << 30, 4, 1, 8, 8,
                                        16, 0.125, 1 << 30, kv.DTYPE_F32, 0)
        assert ei.value.status == kv.E_INVALID
    finally:
        kv.kv_cache_free(c)


def test_score_factor_must_be_a_usable_fp32():
    """k_scale * sm_scale * log2(e) must be finite and nonzero in fp32: a factor
    that underflows to 0 or overflows is refused before any launch."""
    for ks, sm in [(1e-38, 1e-10), (1e38, 1e10)]:
        c = _cache(h=2, d=64, ks=[ks, ks], vs=[1.0, 1.0])
        try:
            with pytest.raises(kv.KvF8Error) as ei:
                kv.paged_attn_decode(c, 0, 1 << 30, 4, 1 << 30, 4, 1 << 30, 2, 64, sm, 1 << 30,
                                     kv.DTYPE_F32, None, 0, 0)
            assert ei.value.status == kv.E_SCALE
            with pytest.raises(kv.KvF8Error) as ei:
                kv.paged_attn_prefill_chunk(c, 0, 1 << 30, 4, 1 << 30, 1 << 30, 1 << 30, 4, 1, 8, 8,
                                            16, sm, 1 << 30, kv.DTYPE_F32, 0)
            assert ei.value.status == kv.E_SCALE
        finally:
            kv.kv_cache_free(c)


def test_workspace_size_is_consistent():
    c = _cache(h=2, d=64)
    try:
        assert kv.paged_attn_decode_workspace(c, 0, 4, 64) == 0
        for L in (1, 64, 100000):
            n = kv.paged_attn_decode_workspace(c, 4, 4, L)
            assert n >= 0 and n % 4 == 0
    finally:
        kv.kv_cache_free(c)


@pytest.mark.parametrize("order", ["package_first", "torch_first"])
def test_one_hip_runtime_per_process(order):
    """Whatever the import order, the library and torch share one HIP runtime:
    two runtimes in one process make the second one see no device."""
    import subprocess
    import sys
    mods = ["fp8_e4m3_scaled_amd", "torch"]
    if order == "torch_first":
        mods.reverse()
    code = (
        "import importlib, sys\n"
        f"sys.path.insert(0, {os.path.dirname(os.path.dirname(os.path.abspath(__file__)))!r})\n"
        f"for m in {mods!r}: importlib.import_module(m)\n"
        "maps = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
        "print(len(maps), sorted(maps))\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    assert out.stdout.startswith("1 "), out.stdout


def test_typed_pools_host_rules():
    """Per-pool element types: bf16 pools keep scale 1, support head_dim <= 128, report
    their types and byte sizes."""
    E, B = kv.ELEM_E4M3, kv.ELEM_BF16
    with pytest.raises(kv.KvF8Error) as ei:
        kv.kv_cache_alloc_typed(1, 8, 16, 2, 64, B, E, [0.5], [0.5], kv.DTYPE_F32, FAKE_K, FAKE_V)
    assert ei.value.status == kv.E_SCALE                                   # bf16 K pool scale != 1
    with pytest.raises(kv.KvF8Error) as ei:
        kv.kv_cache_alloc_typed(1, 8, 16, 2, 256, E, B, None, None, kv.DTYPE_F32, FAKE_K, FAKE_V)
    assert ei.value.status == kv.E_UNSUPPORTED
    with pytest.raises(kv.KvF8Error) as ei:
        kv.kv_cache_alloc_typed(1, 8, 16, 2, 64, 7, E, None, None, kv.DTYPE_F32, FAKE_K, FAKE_V)
    assert ei.value.status == kv.E_INVALID
    for ke, ve in [(E, E), (E, B), (B, E), (B, B)]:
        c = kv.kv_cache_alloc_typed(2, 8, 16, 2, 64, ke, ve, [0.5, 1.0] if ke == E else None,
                                    [0.25, 1.0] if ve == E else None, kv.DTYPE_F32, FAKE_K, FAKE_V)
        try:
            assert kv.kv_cache_elem_types(c) == (ke, ve)
            k0, v0, nbytes = kv.kv_cache_pools(c, 0)
            k1, v1, _ = kv.kv_cache_pools(c, 1)
            ke_b, ve_b = (2 if ke == B else 1), (2 if ve == B else 1)
            assert nbytes == 8 * 2 * 16 * 64 * ke_b
            assert k1 - k0 == 8 * 2 * 16 * 64 * ke_b and v1 - v0 == 8 * 2 * 16 * 64 * ve_b
            if ke == B:
                with pytest.raises(kv.KvF8Error) as ei:
                    kv.kv_cache_set_scales(c, 0, 2.0, None)
                assert ei.value.status == kv.E_SCALE
        finally:
            kv.kv_cache_free(c)


def test_calibrate_host_checks():
    """Scale calibration refuses missing or misaligned state, ragged rows and bad scale
    types before launching anything."""
    A, X = 1 << 30, 1 << 31            # stand-in device addresses (never dereferenced)
    bad = [
        dict(amax=None),
        dict(amax=A + 2),
        dict(num_tokens=-1),
        dict(row_elems=0),
        dict(row_elems=12),
        dict(k=X + 8),                 # not 16-byte aligned
        dict(k_stride=1020),           # below row_elems
        dict(v_stride=1028),           # not a multiple of 8
        dict(scales_out=A + 64, scale_dtype=5),
        dict(scales_out=A + 66, scale_dtype=kv.DTYPE_F32),
        dict(num_tokens=1 << 60),
    ]
    base = dict(k=X, v=X + (1 << 28), k_stride=1024, v_stride=1024, num_tokens=4, row_elems=1024,
                amax=A, scales_out=None, scale_dtype=kv.DTYPE_F32)
    for change in bad:
        a = dict(base, **change)
        with pytest.raises(kv.KvF8Error) as ei:
            kv.kv_calibrate_scales(a["k"], a["v"], a["k_stride"], a["v_stride"], a["num_tokens"],
                                   a["row_elems"], a["amax"], a["scales_out"], a["scale_dtype"], 0)
        assert ei.value.status == kv.E_INVALID, change


def test_rope_table_equals_oracle_table():
    """The host cos/sin table behind the per-slot K-shift holds, for every delta,
    the same fp32 values as the oracle's own angle table (both take cos/sin of
    delta * theta^(-2i/rot) in double and round to fp32)."""
    import numpy as np
    import oracle
    deltas = [-131072, -4096, -1, 0, 1, 3, 17, 4096, 100000, 2 ** 31 - 1]
    for rot, theta in ((256, 1e6), (128, 5e5), (64, 1e4), (40, 1e4), (2, 1e4)):
        t = kv.kv_rope_table(deltas, theta, rot)
        assert t.shape == (len(deltas), rot // 2, 2)
        for j, d in enumerate(deltas):
            c, s = oracle.rope_table(rot, d, theta)
            assert np.array_equal(t[j, :, 0].view(np.uint32), c.view(np.uint32)), (rot, d)
            assert np.array_equal(t[j, :, 1].view(np.uint32), s.view(np.uint32)), (rot, d)
    assert kv.kv_rope_table([], 1e4, 64).shape == (0, 32, 2)
    for rot, theta in ((0, 1e4), (3, 1e4), (258, 1e4), (64, 0.0), (64, float("inf"))):
        with pytest.raises(kv.KvF8Error) as ei:
            kv.kv_rope_table([1], theta, rot)
        assert ei.value.status == kv.E_INVALID


def test_per_slot_shift_host_checks():
    """kv_shift_rope_per_slot validates before launching: rot_dim, style, table
    rows, pointers and table alignment; an empty slot list is a no-op."""
    h = kv.kv_cache_alloc(1, 8, 16, 2, 64, [0.5], [0.5], kv.DTYPE_F32, FAKE_K, FAKE_V)
    try:
        T, S, R = 1 << 33, 1 << 34, 1 << 35
        kv.kv_shift_rope_per_slot(h, 0, None, None, 0, None, 1, 64, kv.ROPE_NEOX, 0)
        for args in [(h, 1, S, R, 4, T, 1, 64, kv.ROPE_NEOX),          # layer
                     (h, 0, S, R, -1, T, 1, 64, kv.ROPE_NEOX),         # n_slots
                     (h, 0, S, R, 4, T, 1, 66, kv.ROPE_NEOX),          # rot_dim > head_dim
                     (h, 0, S, R, 4, T, 1, 63, kv.ROPE_NEOX),          # odd rot_dim
                     (h, 0, S, R, 4, T, 1, 64, 9),                     # style
                     (h, 0, S, R, 4, T, 0, 64, kv.ROPE_NEOX),          # n_rows
                     (h, 0, None, R, 4, T, 1, 64, kv.ROPE_NEOX),
                     (h, 0, S, None, 4, T, 1, 64, kv.ROPE_NEOX),
                     (h, 0, S, R, 4, None, 1, 64, kv.ROPE_NEOX),
                     (h, 0, S, R, 4, T + 8, 1, 64, kv.ROPE_NEOX)]:     # table alignment
            with pytest.raises(kv.KvF8Error) as ei:
                kv.kv_shift_rope_per_slot(*args, 0)
            assert ei.value.status == kv.E_INVALID, args
    finally:
        kv.kv_cache_free(h)


def test_checked_mode_needs_a_cache():
    with pytest.raises(kv.KvF8Error) as ei:
        kv.kv_cache_set_checked(None, True)
    assert ei.value.status == kv.E_INVALID
