"""GPU parity of kv_store_fp8: cache bytes must equal the CPU oracle's bit for bit.

Covers every bf16 bit pattern at several scales (including a negative scale,
a tiny scale that lifts fp32 subnormals into range, and saturation) through
the 16-token run path (consecutive slots) and the token-by-token path
(shuffled slots), runs and broken runs in one call, both the four-token-group
and the single-token V write paths, negative slots,
padded token strides, untouched bytes, library-owned pools, small calls whose
kv-heads are split over several workgroups, and the store shapes of each
workload at reduced size.
"""
import ctypes

import numpy as np
import pytest
import torch

import fp8_e4m3_scaled_amd as kv
import oracle
from synth import Workload, bf16_bits
from tests.gpu_util import DEV, GpuCache, bits_dev, log, t_dev

pytestmark = pytest.mark.gpu

SCALES = [1.0, 0.5, 0.02, 0.015, 0.03, 6.0 / 448.0, 2.0 ** -7, 2.0 ** -13, 1e-30, 1e-38, -0.125, 3e4]


def _oracle_store(k_bits, v_bits, slots, NB, Hkv, D, BS, ks, vs, k_pool=None, v_pool=None):
    kp = np.zeros((NB, Hkv, BS * D), np.uint8) if k_pool is None else k_pool.copy()
    vp = np.zeros((NB, Hkv, BS * D), np.uint8) if v_pool is None else v_pool.copy()
    oracle.store(k_bits, v_bits, slots, kp, vp, Hkv=Hkv, D=D, BS=BS, k_scale=ks, v_scale=vs)
    return kp, vp


def _gpu_store(cache, k_bits, v_bits, slots, layer=0, stride=None):
    T = k_bits.shape[0]
    row = cache.Hkv * cache.D
    stride = row if stride is None else stride
    kd = torch.zeros((T, stride), dtype=torch.bfloat16, device=DEV)
    vd = torch.zeros((T, stride), dtype=torch.bfloat16, device=DEV)
    kd[:, :row] = bits_dev(k_bits.reshape(T, row))
    vd[:, :row] = bits_dev(v_bits.reshape(T, row))
    sd = t_dev(np.asarray(slots, np.int64))
    kv.kv_store_fp8(cache.handle, layer, kd, vd, stride, stride, sd, T)
    return cache.pools(layer)


def _all_patterns(T, Hkv, D):
    bits = np.arange(1 << 16, dtype=np.uint16)
    assert T * Hkv * D == bits.size
    return bits.reshape(T, Hkv, D), bits[::-1].copy().reshape(T, Hkv, D)


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("shuffled", [False, True])
def test_store_every_bf16_pattern(scale, shuffled):
    Hkv, D, BS = 2, 64, 16
    T = (1 << 16) // (Hkv * D)
    NB = T // BS
    k, v = _all_patterns(T, Hkv, D)
    slots = np.arange(T, dtype=np.int64)
    if shuffled:
        slots = np.random.default_rng(1).permutation(slots)
    log(f"store every bf16 pattern: scale={scale} shuffled={shuffled}")
    with GpuCache(NB, BS, Hkv, D, scale, -2.0 * scale if scale < 1e-20 else 1.5 * scale) as c:
        ks, vs = kv.kv_cache_get_scales(c.handle, 0)
        gk, gv = _gpu_store(c, k, v, slots)
    ok, ov = _oracle_store(k, v, slots, NB, Hkv, D, BS, ks, vs)
    assert np.array_equal(gk, ok), f"K bytes differ at {np.count_nonzero(gk != ok)} positions"
    assert np.array_equal(gv, ov), f"V bytes differ at {np.count_nonzero(gv != ov)} positions"


@pytest.mark.parametrize("BS,Hkv,D", [(16, 8, 128), (32, 2, 256), (16, 1, 64), (32, 3, 128)])
def test_store_negative_slots_padding_and_untouched_bytes(BS, Hkv, D):
    rng = np.random.default_rng(BS * D + Hkv)
    NB, T = 9, 37                      # ragged: not a multiple of four tokens
    k = rng.integers(0, 1 << 16, size=(T, Hkv, D), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, size=(T, Hkv, D), dtype=np.uint16)
    group = np.arange(40, 44)                       # one aligned four-token group
    others = np.setdiff1d(np.arange(NB * BS), group)
    slots = rng.choice(others, size=T, replace=False).astype(np.int64)   # no repeated slot
    slots[8:12] = group
    slots[[0, 5, 6, 36]] = -1
    assert len(set(slots[slots >= 0].tolist())) == int((slots >= 0).sum())
    log(f"store ragged/padded: BS={BS} Hkv={Hkv} D={D}")
    with GpuCache(NB, BS, Hkv, D, 0.07, 0.011, fill=0xA5) as c:
        ks, vs = kv.kv_cache_get_scales(c.handle, 0)
        gk, gv = _gpu_store(c, k, v, slots, stride=Hkv * D + 40)
    base = np.full((NB, Hkv, BS * D), 0xA5, np.uint8)
    ok, ov = _oracle_store(k, v, slots, NB, Hkv, D, BS, ks, vs, base, base)
    assert np.array_equal(gk, ok)
    assert np.array_equal(gv, ov)


@pytest.mark.parametrize("BS,Hkv,D", [(16, 8, 128), (32, 3, 256), (16, 1, 64), (32, 2, 128), (16, 3, 64)])
def test_store_sixteen_token_runs_and_broken_runs(BS, Hkv, D):
    """One call whose 16-token groups take both write paths: whole runs of 16
    consecutive slots from a multiple of 16 (block starts and the second half
    of a 32-token block) are written tile by tile; groups whose run is broken
    (a slot past the pool, a negative slot, a run starting 4 slots off, two
    slots exchanged, a last group of 9 tokens) go token by token.  Every byte
    must equal the oracle's, and untouched bytes keep their fill."""
    rng = np.random.default_rng(BS + Hkv + D)
    NB = 16
    Hs = NB * BS
    starts = [0, 16, BS * 5, BS * 7 + (16 if BS == 32 else 0)]
    groups = [np.arange(st, st + 16) for st in starts]
    g = np.arange(BS * 2, BS * 2 + 16)
    g[7] = Hs + 3                                   # past the pool: skipped
    groups.append(g)
    g = np.arange(BS * 3, BS * 3 + 16)
    g[0] = -1                                       # negative: skipped
    groups.append(g)
    groups.append(np.arange(BS * 12 + 4, BS * 12 + 20))  # consecutive, not 16-aligned
    g = np.arange(BS * 10, BS * 10 + 16)
    g[[3, 4]] = g[[4, 3]]                           # two slots exchanged
    groups.append(g)
    groups.append(np.arange(BS * 14, BS * 14 + 9))  # a last group of 9 tokens
    slots = np.concatenate(groups).astype(np.int64)
    valid = slots[(slots >= 0) & (slots < Hs)]
    assert len(set(valid.tolist())) == valid.size
    T = slots.size
    k = rng.integers(0, 1 << 16, size=(T, Hkv, D), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, size=(T, Hkv, D), dtype=np.uint16)
    log(f"store runs and broken runs: BS={BS} Hkv={Hkv} D={D} T={T}")
    with GpuCache(NB, BS, Hkv, D, 0.031, -0.007, fill=0x5A) as c:
        ks, vs = kv.kv_cache_get_scales(c.handle, 0)
        gk, gv = _gpu_store(c, k, v, slots)
    base = np.full((NB, Hkv, BS * D), 0x5A, np.uint8)
    ok, ov = _oracle_store(k, v, slots, NB, Hkv, D, BS, ks, vs, base, base)
    assert np.array_equal(gk, ok), f"K bytes differ at {np.count_nonzero(gk != ok)} positions"
    assert np.array_equal(gv, ov), f"V bytes differ at {np.count_nonzero(gv != ov)} positions"


@pytest.mark.parametrize("Hkv", [1, 3, 8])
@pytest.mark.parametrize("T", [1, 5, 16, 37, 64, 1000])
def test_store_small_calls_split_heads(Hkv, T):
    """Few tokens (a decode step: one token per sequence, scattered slots, or a
    short chunk of consecutive slots) spread each 16-token group's kv-heads over
    several workgroups; every head of every token must land exactly as the
    oracle stores it, and nothing else may change."""
    D, BS, NB = 64, 16, 160
    rng = np.random.default_rng(1000 * Hkv + T)
    if T % 2:
        slots = rng.choice(NB * BS, size=T, replace=False).astype(np.int64)
    else:
        start = BS * int(rng.integers(0, NB - T // BS - 1))
        slots = np.arange(start, start + T, dtype=np.int64)
    k = rng.integers(0, 1 << 16, size=(T, Hkv, D), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, size=(T, Hkv, D), dtype=np.uint16)
    log(f"store small call: Hkv={Hkv} T={T}")
    with GpuCache(NB, BS, Hkv, D, 0.02, 0.05, fill=0x3C) as c:
        ks, vs = kv.kv_cache_get_scales(c.handle, 0)
        gk, gv = _gpu_store(c, k, v, slots)
    base = np.full((NB, Hkv, BS * D), 0x3C, np.uint8)
    ok, ov = _oracle_store(k, v, slots, NB, Hkv, D, BS, ks, vs, base, base)
    assert np.array_equal(gk, ok), f"K bytes differ at {np.count_nonzero(gk != ok)} positions"
    assert np.array_equal(gv, ov), f"V bytes differ at {np.count_nonzero(gv != ov)} positions"


def test_store_into_library_owned_pools():
    Hkv, D, BS, NB = 2, 128, 16, 6
    c = kv.kv_cache_alloc(2, NB, BS, Hkv, D, [0.25, 0.03], [0.5, 0.04])
    try:
        rng = np.random.default_rng(2)
        T = 40
        k = rng.integers(0, 1 << 16, size=(T, Hkv, D), dtype=np.uint16)
        v = rng.integers(0, 1 << 16, size=(T, Hkv, D), dtype=np.uint16)
        slots = rng.choice(NB * BS, size=T, replace=False).astype(np.int64)
        kd, vd, sd = bits_dev(k.reshape(T, -1)), bits_dev(v.reshape(T, -1)), t_dev(slots)
        log("store into library-owned pools, layer 1")
        kv.kv_store_fp8(c, 1, kd, vd, Hkv * D, Hkv * D, sd, T)
        torch.cuda.synchronize()
        hip = ctypes.CDLL("libamdhip64.so")
        hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        out = {}
        for layer in (0, 1):
            kp, vp, n = kv.kv_cache_pools(c, layer)
            hk, hv = np.empty(n, np.uint8), np.empty(n, np.uint8)
            assert hip.hipMemcpy(hk.ctypes.data, kp, n, 2) == 0
            assert hip.hipMemcpy(hv.ctypes.data, vp, n, 2) == 0
            out[layer] = (hk.reshape(NB, Hkv, -1), hv.reshape(NB, Hkv, -1))
        assert not out[0][0].any() and not out[0][1].any()      # zero-filled, untouched
        ok, ov = _oracle_store(k, v, slots, NB, Hkv, D, BS, np.float32(0.03), np.float32(0.04))
        assert np.array_equal(out[1][0], ok) and np.array_equal(out[1][1], ov)
    finally:
        kv.kv_cache_free(c)


@pytest.mark.parametrize("name,sd", [("tiny", 1), ("llama8b", 16), ("varlen", 16), ("prefill", 8),
                                     ("longctx", 256)])
def test_store_workloads_reduced(name, sd):
    w = Workload(name, scale_down=sd, pool_frac=0.0)
    ks, vs, dt = w.scales()
    log(f"store workload {name} scale_down={sd}: B={w.B} NB={w.NB}")
    with GpuCache(w.NB, w.BS, w.Hkv, w.D, float(ks), float(vs)) as c:
        ok = np.zeros((w.NB, w.Hkv, w.BS * w.D), np.uint8)
        ov = np.zeros_like(ok)
        for b in range(w.B):
            L = int(w.total_lengths[b])
            k, v = w.kv(b, 0, L)
            kb, vb = bf16_bits(k), bf16_bits(v)
            s = w.slots(b, 0, L)
            # the context first, then the step's new tokens, as two calls
            split = int(w.lengths[b])
            for lo, hi in ((0, split), (split, L)):
                if hi > lo:
                    _gpu_store(c, kb[lo:hi], vb[lo:hi], s[lo:hi])
            oracle.store(kb, vb, s, ok, ov, Hkv=w.Hkv, D=w.D, BS=w.BS, k_scale=ks, v_scale=vs)
        gk, gv = c.pools()
    assert np.array_equal(gk, ok)
    assert np.array_equal(gv, ov)
