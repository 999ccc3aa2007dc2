"""Routing defects that a comparison of two fp8 runs cannot see must turn the
comparison against the oracle red ([P3], "Round 4": only a reference catches
a read or write that is wired to the wrong place).  Each defect is planted in
how the library is called (a handle over swapped pools, swapped scales, slots
with their in-block offset dropped), never in the library, and every check
first shows the unmutated call green.

  store:   the pools' bytes must differ from the oracle's;
  prefill: the outputs must leave the attention tolerance.
"""
import numpy as np
import pytest
import torch

import fp8_e4m3_scaled_amd as kv
import oracle
from synth import Workload, bf16_bits
from tests.gpu_util import DEV, GpuCache, log, t_dev
from tests.test_gpu_decode import assert_close
from tests.test_gpu_prefill import Chunked

pytestmark = pytest.mark.gpu

KS, VS = 0.02, 0.15           # unequal, so that swapped scales change every byte's meaning


def _store_all(handle, w, slots_of):
    """Every sequence of w through kv_store_fp8 with slots_of(b, slots) as the slot list,
    one token per call (a mutation that maps two tokens to one slot stays defined)."""
    row = w.Hkv * w.D
    for b in range(w.B):
        L = int(w.lengths[b])
        k, v = w.kv(b, 0, L)
        s = slots_of(b, w.slots(b, 0, L))
        kd, vd = k.to(DEV).reshape(L, row), v.to(DEV).reshape(L, row)
        for i in range(L):
            kv.kv_store_fp8(handle, 0, kd[i:i + 1], vd[i:i + 1], row, row, t_dev(s[i:i + 1].copy()), 1)
    torch.cuda.synchronize()


def _oracle_pools(w):
    ok = np.zeros((w.NB, w.Hkv, w.BS * w.D), np.uint8)
    ov = np.zeros_like(ok)
    for b in range(w.B):
        L = int(w.lengths[b])
        k, v = w.kv(b, 0, L)
        oracle.store(bf16_bits(k), bf16_bits(v), w.slots(b, 0, L), ok, ov, Hkv=w.Hkv, D=w.D, BS=w.BS,
                     k_scale=np.float32(KS), v_scale=np.float32(VS))
    return ok, ov


def test_store_routing_mutations_are_caught():
    w = Workload("tiny")
    ok, ov = _oracle_pools(w)
    same = lambda b, s: s                                   # noqa: E731
    no_offset = lambda b, s: s - s % w.BS                   # noqa: E731
    for what, ks, vs, swap, slots_of, red in [
            ("unmutated", KS, VS, False, same, False),
            ("K/V pools swapped", KS, VS, True, same, True),
            ("scales swapped", VS, KS, False, same, True),
            ("in-block offset dropped", KS, VS, False, no_offset, True)]:
        log(f"store mutation: {what}")
        with GpuCache(w.NB, w.BS, w.Hkv, w.D, KS, VS) as c:
            h = kv.kv_cache_alloc(1, w.NB, w.BS, w.Hkv, w.D, [ks], [vs], kv.DTYPE_F32,
                                  c.v_pool if swap else c.k_pool, c.k_pool if swap else c.v_pool)
            try:
                _store_all(h, w, slots_of)
            finally:
                kv.kv_cache_free(h)
            gk, gv = c.pools()
        equal = np.array_equal(gk, ok) and np.array_equal(gv, ov)
        assert equal != red, f"store, {what}: bytes {'equal' if equal else 'differ'}"


def test_prefill_routing_mutations_are_caught():
    c = Chunked(8, 2, 64, 16, [40, 0, 75], [30, 51, 16], 7300, ks=KS, vs=VS)
    try:
        want = c.oracle()
        w = c.w
        assert_close(c.run(), want, "unmutated")
        pools = c.f.cache
        mutants = [("K/V pools swapped", [KS], [VS], pools.v_pool, pools.k_pool),
                   ("scales swapped", [VS], [KS], pools.k_pool, pools.v_pool)]
        for what, ks, vs, kp, vp in mutants:
            log(f"prefill mutation: {what}")
            h = kv.kv_cache_alloc(1, pools.NB, pools.BS, pools.Hkv, pools.D, ks, vs, kv.DTYPE_F32, kp, vp)
            try:
                c.f.cache.handle, keep = h, c.f.cache.handle
                got = c.run()
            finally:
                c.f.cache.handle = keep
                kv.kv_cache_free(h)
            with pytest.raises(AssertionError):
                assert_close(got, want, what)
        # the same sequences stored with their in-block offsets dropped, read through the right tables
        log("prefill mutation: in-block offset dropped")
        with GpuCache(w.NB, w.BS, w.Hkv, w.D, KS, VS) as bad:
            _store_all(bad.handle, w, lambda b, s: s - s % w.BS)
            c.f.cache.handle, keep = bad.handle, c.f.cache.handle
            try:
                got = c.run()
            finally:
                c.f.cache.handle = keep
        with pytest.raises(AssertionError):
            assert_close(got, want, "in-block offset dropped")
    finally:
        c.close()
