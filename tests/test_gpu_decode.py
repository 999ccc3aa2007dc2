"""GPU parity of paged_attn_decode against the fp64 CPU oracle.

The oracle's pools are filled by the oracle's own store from the same bf16
inputs (never copied from the GPU); the GPU pools are also checked bit-exact
against them.  Attention outputs must satisfy, per element,
    |gpu - oracle| <= 2e-3 + 1e-2 * |oracle|
and, for fp32 outputs, max |gpu - oracle| <= 2e-3.

Also: ragged lengths (not multiples of the block), zero and one-token
sequences, group sizes 1..16, split-K with a reduce, bf16 outputs,
power-of-two scale invariance (bitwise equal outputs), and routing
mutations (swapped pools, swapped scales) that the comparison must catch.
"""
import numpy as np
import pytest
import torch

import fp8_e4m3_scaled_amd as kv
import oracle
from synth import Spec, Workload, bf16_bits
from tests.gpu_util import DEV, GpuCache, bits_dev, log, t_dev

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-3, 1e-2


def assert_close(got, want, what):
    got = np.asarray(got, np.float64)
    err = np.abs(got - want)
    bound = ATOL + RTOL * np.abs(want)
    bad = ~(err <= bound)
    assert not bad.any(), (f"{what}: {int(bad.sum())}/{bad.size} outside |d| <= {ATOL} + {RTOL}|ref|; "
                           f"max |d| {float(np.nanmax(err)):.3g}")


class Filled:
    """A workload stored on the GPU (through kv_store_fp8) and in oracle pools."""

    def __init__(self, w: Workload, upto=None, scales=None, swap_pools=False):
        self.w = w
        ks, vs, _ = w.scales() if scales is None else (*scales, "f32")
        self.ks, self.vs = np.float32(ks), np.float32(vs)
        self.cache = GpuCache(w.NB, w.BS, w.Hkv, w.D, float(ks), float(vs))
        self.ok = np.zeros((w.NB, w.Hkv, w.BS * w.D), np.uint8)
        self.ov = np.zeros_like(self.ok)
        self.lens = np.asarray(w.total_lengths if upto is None else upto, np.int64)
        for b in range(w.B):
            L = int(self.lens[b])
            if L == 0:
                continue
            k, v = w.kv(b, 0, L)
            s = w.slots(b, 0, L)
            kd, vd = k.to(DEV).reshape(L, -1), v.to(DEV).reshape(L, -1)
            kv.kv_store_fp8(self.cache.handle, 0, kd, vd, kd.shape[1], vd.shape[1], t_dev(s), L)
            oracle.store(bf16_bits(k), bf16_bits(v), s, self.ok, self.ov, Hkv=w.Hkv, D=w.D, BS=w.BS,
                         k_scale=self.ks, v_scale=self.vs)
        self.tables = t_dev(w.block_tables.astype(np.int32))

    def check_bytes(self):
        gk, gv = self.cache.pools()
        assert np.array_equal(gk, self.ok) and np.array_equal(gv, self.ov), "cache bytes differ"

    def decode(self, q, lens, out_dtype=kv.DTYPE_F32, handle=None, max_len=None):
        w = self.w
        lens = np.asarray(lens, np.int32)
        max_len = int(lens.max()) if max_len is None else max_len
        h = self.cache.handle if handle is None else handle
        ws_bytes = kv.paged_attn_decode_workspace(h, w.B, w.Hq, max_len)
        ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=DEV)
        dt = torch.float32 if out_dtype == kv.DTYPE_F32 else torch.bfloat16
        out = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=dt, device=DEV)
        kv.paged_attn_decode(h, 0, q, w.Hq, self.tables, w.max_blocks, t_dev(lens), w.B, max_len,
                             w.sm_scale(), out, out_dtype, ws, ws_bytes)
        torch.cuda.synchronize()
        return out.float().cpu().numpy()

    def oracle_decode(self, q_bits, lens, sel=None):
        w = self.w
        return oracle.decode_attn(q_bits, self.ok, self.ov, w.block_tables, np.asarray(lens, np.int32),
                                  Hq=w.Hq, Hkv=w.Hkv, D=w.D, BS=w.BS, k_scale=self.ks,
                                  v_scale=self.vs, sm_scale=w.sm_scale(), sel=sel)

    def close(self):
        self.cache.close()


def _run(w, out_dtype=kv.DTYPE_F32, lens=None):
    f = Filled(w)
    try:
        f.check_bytes()
        lens = f.lens if lens is None else np.asarray(lens)
        q = w.q_decode()
        log(f"decode {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} BS={w.BS} "
            f"max_len={int(lens.max())} out={'f32' if out_dtype == kv.DTYPE_F32 else 'bf16'}")
        got = f.decode(q.to(DEV), lens, out_dtype)
        want = f.oracle_decode(bf16_bits(q), lens)
        assert_close(got, want, f"decode {w.name}")
        if out_dtype == kv.DTYPE_F32:
            assert float(np.max(np.abs(got - want))) <= ATOL
        return got, want
    finally:
        f.close()


@pytest.mark.parametrize("out_dtype", [kv.DTYPE_F32, kv.DTYPE_BF16])
def test_decode_tiny(out_dtype):
    _run(Workload("tiny"), out_dtype)


@pytest.mark.parametrize("name,sd", [("llama8b", 8), ("varlen", 16), ("longctx", 64), ("prefill", 8)])
def test_decode_workloads_reduced(name, sd):
    _run(Workload(name, scale_down=sd, pool_frac=0.0))


@pytest.mark.parametrize("Hq,Hkv,D,BS", [(8, 8, 128, 16), (16, 1, 64, 32), (32, 2, 256, 16),
                                         (12, 4, 128, 32), (6, 2, 64, 16)])
def test_decode_group_sizes_and_ragged_lengths(Hq, Hkv, D, BS):
    lengths = [0, 1, 2, 15, 16, 17, 31, 33, 127, 128, 129, 300, 777]
    spec = Spec("ragged", Hq, Hkv, D, BS, lengths, 4000 + Hq + D + BS, 0.05, 0.02)
    _run(Workload("ragged", spec=spec))


def test_decode_long_split_with_reduce():
    # one sequence-head pair per kv-head and long sequences: many splits + reduce kernel
    spec = Spec("longsplit", 16, 2, 256, 32, [20000, 9000, 131], 4100, 0.03, 0.03)
    w = Workload("longsplit", spec=spec)
    f = Filled(w)
    try:
        assert kv.paged_attn_decode_workspace(f.cache.handle, w.B, w.Hq, 20000) > 0
        q = w.q_decode()
        got = f.decode(q.to(DEV), f.lens)
        sel = np.array([[b, h] for b in range(w.B) for h in (0, 5, 8, 15)], np.int32)
        want = f.oracle_decode(bf16_bits(q), f.lens, sel=sel)
        for b, h in sel:
            assert_close(got[b, h], want[b, h], f"long split b={b} h={h}")
    finally:
        f.close()


def test_decode_max_len_larger_than_lengths():
    """The host bound may exceed every length: the extra splits must be empty, not garbage."""
    w = Workload("tiny")
    f = Filled(w)
    try:
        q = w.q_decode()
        got = f.decode(q.to(DEV), f.lens, max_len=int(w.max_blocks * w.BS))
        assert_close(got, f.oracle_decode(bf16_bits(q), f.lens), "max_len bound")
    finally:
        f.close()


def _small_magnitude_workload(seed):
    spec = Spec("pow2", 8, 2, 128, 16, [100, 37, 64], seed, 1.0, 1.0)
    w = Workload("pow2", spec=spec)
    rng = np.random.default_rng(seed)

    def draw(b, start, count, device=None):
        n = (count, w.Hkv, w.D)
        mag = np.exp2(rng.uniform(np.log2(1.3e-4), np.log2(0.05), size=n))
        x = (mag * np.where(rng.random(n) < 0.5, -1, 1)).astype(np.float32)
        t = torch.from_numpy(x).to(torch.bfloat16)
        return t, t.flip(-1).contiguous()
    w.kv = draw
    return w


def test_decode_power_of_two_scale_invariance():
    """[P3, "Round 4": s*D(Q(x/s)) == s'*D(Q(x/s')) for power-of-two scales when every value
    is normal and unsaturated]: the attention outputs must be bitwise equal."""
    outs, caches = [], []
    for ks, vs in [(2.0 ** -7, 2.0 ** -13), (2.0 ** -11, 2.0 ** -9)]:
        w = _small_magnitude_workload(77)
        f = Filled(w, scales=(ks, vs))
        caches.append(f.cache.pools())
        q = w.q_decode()
        outs.append(f.decode(q.to(DEV), f.lens))
        want = f.oracle_decode(bf16_bits(q), f.lens)
        assert_close(outs[-1], want, "pow2 run")
        codes = np.concatenate([f.ok.ravel(), f.ov.ravel()])
        used = codes[codes != 0]
        e = (used >> 3) & 0xF
        assert np.all((e >= 1) & (e <= 15)) and not np.any((used & 0x7F) >= 0x7E), "precondition"
        f.close()
    assert not np.array_equal(caches[0][0], caches[1][0])          # the bytes differ ...
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))   # ... the outputs do not


def test_decode_routing_mutations_are_caught():
    """Two fp8 runs cannot see routing defects [P3, "Round 4"]: comparing against the oracle
    must.  A handle with the pools swapped, or with the scales swapped, must fail parity."""
    w = Workload("tiny")
    f = Filled(w, scales=(0.02, 0.15))
    try:
        q = w.q_decode()
        want = f.oracle_decode(bf16_bits(q), f.lens)
        c = f.cache
        swapped = kv.kv_cache_alloc(1, c.NB, c.BS, c.Hkv, c.D, [0.02], [0.15], kv.DTYPE_F32,
                                    c.v_pool, c.k_pool)
        scales_swapped = kv.kv_cache_alloc(1, c.NB, c.BS, c.Hkv, c.D, [0.15], [0.02], kv.DTYPE_F32,
                                           c.k_pool, c.v_pool)
        try:
            for h, what in [(swapped, "pools swapped"), (scales_swapped, "scales swapped")]:
                got = f.decode(q.to(DEV), f.lens, handle=h)
                with pytest.raises(AssertionError):
                    assert_close(got, want, what)
        finally:
            kv.kv_cache_free(swapped)
            kv.kv_cache_free(scales_swapped)
        assert_close(f.decode(q.to(DEV), f.lens), want, "unmutated")
    finally:
        f.close()


def test_decode_empty_and_negative_lengths_with_splits():
    """Lengths 0 and below give zero rows, also when the launch is split and the
    reduce combines partials (no split produced anything for those rows)."""
    spec = Spec("emptysplit", 16, 2, 128, 16, [6000, 0, 17, 4100], 4200, 0.03, 0.03)
    w = Workload("emptysplit", spec=spec)
    f = Filled(w)
    try:
        lens = np.array([6000, 0, 17, -3], np.int32)
        assert kv.paged_attn_decode_workspace(f.cache.handle, w.B, w.Hq, 6000) > 0
        q = w.q_decode()
        got = f.decode(q.to(DEV), lens)
        assert np.all(got[1] == 0.0) and np.all(got[3] == 0.0)
        want = f.oracle_decode(bf16_bits(q), np.maximum(lens, 0))
        for b in (0, 2):
            assert_close(got[b], want[b], f"split decode b={b}")
    finally:
        f.close()
