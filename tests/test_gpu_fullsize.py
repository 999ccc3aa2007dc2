"""Parity at the full workload sizes, in the launch configuration bench.py times.

Every workload is stored and computed on the GPU exactly as the benchmark does
it (the same store calls, one decode / prefill launch over the whole batch,
the same split plan and pool), with bf16 and fp32 outputs.  The oracle stores every sequence's own
bf16 K/V into full-size host pools with the same block tables (inputs come
from the seeded generators on the GPU and reach both sides as the same bf16
bits; no expected value comes from the HIP library), and
  * the whole K and V pools must equal the oracle's bit for bit;
  * attention outputs satisfy |gpu - oracle| <= 2e-3 + 1e-2 |oracle|, and
    fp32 outputs max |gpu - oracle| <= 2e-3:
    every (sequence, head) of the Llama-shaped decode (E4M3 and its bf16
    twin) and of the variable-length decode and
    of both long-context decodes, and 8,192 prefill (query, head) rows that
    include the first and last 32 query tokens of every sequence (all heads).
Oracle calls run on a thread pool over disjoint sequences / groups (the C
oracle keeps no shared state and releases the GIL).
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import fp8_e4m3_scaled_amd as kv
import oracle
from synth import Workload, bf16_bits
from tests.gpu_util import DEV, log, t_dev
from tests.test_gpu_decode import ATOL, assert_close

pytestmark = pytest.mark.gpu

FILL_STEP = 65536


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _pmap(fn, items):
    oracle._load()
    with ThreadPoolExecutor(max_workers=_threads()) as ex:
        return list(ex.map(fn, items))


class FullCache:
    """A full-size one-layer cache over torch-owned zeroed pools."""

    def __init__(self, w: Workload, elems=(kv.ELEM_E4M3, kv.ELEM_E4M3)):
        self.w = w
        ks, vs, _ = w.scales()
        self.keb, self.veb = (1 if elems[0] == kv.ELEM_E4M3 else 2), (1 if elems[1] == kv.ELEM_E4M3 else 2)
        self.ks = np.float32(ks if self.keb == 1 else 1.0)     # a bf16 pool keeps scale 1
        self.vs = np.float32(vs if self.veb == 1 else 1.0)
        self.k_pool = torch.zeros((w.NB, w.Hkv, w.BS * w.D * self.keb), dtype=torch.uint8, device=DEV)
        self.v_pool = torch.zeros((w.NB, w.Hkv, w.BS * w.D * self.veb), dtype=torch.uint8, device=DEV)
        self.handle = kv.kv_cache_alloc_typed(1, w.NB, w.BS, w.Hkv, w.D, elems[0], elems[1], [float(self.ks)],
                                              [float(self.vs)], kv.DTYPE_F32, self.k_pool, self.v_pool)

    def fill(self, upto):
        """Tokens 0..upto[b]-1 of every sequence, in the benchmark's store calls."""
        w, row = self.w, self.w.Hkv * self.w.D
        for b in range(w.B):
            L = int(upto[b])
            for lo in range(0, L, FILL_STEP):
                n = min(FILL_STEP, L - lo)
                k, v = w.kv(b, lo, n, device=DEV)
                kv.kv_store_fp8(self.handle, 0, k.reshape(n, row), v.reshape(n, row), row, row,
                                t_dev(w.slots(b, lo, n)), n)
        torch.cuda.synchronize()

    def pools(self):
        torch.cuda.synchronize()
        views = {1: np.uint8, 2: np.uint16}
        return (self.k_pool.cpu().numpy().view(views[self.keb]), self.v_pool.cpu().numpy().view(views[self.veb]))

    def close(self):
        if self.handle:
            kv.kv_cache_free(self.handle)
            self.handle = None


class OraclePools:
    """Full-size oracle pools: every sequence's tokens [lo, hi) stored by the oracle."""

    def __init__(self, w: Workload, ks, vs, keb=1, veb=1):
        self.w, self.ks, self.vs = w, ks, vs
        types = {1: np.uint8, 2: np.uint16}
        self.kp = np.zeros((w.NB, w.Hkv, w.BS * w.D), types[keb])
        self.vp = np.zeros((w.NB, w.Hkv, w.BS * w.D), types[veb])

    def store(self, ranges):
        """ranges: (b, lo, hi) triples; different sequences write disjoint slots."""
        w = self.w

        def one(r):
            b, lo, hi = r
            for s in range(lo, hi, FILL_STEP):
                n = min(FILL_STEP, hi - s)
                k, v = w.kv(b, s, n, device=DEV)
                oracle.store(bf16_bits(k), bf16_bits(v), w.slots(b, s, n), self.kp, self.vp,
                             Hkv=w.Hkv, D=w.D, BS=w.BS, k_scale=self.ks, v_scale=self.vs)
        _pmap(one, ranges)

    def check_bytes(self, cache: FullCache, what):
        gk, gv = cache.pools()
        nk = int(np.count_nonzero(gk != self.kp))
        nv = int(np.count_nonzero(gv != self.vp))
        assert nk == 0 and nv == 0, f"{what}: {nk} K and {nv} V elements differ from the oracle"

    def decode_all(self, q_bits, lens):
        """Oracle decode of every (sequence, head): [B][Hq][D] fp64."""
        w = self.w
        lens = np.asarray(lens, np.int32)

        def one(b):
            sel = np.array([[b, h] for h in range(w.Hq)], np.int32)
            ref = oracle.decode_attn(q_bits, self.kp, self.vp, w.block_tables, lens, Hq=w.Hq, Hkv=w.Hkv,
                                     D=w.D, BS=w.BS, k_scale=self.ks, v_scale=self.vs,
                                     sm_scale=w.sm_scale(), sel=sel)
            return ref[b]
        return np.stack(_pmap(one, range(w.B)))


def _decode_full(w, cache, q, lens, tables=None):
    """One decode launch over the whole batch, as the benchmark runs it, once
    with bf16 outputs and once with fp32 outputs: {dtype: [B][Hq][D]}."""
    max_len = int(lens.max())
    ws_bytes = kv.paged_attn_decode_workspace(cache.handle, w.B, w.Hq, max_len)
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=DEV)
    tables = t_dev(w.block_tables.astype(np.int32)) if tables is None else tables
    got = {}
    for dt, tdt in ((kv.DTYPE_BF16, torch.bfloat16), (kv.DTYPE_F32, torch.float32)):
        out = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=tdt, device=DEV)
        kv.paged_attn_decode(cache.handle, 0, q, w.Hq, tables, w.max_blocks, t_dev(lens.astype(np.int32)), w.B,
                             max_len, w.sm_scale(), out, dt, ws, ws_bytes)
        torch.cuda.synchronize()
        got[dt] = out.float().cpu().numpy()
    return got, ws_bytes


def assert_both(got, want, what):
    """Both output dtypes within |d| <= 2e-3 + 1e-2 |ref|; fp32 outputs also max |d| <= 2e-3."""
    assert_close(got[kv.DTYPE_BF16], want, what + " (bf16 out)")
    assert_close(got[kv.DTYPE_F32], want, what + " (fp32 out)")
    err = float(np.max(np.abs(got[kv.DTYPE_F32] - want)))
    log(f"{what}: fp32-output max |d| = {err:.3g}")
    assert err <= ATOL, f"{what}: fp32-output max |d| {err:.3g} > {ATOL}"


ELEMS = [(kv.ELEM_E4M3, kv.ELEM_E4M3), (kv.ELEM_BF16, kv.ELEM_BF16), (kv.ELEM_E4M3, kv.ELEM_BF16),
         (kv.ELEM_BF16, kv.ELEM_E4M3)]
ELEM_IDS = ["e4m3", "bf16_twin", "e4m3k_bf16v", "bf16k_e4m3v"]


@pytest.mark.parametrize("elems", ELEMS, ids=ELEM_IDS)
def test_llama8b_full_size(elems):
    """64 x 4096 tokens, 32 q / 8 kv heads, D 128, block 16: one store launch
    over all 262,144 tokens, one decode launch; all bytes, all 2,048 heads.
    Also for the bf16 twin and the two mixed caches the benchmark times beside
    the E4M3 cache."""
    w = Workload("llama8b", device=DEV)
    cache = FullCache(w, elems)
    try:
        row = w.Hkv * w.D
        T = int(w.total_lengths.sum())
        K = torch.empty((T, row), dtype=torch.bfloat16, device=DEV)
        V = torch.empty_like(K)
        slots = np.empty(T, np.int64)
        pos = 0
        for b in range(w.B):
            L = int(w.total_lengths[b])
            k, v = w.kv(b, 0, L, device=DEV)
            K[pos:pos + L], V[pos:pos + L] = k.reshape(L, row), v.reshape(L, row)
            slots[pos:pos + L] = w.slots(b, 0, L)
            pos += L
        log(f"llama8b full ({elems}): one store of {T} tokens, one decode of {w.B} sequences")
        kv.kv_store_fp8(cache.handle, 0, K, V, row, row, t_dev(slots), T)
        del K, V
        q = w.q_decode(DEV)
        got, ws_bytes = _decode_full(w, cache, q, w.total_lengths)
        assert ws_bytes == 0                       # the benchmark's plan: one chunk per sequence
        orc = OraclePools(w, cache.ks, cache.vs, cache.keb, cache.veb)
        orc.store([(b, 0, int(w.total_lengths[b])) for b in range(w.B)])
        orc.check_bytes(cache, "llama8b")
        want = orc.decode_all(bf16_bits(q), w.total_lengths)
        assert_both(got, want, "llama8b decode, every head")
    finally:
        cache.close()


class _Handle:
    def __init__(self, h):
        self.handle = h


def test_varlen_full_size():
    """256 sequences with lengths in [512, 32768] (+1 new token) over the
    benchmark's own pool, 50 % of 288 GB (4.39 M blocks): block tables drawn by
    the library's allocator (kv_block_shuffle, then kv_block_alloc per
    sequence), scales given as bf16 bit patterns (KVF8_DTYPE_BF16), 8 splits +
    reduce.  Every byte of every block in use and all 8,192 heads against the
    oracle, which holds those blocks under compact ids (the same bytes, 8.7 GB
    instead of the pool's 144 GB)."""
    from synth import f32_to_bf16_bits
    w = Workload("varlen", device=DEV)
    ks, vs, sdt = w.scales()
    assert sdt == "bf16" and w.NB > 4_000_000
    k_pool = torch.zeros((w.NB, w.Hkv, w.BS * w.D), dtype=torch.uint8, device=DEV)
    v_pool = torch.zeros_like(k_pool)
    h = kv.kv_cache_alloc(1, w.NB, w.BS, w.Hkv, w.D, [f32_to_bf16_bits(float(ks))], [f32_to_bf16_bits(float(vs))],
                          kv.DTYPE_BF16, k_pool, v_pool)
    try:
        assert kv.kv_cache_get_scales(h, 0) == (float(ks), float(vs))     # the bf16 bits, widened exactly
        kv.kv_block_shuffle(h, 1003)
        nblk = [-(-int(L) // w.BS) for L in w.total_lengths]
        tables = np.zeros((w.B, w.max_blocks), np.int32)
        for b in range(w.B):
            tables[b, :nblk[b]] = kv.kv_block_alloc(h, nblk[b])
        assert kv.kv_blocks_free(h) == w.NB - sum(nblk)
        assert tables.max() > w.NB // 2                          # scattered over the whole pool
        w.block_tables = tables
        row = w.Hkv * w.D
        log(f"varlen full on the {w.NB}-block pool: fill {int(w.lengths.sum())} tokens, store 1 x {w.B}, decode")
        for b in range(w.B):
            L = int(w.lengths[b])
            for lo in range(0, L, FILL_STEP):
                n = min(FILL_STEP, L - lo)
                k, v = w.kv(b, lo, n, device=DEV)
                kv.kv_store_fp8(h, 0, k.reshape(n, row), v.reshape(n, row), row, row, t_dev(w.slots(b, lo, n)), n)
        L = w.lengths
        K = torch.cat([w.kv(b, int(L[b]), 1, device=DEV)[0].reshape(1, row) for b in range(w.B)])
        V = torch.cat([w.kv(b, int(L[b]), 1, device=DEV)[1].reshape(1, row) for b in range(w.B)])
        sd = t_dev(np.concatenate([w.slots(b, int(L[b]), 1) for b in range(w.B)]))
        kv.kv_store_fp8(h, 0, K, V, row, row, sd, w.B)
        q = w.q_decode(DEV)
        got, ws_bytes = _decode_full(w, _Handle(h), q, w.total_lengths, t_dev(tables))
        assert ws_bytes > 0                        # split-K with the reduce, as benchmarked

        # the oracle's pools: the blocks in use, renumbered 0.. in table order
        ctables = np.zeros_like(tables)
        used = []
        pos = 0
        for b in range(w.B):
            ctables[b, :nblk[b]] = np.arange(pos, pos + nblk[b])
            used.append(tables[b, :nblk[b]])
            pos += nblk[b]
        used = np.concatenate(used)
        okp = np.zeros((pos, w.Hkv, w.BS * w.D), np.uint8)
        ovp = np.zeros_like(okp)

        def store(b):
            Lb = int(w.total_lengths[b])
            for lo in range(0, Lb, FILL_STEP):
                n = min(FILL_STEP, Lb - lo)
                k, v = w.kv(b, lo, n, device=DEV)
                p_ = np.arange(lo, lo + n, dtype=np.int64)
                slots = ctables[b, p_ // w.BS].astype(np.int64) * w.BS + p_ % w.BS
                oracle.store(bf16_bits(k), bf16_bits(v), slots, okp, ovp, Hkv=w.Hkv, D=w.D, BS=w.BS,
                             k_scale=np.float32(ks), v_scale=np.float32(vs))
        _pmap(store, range(w.B))
        bad_k = bad_v = 0
        for lo in range(0, pos, 32768):
            idx = torch.from_numpy(used[lo:lo + 32768].astype(np.int64)).to(DEV)
            gk = k_pool.index_select(0, idx).cpu().numpy()
            gv = v_pool.index_select(0, idx).cpu().numpy()
            bad_k += int(np.count_nonzero(gk != okp[lo:lo + 32768]))
            bad_v += int(np.count_nonzero(gv != ovp[lo:lo + 32768]))
        assert bad_k == 0 and bad_v == 0, f"varlen: {bad_k} K and {bad_v} V bytes differ from the oracle"
        lens = w.total_lengths.astype(np.int32)
        qb = bf16_bits(q)

        def one(b):
            sel = np.array([[b, hh] for hh in range(w.Hq)], np.int32)
            ref = oracle.decode_attn(qb, okp, ovp, ctables, lens, Hq=w.Hq, Hkv=w.Hkv, D=w.D, BS=w.BS,
                                     k_scale=np.float32(ks), v_scale=np.float32(vs), sm_scale=w.sm_scale(), sel=sel)
            return ref[b]
        want = np.stack(_pmap(one, range(w.B)))
        assert_both(got, want, "varlen decode, every head")
    finally:
        kv.kv_cache_free(h)
        del k_pool, v_pool
        torch.cuda.empty_cache()


def test_longctx_full_size_with_shift():
    """8 x 131072 tokens, 16 q / 2 kv heads, D 256, block 32, 32 splits: decode,
    K-shift of every cached token by -4096 (theta 1e6, NEOX), decode again; all
    bytes after the shift and every head of both decodes against the oracle's
    own chain."""
    w = Workload("longctx", device=DEV)
    cache = FullCache(w)
    try:
        log("longctx full: fill 8 x 131072 tokens, decode, shift, decode")
        cache.fill(w.lengths)
        lens = w.lengths
        q = w.q_decode(DEV)
        qb = bf16_bits(q)
        got1, ws_bytes = _decode_full(w, cache, q, lens)
        assert ws_bytes > 0
        slots = np.concatenate([w.slots(b, 0, int(lens[b])) for b in range(w.B)])
        kv.kv_shift_rope(cache.handle, 0, t_dev(slots), slots.size, w.spec.delta, w.spec.theta, w.D,
                         kv.ROPE_NEOX)
        got2, _ = _decode_full(w, cache, q, lens)
        orc = OraclePools(w, cache.ks, cache.vs)
        orc.store([(b, 0, int(lens[b])) for b in range(w.B)])
        assert_both(got1, orc.decode_all(qb, lens), "longctx decode before shift, every head")
        # the oracle's own shift, per sequence (disjoint slots)
        _pmap(lambda b: oracle.kshift(orc.kp, w.slots(b, 0, int(lens[b])), Hkv=w.Hkv, D=w.D, BS=w.BS,
                                      delta=w.spec.delta, theta=w.spec.theta, rot_dim=w.D, neox=True),
              range(w.B))
        orc.check_bytes(cache, "longctx after shift")
        assert_both(got2, orc.decode_all(qb, lens), "longctx decode after shift, every head")
    finally:
        cache.close()


@pytest.mark.parametrize("elems", ELEMS, ids=ELEM_IDS)
def test_prefill_full_size(elems):
    """4 sequences x (16384 cached + 2048-token chunk), 32 q / 8 kv heads: the
    chunk's store launch then one prefill launch; all bytes, and 8,192 (query,
    head) rows: the first and last 32 tokens of every chunk with all heads,
    plus seeded rows in between.  For the E4M3 cache and for the bf16 twin and
    mixed caches the benchmark times beside it."""
    w = Workload("prefill", device=DEV)
    cache = FullCache(w, elems)
    try:
        log(f"prefill full ({elems}): fill 4 x 16384 tokens, store 4 x 2048, prefill")
        cache.fill(w.lengths)
        n = w.spec.new_tokens
        row = w.Hkv * w.D
        ctx = w.lengths.astype(np.int32)
        K = torch.cat([w.kv(b, int(ctx[b]), n, device=DEV)[0].reshape(n, row) for b in range(w.B)])
        V = torch.cat([w.kv(b, int(ctx[b]), n, device=DEV)[1].reshape(n, row) for b in range(w.B)])
        sd = t_dev(np.concatenate([w.slots(b, int(ctx[b]), n) for b in range(w.B)]))
        T = w.B * n
        kv.kv_store_fp8(cache.handle, 0, K, V, row, row, sd, T)
        q = w.q_chunk(DEV)
        cu = (np.arange(w.B + 1) * n).astype(np.int32)
        got = {}
        for dt, tdt in ((kv.DTYPE_BF16, torch.bfloat16), (kv.DTYPE_F32, torch.float32)):
            out = torch.full((T, w.Hq, w.D), float("nan"), dtype=tdt, device=DEV)
            kv.paged_attn_prefill_chunk(cache.handle, 0, q, w.Hq, t_dev(cu), t_dev(ctx),
                                        t_dev(w.block_tables.astype(np.int32)), w.max_blocks, w.B, T, n,
                                        int(ctx.max()), w.sm_scale(), out, dt)
            torch.cuda.synchronize()
            got[dt] = out.float().cpu().numpy()
            assert np.isfinite(got[dt]).all()
            del out
        orc = OraclePools(w, cache.ks, cache.vs, cache.keb, cache.veb)
        orc.store([(b, 0, int(w.total_lengths[b])) for b in range(w.B)])
        orc.check_bytes(cache, "prefill")
        rng = np.random.default_rng(14)
        rows = set()
        for b in range(w.B):
            for i in list(range(32)) + list(range(n - 32, n)):
                rows.update((b * n + i, h) for h in range(w.Hq))
        while len(rows) < 8192:
            rows.add((int(rng.integers(T)), int(rng.integers(w.Hq))))
        G = w.Hq // w.Hkv
        groups = {}
        for qi, h in sorted(rows):
            groups.setdefault((qi // n, h // G), []).append((qi, h))
        qb = bf16_bits(q)

        def one(key):
            sel = np.array(sorted(groups[key]), np.int64)
            ref = oracle.prefill_attn(qb, orc.kp, orc.vp, cu, ctx, w.block_tables, Hq=w.Hq, Hkv=w.Hkv,
                                      D=w.D, BS=w.BS, k_scale=cache.ks, v_scale=cache.vs,
                                      sm_scale=w.sm_scale(), sel=sel)
            return sel, ref[sel[:, 0], sel[:, 1]]
        err = 0.0
        for sel, ref in _pmap(one, sorted(groups)):
            what = f"prefill rows of group ({sel[0, 0] // n}, ...)"
            assert_close(got[kv.DTYPE_BF16][sel[:, 0], sel[:, 1]], ref, what + " (bf16 out)")
            gf = got[kv.DTYPE_F32][sel[:, 0], sel[:, 1]]
            assert_close(gf, ref, what + " (fp32 out)")
            err = max(err, float(np.max(np.abs(gf - ref))))
        log(f"prefill sampled rows: fp32-output max |d| = {err:.3g}")
        assert err <= ATOL, f"prefill: fp32-output max |d| {err:.3g} > {ATOL}"
        assert len(rows) >= 4096
    finally:
        cache.close()
