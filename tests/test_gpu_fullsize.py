"""Parity at the full workload sizes, in the launch configuration bench.py times.

Every workload is stored and computed on the GPU exactly as the benchmark does
it (the same store calls, one decode / prefill launch over the whole batch,
the same split plan, bf16 outputs).  The oracle then checks a seeded sample
it can afford: for each sampled sequence it stores that sequence's own bf16
K/V into compact pools (the sampled sequences only, blocks renumbered), and
  * the GPU bytes of the sequence's blocks must equal the oracle's bit for bit;
  * the sampled attention outputs must satisfy |gpu - oracle| <= 2e-3 + 1e-2|oracle|.
Inputs come from the seeded generators on the GPU and are handed to both
sides as the same bf16 bits; no expected value comes from the HIP library.
"""
import numpy as np
import pytest
import torch

import fp8_e4m3_scaled_amd as kv
import oracle
from synth import Workload, bf16_bits
from tests.gpu_util import DEV, log, t_dev
from tests.test_gpu_decode import assert_close

pytestmark = pytest.mark.gpu

FILL_STEP = 65536


class FullCache:
    """A full-size one-layer cache over torch-owned zeroed pools."""

    def __init__(self, w: Workload):
        self.w = w
        ks, vs, _ = w.scales()
        self.ks, self.vs = np.float32(ks), np.float32(vs)
        self.k_pool = torch.zeros((w.NB, w.Hkv, w.BS * w.D), dtype=torch.uint8, device=DEV)
        self.v_pool = torch.zeros_like(self.k_pool)
        self.handle = kv.kv_cache_alloc(1, w.NB, w.BS, w.Hkv, w.D, [float(ks)], [float(vs)],
                                        kv.DTYPE_F32, self.k_pool, self.v_pool)

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

    def blocks(self, b, L):
        """GPU bytes of the blocks that hold tokens 0..L-1 of sequence b."""
        idx = torch.from_numpy(self.w.block_tables[b, :-(-L // self.w.BS)].astype(np.int64)).to(DEV)
        torch.cuda.synchronize()
        return self.k_pool[idx].cpu().numpy(), self.v_pool[idx].cpu().numpy()

    def close(self):
        if self.handle:
            kv.kv_cache_free(self.handle)
            self.handle = None


class OracleSample:
    """Oracle pools holding only the sampled sequences, blocks renumbered."""

    def __init__(self, w: Workload, seqs, lens, ks, vs):
        self.w, self.seqs = w, list(seqs)
        self.lens = np.array([int(lens[b]) for b in self.seqs], np.int64)
        nblk = [-(-int(L) // w.BS) for L in self.lens]
        self.table = np.zeros((len(self.seqs), max(nblk)), np.int32)
        off = 0
        for i, n in enumerate(nblk):
            self.table[i, :n] = np.arange(off, off + n)
            off += n
        self.nblk = nblk
        self.kp = np.zeros((off, w.Hkv, w.BS * w.D), np.uint8)
        self.vp = np.zeros_like(self.kp)
        self.ks, self.vs = ks, vs
        for i, b in enumerate(self.seqs):
            self.store(i, 0, int(self.lens[i]))

    def slots(self, i, lo, n):
        p = np.arange(lo, lo + n, dtype=np.int64)
        return self.table[i, p // self.w.BS].astype(np.int64) * self.w.BS + p % self.w.BS

    def store(self, i, lo, count):
        w, b = self.w, self.seqs[i]
        for s in range(lo, lo + count, FILL_STEP):
            n = min(FILL_STEP, lo + count - s)
            k, v = w.kv(b, s, n, device=DEV)
            oracle.store(bf16_bits(k), bf16_bits(v), self.slots(i, s, n), self.kp, self.vp,
                         Hkv=w.Hkv, D=w.D, BS=w.BS, k_scale=self.ks, v_scale=self.vs)

    def check_bytes(self, cache: FullCache):
        for i, b in enumerate(self.seqs):
            gk, gv = cache.blocks(b, int(self.lens[i]))
            rows = self.table[i, :self.nblk[i]]
            assert np.array_equal(gk, self.kp[rows]), f"K bytes of sequence {b} differ"
            assert np.array_equal(gv, self.vp[rows]), f"V bytes of sequence {b} differ"

    def decode(self, q_bits, heads):
        """Oracle decode of the sampled sequences; returns [len(seqs)][Hq][D] (NaN off `heads`)."""
        w = self.w
        sel = np.array([[i, h] for i in range(len(self.seqs)) for h in heads], np.int32)
        return oracle.decode_attn(q_bits[self.seqs], self.kp, self.vp, self.table,
                                  self.lens.astype(np.int32), Hq=w.Hq, Hkv=w.Hkv, D=w.D, BS=w.BS,
                                  k_scale=self.ks, v_scale=self.vs, sm_scale=w.sm_scale(), sel=sel)


def _decode_full(w, cache, q, lens):
    """One decode launch over the whole batch, bf16 out, as the benchmark runs it."""
    max_len = int(lens.max())
    ws_bytes = kv.paged_attn_decode_workspace(cache.handle, w.B, w.Hq, max_len)
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=DEV)
    out = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.bfloat16, device=DEV)
    kv.paged_attn_decode(cache.handle, 0, q, w.Hq, t_dev(w.block_tables.astype(np.int32)), w.max_blocks,
                         t_dev(lens.astype(np.int32)), w.B, max_len, w.sm_scale(), out, kv.DTYPE_BF16,
                         ws, ws_bytes)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), ws_bytes


def _check_decode(w, sample, got, q, heads, what):
    want = sample.decode(bf16_bits(q), heads)
    for i, b in enumerate(sample.seqs):
        assert_close(got[b][heads], want[i][heads], f"{what} sequence {b}")
    assert np.isfinite(got).all(), f"{what}: non-finite outputs"


def test_llama8b_full_size():
    """64 x 4096 tokens, 32 q / 8 kv heads, D 128, block 16: one store launch
    over all 262,144 tokens, one decode launch; 4 sampled sequences, all heads."""
    w = Workload("llama8b", device=DEV)
    cache = FullCache(w)
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
        log(f"llama8b full: one store of {T} tokens, one decode of {w.B} sequences")
        kv.kv_store_fp8(cache.handle, 0, K, V, row, row, t_dev(slots), T)
        del K, V
        q = w.q_decode(DEV)
        got, ws_bytes = _decode_full(w, cache, q, w.total_lengths)
        assert ws_bytes == 0                       # the benchmark's plan: one chunk per sequence
        seqs = np.random.default_rng(11).choice(w.B, 4, replace=False)
        sample = OracleSample(w, seqs, w.total_lengths, cache.ks, cache.vs)
        sample.check_bytes(cache)
        _check_decode(w, sample, got, q, list(range(w.Hq)), "llama8b decode")
    finally:
        cache.close()


def test_varlen_full_size():
    """256 sequences with lengths in [512, 32768] (+1 new token), bf16 scales,
    8 splits + reduce; the shortest, the longest and 3 seeded sequences."""
    w = Workload("varlen", device=DEV, pool_frac=0.0)    # compact pool; same launch shapes
    cache = FullCache(w)
    try:
        log(f"varlen full: fill {int(w.lengths.sum())} tokens, store 1 token x {w.B}, decode")
        cache.fill(w.lengths)
        row = w.Hkv * w.D
        L = w.lengths
        K = torch.cat([w.kv(b, int(L[b]), 1, device=DEV)[0].reshape(1, row) for b in range(w.B)])
        V = torch.cat([w.kv(b, int(L[b]), 1, device=DEV)[1].reshape(1, row) for b in range(w.B)])
        sd = t_dev(np.concatenate([w.slots(b, int(L[b]), 1) for b in range(w.B)]))
        kv.kv_store_fp8(cache.handle, 0, K, V, row, row, sd, w.B)
        q = w.q_decode(DEV)
        got, ws_bytes = _decode_full(w, cache, q, w.total_lengths)
        assert ws_bytes > 0                        # split-K with the reduce, as benchmarked
        rng = np.random.default_rng(12)
        seqs = sorted({int(np.argmin(w.total_lengths)), int(np.argmax(w.total_lengths)),
                       *rng.choice(w.B, 3, replace=False).tolist()})
        sample = OracleSample(w, seqs, w.total_lengths, cache.ks, cache.vs)
        sample.check_bytes(cache)
        heads = sorted(rng.choice(w.Hq, 8, replace=False).tolist())
        _check_decode(w, sample, got, q, heads, "varlen decode")
    finally:
        cache.close()


def test_longctx_full_size_with_shift():
    """8 x 131072 tokens, 16 q / 2 kv heads, D 256, block 32, 32 splits: decode,
    K-shift of every cached token by -4096 (theta 1e6, NEOX), decode again;
    one sampled sequence through the oracle's own chain."""
    w = Workload("longctx", device=DEV)
    cache = FullCache(w)
    try:
        log("longctx full: fill 8 x 131072 tokens, decode, shift, decode")
        cache.fill(w.lengths)
        lens = w.lengths
        q = w.q_decode(DEV)
        got1, ws_bytes = _decode_full(w, cache, q, lens)
        assert ws_bytes > 0
        slots = np.concatenate([w.slots(b, 0, int(lens[b])) for b in range(w.B)])
        kv.kv_shift_rope(cache.handle, 0, t_dev(slots), slots.size, w.spec.delta, w.spec.theta, w.D,
                         kv.ROPE_NEOX)
        got2, _ = _decode_full(w, cache, q, lens)
        seqs = [int(np.random.default_rng(13).integers(w.B))]
        sample = OracleSample(w, seqs, lens, cache.ks, cache.vs)
        heads = list(range(w.Hq))
        _check_decode(w, sample, got1, q, heads, "longctx decode before shift")
        osl = np.concatenate([sample.slots(i, 0, int(sample.lens[i])) for i in range(len(seqs))])
        oracle.kshift(sample.kp, osl, Hkv=w.Hkv, D=w.D, BS=w.BS, delta=w.spec.delta,
                      theta=w.spec.theta, rot_dim=w.D, neox=True)
        sample.check_bytes(cache)
        _check_decode(w, sample, got2, q, heads, "longctx decode after shift")
    finally:
        cache.close()


def test_prefill_full_size():
    """4 sequences x (16384 cached + 2048-token chunk), 32 q / 8 kv heads: the
    chunk's store launch then one prefill launch; 48 sampled (query, head) rows
    that include each chunk's first and last token."""
    w = Workload("prefill", device=DEV)
    cache = FullCache(w)
    try:
        log("prefill full: fill 4 x 16384 tokens, store 4 x 2048, prefill")
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
        out = torch.full((T, w.Hq, w.D), float("nan"), dtype=torch.bfloat16, device=DEV)
        kv.paged_attn_prefill_chunk(cache.handle, 0, q, w.Hq, t_dev(cu), t_dev(ctx),
                                    t_dev(w.block_tables.astype(np.int32)), w.max_blocks, w.B, T, n,
                                    int(ctx.max()), w.sm_scale(), out, kv.DTYPE_BF16)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        assert np.isfinite(got).all()
        seqs = list(range(w.B))
        sample = OracleSample(w, seqs, w.total_lengths, cache.ks, cache.vs)
        sample.check_bytes(cache)
        rng = np.random.default_rng(14)
        rows = [(b * n, int(rng.integers(w.Hq))) for b in range(w.B)]
        rows += [(b * n + n - 1, int(rng.integers(w.Hq))) for b in range(w.B)]
        rows += [(int(rng.integers(T)), int(rng.integers(w.Hq))) for _ in range(40)]
        sel = np.array(rows, np.int64)
        want = oracle.prefill_attn(bf16_bits(q), sample.kp, sample.vp, cu, ctx, sample.table, Hq=w.Hq,
                                   Hkv=w.Hkv, D=w.D, BS=w.BS, k_scale=cache.ks, v_scale=cache.vs,
                                   sm_scale=w.sm_scale(), sel=sel)
        for qi, h in rows:
            assert_close(got[qi, h], want[qi, h], f"prefill row {qi} head {h}")
    finally:
        cache.close()
