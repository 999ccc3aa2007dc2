"""Checked mode: repeated slots, lengths past their bounds and table entries
outside the pool are reported as KVF8_E_INVALID before anything writes the
cache; valid calls give exactly the unchecked results."""
import numpy as np
import pytest
import torch

import fp8_e4m3_scaled_amd as kv
import oracle
from synth import Spec, Workload, bf16_bits
from tests.gpu_util import DEV, GpuCache, t_dev

pytestmark = pytest.mark.gpu


def _setup():
    w = Workload("checked", spec=Spec("checked", 8, 2, 64, 16, [40, 100, 17], 7700, 0.03, 0.02))
    c = GpuCache(w.NB, w.BS, w.Hkv, w.D, 0.03, 0.02)
    row = w.Hkv * w.D
    L = [int(x) for x in w.total_lengths]
    K = torch.cat([w.kv(b, 0, L[b])[0].reshape(-1, row) for b in range(w.B)]).to(DEV)
    V = torch.cat([w.kv(b, 0, L[b])[1].reshape(-1, row) for b in range(w.B)]).to(DEV)
    slots = np.concatenate([w.slots(b, 0, L[b]) for b in range(w.B)])
    return w, c, row, K, V, slots


def _expect_invalid(fn):
    with pytest.raises(kv.KvF8Error) as ei:
        fn()
    assert ei.value.status == kv.E_INVALID
    return str(ei.value)


def test_checked_store_and_shift_reject_repeated_slots():
    w, c, row, K, V, slots = _setup()
    try:
        kv.kv_cache_set_checked(c.handle, True)
        kv.kv_store_fp8(c.handle, 0, K, V, row, row, t_dev(slots), slots.size)
        before = c.pools()
        ok = np.zeros_like(before[0]), np.zeros_like(before[1])
        oracle.store(bf16_bits(K.cpu()), bf16_bits(V.cpu()), slots, ok[0], ok[1], Hkv=w.Hkv, D=w.D, BS=w.BS,
                     k_scale=0.03, v_scale=0.02)
        assert np.array_equal(before[0], ok[0]) and np.array_equal(before[1], ok[1])
        dup = slots.copy()
        dup[-1] = dup[3]
        K2, V2 = K * 2, V * 2
        msg = _expect_invalid(lambda: kv.kv_store_fp8(c.handle, 0, K2, V2, row, row, t_dev(dup), dup.size))
        assert "more than once" in msg
        after = c.pools()
        assert np.array_equal(after[0], before[0]) and np.array_equal(after[1], before[1])
        # out-of-pool and negative slots are skipped, not errors, even when repeated
        skip = np.array([-1, -1, w.NB * w.BS, w.NB * w.BS], np.int64)
        kv.kv_store_fp8(c.handle, 0, K2[:4], V2[:4], row, row, t_dev(skip), 4)
        _expect_invalid(lambda: kv.kv_shift_rope(c.handle, 0, t_dev(dup), dup.size, -3, 1e4, w.D, kv.ROPE_NEOX))
        table = t_dev(kv.kv_rope_table([-3], 1e4, w.D))
        rows = t_dev(np.zeros(dup.size, np.int32))
        _expect_invalid(lambda: kv.kv_shift_rope_per_slot(c.handle, 0, t_dev(dup), rows, dup.size, table, 1, w.D,
                                                          kv.ROPE_NEOX))
        after = c.pools()
        assert np.array_equal(after[0], before[0]) and np.array_equal(after[1], before[1])
        # checked mode off: the same repeated list is accepted
        kv.kv_cache_set_checked(c.handle, False)
        kv.kv_store_fp8(c.handle, 0, K2, V2, row, row, t_dev(dup), dup.size)
        torch.cuda.synchronize()
    finally:
        c.close()


def test_checked_decode_and_prefill_bounds():
    w, c, row, K, V, slots = _setup()
    try:
        kv.kv_store_fp8(c.handle, 0, K, V, row, row, t_dev(slots), slots.size)
        kv.kv_cache_set_checked(c.handle, True)
        lens = w.total_lengths.astype(np.int32)
        ml = int(lens.max())
        q = w.q_decode(DEV)
        tables = w.block_tables.astype(np.int32).copy()

        def decode(lens_, ml_, tables_, checked=True):
            ws_bytes = kv.paged_attn_decode_workspace(c.handle, w.B, w.Hq, ml_)
            ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=DEV)
            out = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device=DEV)
            kv.paged_attn_decode(c.handle, 0, q, w.Hq, t_dev(tables_), w.max_blocks, t_dev(lens_), w.B, ml_,
                                 w.sm_scale(), out, kv.DTYPE_F32, ws, ws_bytes)
            torch.cuda.synchronize()
            return out.cpu().numpy()

        good = decode(lens, ml, tables)
        kv.kv_cache_set_checked(c.handle, False)
        assert np.array_equal(good, decode(lens, ml, tables))
        kv.kv_cache_set_checked(c.handle, True)
        _expect_invalid(lambda: decode(lens, ml - 1, tables))                  # a length above max_seq_len
        bad = tables.copy()
        bad[1, (int(lens[1]) - 1) // w.BS] = w.NB                              # the last block in use
        assert "outside the pool" in _expect_invalid(lambda: decode(lens, ml, bad))
        unused = tables.copy()
        if unused.shape[1] > (int(lens[2]) + w.BS - 1) // w.BS:
            unused[2, -1] = -5                                                 # not in use: accepted
            assert np.array_equal(decode(lens, ml, unused), good)

        n = 8
        cu = np.array([0, n, 2 * n, 3 * n], np.int32)
        ctx = (lens - n).astype(np.int32)
        qc = torch.randn((3 * n, w.Hq, w.D), generator=torch.Generator().manual_seed(1)).to(torch.bfloat16).to(DEV)

        def prefill(cu_, ctx_, total_q, max_q, max_ctx, tables_):
            out = torch.full((3 * n, w.Hq, w.D), float("nan"), dtype=torch.float32, device=DEV)
            kv.paged_attn_prefill_chunk(c.handle, 0, qc, w.Hq, t_dev(cu_), t_dev(ctx_), t_dev(tables_), w.max_blocks,
                                        w.B, total_q, max_q, max_ctx, w.sm_scale(), out, kv.DTYPE_F32)
            torch.cuda.synchronize()
            return out.cpu().numpy()

        pgood = prefill(cu, ctx, 3 * n, n, int(ctx.max()), tables)
        kv.kv_cache_set_checked(c.handle, False)
        assert np.array_equal(pgood, prefill(cu, ctx, 3 * n, n, int(ctx.max()), tables))
        kv.kv_cache_set_checked(c.handle, True)
        _expect_invalid(lambda: prefill(cu, ctx, 3 * n, n, int(ctx.max()) - 1, tables))   # context above its bound
        _expect_invalid(lambda: prefill(cu, ctx, 3 * n, n - 1, int(ctx.max()), tables))   # chunk above max_q_len
        _expect_invalid(lambda: prefill(cu, ctx, 3 * n - 1, n, int(ctx.max()), tables))   # offsets vs total_q
        _expect_invalid(lambda: prefill(cu, ctx, 3 * n, n, int(ctx.max()), bad))           # table entry
    finally:
        c.close()
