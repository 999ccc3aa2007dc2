"""The hot path captures into a HIP graph: a store, a (split) decode and a
prefill chunk recorded with torch.cuda.graph replay several times, with eager
work and synchronizations between the replays, and every replay equals the
eager result bit for bit (the kernels are deterministic and the library
records no memset or allocation)."""
import numpy as np
import pytest
import torch

import fp8_e4m3_scaled_amd as kv
from synth import Spec, Workload
from tests.gpu_util import DEV, GpuCache, t_dev

pytestmark = pytest.mark.gpu


def test_graph_replays_equal_eager():
    w = Workload("graph", spec=Spec("graph", 16, 2, 128, 16, [9000, 300, 4097, 16], 7300, 0.03, 0.02))
    row = w.Hkv * w.D
    cache = GpuCache(w.NB, w.BS, w.Hkv, w.D, 0.03, 0.02)
    try:
        T = int(w.total_lengths.sum())
        K = torch.cat([w.kv(b, 0, int(w.total_lengths[b]), device=DEV)[0].reshape(-1, row) for b in range(w.B)])
        V = torch.cat([w.kv(b, 0, int(w.total_lengths[b]), device=DEV)[1].reshape(-1, row) for b in range(w.B)])
        slots = t_dev(np.concatenate([w.slots(b, 0, int(w.total_lengths[b])) for b in range(w.B)]))
        tables = t_dev(w.block_tables.astype(np.int32))
        lens = t_dev(w.total_lengths.astype(np.int32))
        ml = int(w.total_lengths.max())
        q = w.q_decode(DEV)
        ws_bytes = kv.paged_attn_decode_workspace(cache.handle, w.B, w.Hq, ml)
        assert ws_bytes > 0                                   # the split path with its reduce
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
        n = 40
        cu = t_dev(np.arange(w.B + 1, dtype=np.int32) * n)
        ctx = t_dev((w.total_lengths - n).astype(np.int32))
        qc = torch.randn((w.B * n, w.Hq, w.D), generator=torch.Generator(device=DEV).manual_seed(9),
                         device=DEV).to(torch.bfloat16)
        out_d = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=DEV)
        out_p = torch.empty((w.B * n, w.Hq, w.D), dtype=torch.bfloat16, device=DEV)

        def step():
            kv.kv_store_fp8(cache.handle, 0, K, V, row, row, slots, T)
            kv.paged_attn_decode(cache.handle, 0, q, w.Hq, tables, w.max_blocks, lens, w.B, ml, w.sm_scale(),
                                 out_d, kv.DTYPE_F32, ws, ws_bytes)
            kv.paged_attn_prefill_chunk(cache.handle, 0, qc, w.Hq, cu, ctx, tables, w.max_blocks, w.B, w.B * n,
                                        n, ml - n, w.sm_scale(), out_p, kv.DTYPE_BF16)

        step()
        torch.cuda.synchronize()
        want = (cache.k_pool.clone(), cache.v_pool.clone(), out_d.clone(), out_p.clone())

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):               # warm-up off the default stream, as torch advises
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for r in range(4):
            cache.k_pool.zero_()                     # eager work between replays
            cache.v_pool.zero_()
            out_d.fill_(float("nan"))
            out_p.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = (cache.k_pool, cache.v_pool, out_d, out_p)
            for i, (x, y) in enumerate(zip(got, want)):
                assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), (r, i)
        del g
    finally:
        cache.close()
