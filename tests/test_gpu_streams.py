"""The library launches on the stream it is given: a store, decode, prefill,
K-shift and calibration issued on a side stream (torch.cuda.Stream, default
priority) and synchronized only through that stream give the same bytes and
outputs as the same calls on torch's current stream."""
import numpy as np
import pytest
import torch

import fp8_e4m3_scaled_amd as kv
from synth import Spec, Workload
from tests.gpu_util import DEV, GpuCache, t_dev

pytestmark = pytest.mark.gpu


def _pipeline(w, stream):
    """Store everything, decode, prefill a chunk, shift, decode again, calibrate; all on `stream`."""
    row = w.Hkv * w.D
    with torch.cuda.stream(stream):
        cache = GpuCache(w.NB, w.BS, w.Hkv, w.D, 0.03, 0.02)
        T = int(w.total_lengths.sum())
        K = torch.cat([w.kv(b, 0, int(w.total_lengths[b]), device=DEV)[0].reshape(-1, row) for b in range(w.B)])
        V = torch.cat([w.kv(b, 0, int(w.total_lengths[b]), device=DEV)[1].reshape(-1, row) for b in range(w.B)])
        slots = t_dev(np.concatenate([w.slots(b, 0, int(w.total_lengths[b])) for b in range(w.B)]))
        tables = t_dev(w.block_tables.astype(np.int32))
        lens = t_dev(w.total_lengths.astype(np.int32))
        q = w.q_decode(DEV)
        out1 = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=DEV)
        out2 = torch.empty_like(out1)
        amax = torch.zeros(2, dtype=torch.float32, device=DEV)
        scales = torch.zeros(2, dtype=torch.int32, device=DEV)
        kv.kv_calibrate_scales(K, V, row, row, T, row, amax, scales, kv.DTYPE_F32, stream)
        kv.kv_store_fp8(cache.handle, 0, K, V, row, row, slots, T, stream)
        ml = int(w.total_lengths.max())
        ws_bytes = kv.paged_attn_decode_workspace(cache.handle, w.B, w.Hq, ml)
        ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=DEV)
        kv.paged_attn_decode(cache.handle, 0, q, w.Hq, tables, w.max_blocks, lens, w.B, ml, w.sm_scale(), out1,
                             kv.DTYPE_F32, ws, ws_bytes, stream)
        n = 16
        cu = t_dev(np.arange(w.B + 1, dtype=np.int32) * n)
        ctx = t_dev((w.total_lengths - n).astype(np.int32))
        qc = torch.randn((w.B * n, w.Hq, w.D), generator=torch.Generator(device=DEV).manual_seed(3),
                         device=DEV).to(torch.bfloat16)
        outp = torch.empty((w.B * n, w.Hq, w.D), dtype=torch.float32, device=DEV)
        kv.paged_attn_prefill_chunk(cache.handle, 0, qc, w.Hq, cu, ctx, tables, w.max_blocks, w.B, w.B * n, n,
                                    int(w.total_lengths.max()) - n, w.sm_scale(), outp, kv.DTYPE_F32, stream)
        kv.kv_shift_rope(cache.handle, 0, slots, T, -9, 1e4, w.D, kv.ROPE_NEOX, stream)
        kv.paged_attn_decode(cache.handle, 0, q, w.Hq, tables, w.max_blocks, lens, w.B, ml, w.sm_scale(), out2,
                             kv.DTYPE_F32, ws, ws_bytes, stream)
        stream.synchronize()
        res = (cache.k_pool.cpu().numpy(), cache.v_pool.cpu().numpy(), out1.cpu().numpy(), outp.cpu().numpy(),
               out2.cpu().numpy(), scales.cpu().numpy())
        cache.close()
    return res


def test_side_stream_equals_current_stream():
    w = Workload("streams", spec=Spec("streams", 16, 4, 128, 16, [3000, 700, 4500, 33], 7100, 0.03, 0.02))
    side = torch.cuda.Stream()
    a = _pipeline(w, side)
    b = _pipeline(w, torch.cuda.current_stream())
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
