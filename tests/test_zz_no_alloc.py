"""paged_attn_decode_noalloc: the decode without a workspace argument, for
callers that cannot allocate (its split-K partials live in a fixed device
array of the library).  Through the C ABI it must give the same outputs as
paged_attn_decode with a caller workspace (bit for bit: the same kernels and
partial layout) and stay within the attention tolerance of the fp64 oracle,
on two calls in a row, the second with a smaller input; shapes whose
workspace exceeds the array are rejected before anything is launched."""
import numpy as np
import pytest
import torch

import fp8_e4m3_scaled_amd as kv
from synth import Spec, Workload, bf16_bits
from tests.gpu_util import DEV, log, t_dev
from tests.test_gpu_decode import ATOL, Filled, assert_close

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 64 << 20


def _both(f: Filled, q, lens, out_dtype):
    w = f.w
    lens = np.asarray(lens, np.int32)
    max_len = int(lens.max())
    ws_bytes = kv.paged_attn_decode_workspace(f.cache.handle, w.B, w.Hq, max_len)
    assert 0 < ws_bytes <= SCRATCH_BYTES            # split-K: the scratch array is in use
    dt = torch.float32 if out_dtype == kv.DTYPE_F32 else torch.bfloat16
    tables, dlens = f.tables, t_dev(lens)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    ref = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=dt, device=DEV)
    kv.paged_attn_decode(f.cache.handle, 0, q, w.Hq, tables, w.max_blocks, dlens, w.B, max_len, w.sm_scale(),
                         ref, out_dtype, ws, ws_bytes)
    got = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=dt, device=DEV)
    kv.paged_attn_decode_noalloc(f.cache.handle, 0, q, w.Hq, tables, w.max_blocks, dlens, w.B, max_len,
                                 w.sm_scale(), got, out_dtype)
    torch.cuda.synchronize()
    return got.float().cpu().numpy(), ref.float().cpu().numpy()


def test_noalloc_decode_equals_workspace_decode_twice():
    cases = [
        # a larger call first, then a smaller one (fewer sequences, shorter
        # lengths, smaller heads) that reuses the same device array
        (Spec("noalloc_big", 32, 8, 128, 16, [9000, 4100, 17, 12288, 6000, 333, 8191, 2], 9100), kv.DTYPE_F32),
        (Spec("noalloc_small", 8, 2, 64, 32, [700, 129, 1500], 9200, 0.05, 0.02), kv.DTYPE_BF16),
    ]
    for spec, out_dtype in cases:
        w = Workload(spec.name, spec=spec)
        f = Filled(w)
        try:
            q = w.q_decode().to(DEV)
            log(f"noalloc decode {spec.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} BS={w.BS} "
                f"max_len={int(f.lens.max())}")
            got, ref = _both(f, q, f.lens, out_dtype)
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), "differs from paged_attn_decode"
            want = f.oracle_decode(bf16_bits(q.cpu()), f.lens)
            assert_close(got, want, f"noalloc decode {spec.name}")
            if out_dtype == kv.DTYPE_F32:
                assert float(np.max(np.abs(got - want))) <= ATOL
        finally:
            f.close()


def test_noalloc_decode_rejects_a_workspace_beyond_its_array():
    w = Workload("noalloc_tiny", spec=Spec("noalloc_tiny", 32, 8, 128, 16, [40, 17], 9300, 0.05, 0.02))
    f = Filled(w)
    try:
        B, max_len = 1024, 65536
        need = kv.paged_attn_decode_workspace(f.cache.handle, B, w.Hq, max_len)
        assert need > SCRATCH_BYTES
        out = torch.zeros((2, w.Hq, w.D), dtype=torch.float32, device=DEV)
        sentinel = out.clone()
        with pytest.raises(kv.KvF8Error) as ei:
            kv.paged_attn_decode_noalloc(f.cache.handle, 0, torch.zeros((2, w.Hq, w.D), dtype=torch.bfloat16,
                                                                        device=DEV),
                                         w.Hq, f.tables, max_len // w.BS, t_dev(np.array([40, 17], np.int32)), B,
                                         max_len, w.sm_scale(), out, kv.DTYPE_F32)
        assert ei.value.status == 5 and str(need) in str(ei.value)       # KVF8_E_UNSUPPORTED, with the size
        torch.cuda.synchronize()
        assert torch.equal(out, sentinel)               # nothing was launched
    finally:
        f.close()
