"""GPU parity of paged_attn_prefill_chunk against the fp64 CPU oracle.

Each sequence stores its context and its chunk (through kv_store_fp8 on the
GPU, through the oracle's store on the CPU); the chunk's queries then attend
causally over the cache.  Covered: contexts of 0 and of ragged lengths,
chunks of 1 token and of lengths that straddle tiles, empty chunks, group
sizes 1..16 (including ones that do not divide the 128-row tile), head dims
64/128/256, blocks 16/32, fp32 and bf16 outputs, and a one-token chunk
against the decode kernel.
"""
import numpy as np
import pytest
import torch

import fp8_e4m3_scaled_amd as kv
import oracle
from synth import Spec, Workload, bf16_bits
from tests.gpu_util import DEV, log, t_dev
from tests.test_gpu_decode import ATOL, Filled, assert_close

pytestmark = pytest.mark.gpu


class Chunked:
    """Sequence b has lengths[b] context tokens and chunks[b] new tokens, all stored."""

    def __init__(self, Hq, Hkv, D, BS, ctx, chunks, seed, ks=0.04, vs=0.03):
        self.ctx = np.asarray(ctx, np.int32)
        self.chunks = np.asarray(chunks, np.int32)
        spec = Spec("chunked", Hq, Hkv, D, BS, list(self.ctx + self.chunks), seed, ks, vs)
        self.w = Workload("chunked", spec=spec)
        self.f = Filled(self.w)
        self.cu = np.concatenate([[0], np.cumsum(self.chunks)]).astype(np.int32)
        g = torch.Generator().manual_seed(seed + 1)
        self.q = torch.randn((int(self.cu[-1]), Hq, D), generator=g).to(torch.bfloat16)

    def run(self, out_dtype=kv.DTYPE_F32):
        w = self.w
        dt = torch.float32 if out_dtype == kv.DTYPE_F32 else torch.bfloat16
        out = torch.full((int(self.cu[-1]), w.Hq, w.D), float("nan"), dtype=dt, device=DEV)
        kv.paged_attn_prefill_chunk(self.f.cache.handle, 0, self.q.to(DEV), w.Hq, t_dev(self.cu),
                                    t_dev(self.ctx), self.f.tables, w.max_blocks, w.B, int(self.cu[-1]),
                                    int(self.chunks.max()), int(self.ctx.max()), w.sm_scale(), out,
                                    out_dtype)
        torch.cuda.synchronize()
        return out.float().cpu().numpy()

    def oracle(self, sel=None):
        w = self.w
        return oracle.prefill_attn(bf16_bits(self.q), self.f.ok, self.f.ov, self.cu, self.ctx,
                                   w.block_tables, Hq=w.Hq, Hkv=w.Hkv, D=w.D, BS=w.BS,
                                   k_scale=self.f.ks, v_scale=self.f.vs, sm_scale=w.sm_scale(), sel=sel)

    def close(self):
        self.f.close()


@pytest.mark.parametrize("Hq,Hkv,D,BS", [(4, 2, 64, 16), (32, 8, 128, 16), (16, 2, 256, 32),
                                         (8, 8, 128, 32), (16, 1, 64, 16), (12, 4, 128, 16)])
@pytest.mark.parametrize("out_dtype", [kv.DTYPE_F32, kv.DTYPE_BF16])
def test_prefill_shapes(Hq, Hkv, D, BS, out_dtype):
    ctx = [0, 37, 100, 5, 64]
    chunks = [21, 50, 1, 0, 160]
    log(f"prefill Hq={Hq} Hkv={Hkv} D={D} BS={BS} out={out_dtype}")
    c = Chunked(Hq, Hkv, D, BS, ctx, chunks, 5000 + Hq + D + BS)
    try:
        c.f.check_bytes()
        got = c.run(out_dtype)
        want = c.oracle()
        assert_close(got, want, "prefill")
        if out_dtype == kv.DTYPE_F32:
            assert float(np.max(np.abs(got - want))) <= ATOL
    finally:
        c.close()


def test_prefill_workload_reduced():
    """The chunked-prefill workload at 1/8 size: 4 sequences, 2048 cached + 256 new tokens,
    32 q / 8 kv heads, head_dim 128, fp32 amax/448 scales of the cached tokens."""
    w = Workload("prefill", scale_down=8)
    f = Filled(w)
    try:
        f.check_bytes()
        ctx = w.lengths.astype(np.int32)
        n = w.spec.new_tokens
        cu = (np.arange(w.B + 1) * n).astype(np.int32)
        q = w.q_chunk()
        out = torch.empty((w.B * n, w.Hq, w.D), dtype=torch.float32, device=DEV)
        log(f"prefill workload reduced: B={w.B} ctx={int(ctx[0])} chunk={n}")
        kv.paged_attn_prefill_chunk(f.cache.handle, 0, q.to(DEV), w.Hq, t_dev(cu), t_dev(ctx), f.tables,
                                    w.max_blocks, w.B, w.B * n, n, int(ctx.max()), w.sm_scale(), out,
                                    kv.DTYPE_F32)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        rng = np.random.default_rng(3)
        rows = np.concatenate([np.arange(0, w.B * n, 37), [w.B * n - 1]])
        sel = np.array([[r, h] for r in rows for h in rng.choice(w.Hq, 6, replace=False)], np.int64)
        want = oracle.prefill_attn(bf16_bits(q), f.ok, f.ov, cu, ctx, w.block_tables, Hq=w.Hq, Hkv=w.Hkv,
                                   D=w.D, BS=w.BS, k_scale=f.ks, v_scale=f.vs, sm_scale=w.sm_scale(), sel=sel)
        for r, h in sel:
            assert_close(got[r, h], want[r, h], f"row {r} head {h}")
    finally:
        f.close()


def test_one_token_chunk_equals_decode():
    c = Chunked(32, 8, 128, 16, [300, 17, 64], [1, 1, 1], 6100)
    try:
        got = c.run()
        w = c.w
        dec = c.f.decode(c.q.reshape(w.B, w.Hq, w.D).to(DEV), c.ctx + 1)
        want = c.oracle()
        assert_close(got, want, "prefill")
        assert_close(dec, want, "decode")
        assert float(np.max(np.abs(got - dec))) <= 2 * ATOL
    finally:
        c.close()
