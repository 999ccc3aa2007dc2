"""GPU parity of multi-layer caches: every call addresses its own layer's pools
with that layer's scales.  A three-layer cache (different scales per layer,
E4M3 and bf16 pools) gets different inputs per layer at the same slots; each
layer's bytes are checked against its own oracle pools, each layer is decoded
and prefilled against the oracle, a K-shift of one layer leaves the others
unchanged, and new scales on one layer change only what that layer stores
next."""
import numpy as np
import pytest
import torch

import fp8_e4m3_scaled_amd as kv
import oracle
from synth import Spec, Workload, bf16_bits
from tests.gpu_util import DEV, log, t_dev
from tests.test_gpu_decode import ATOL, assert_close

pytestmark = pytest.mark.gpu

E, B = kv.ELEM_E4M3, kv.ELEM_BF16
NP = {E: np.uint8, B: np.uint16}
EB = {E: 1, B: 2}


class Layered:
    def __init__(self, ke, ve, layers=3):
        self.ke, self.ve, self.L = ke, ve, layers
        self.ctx = np.array([0, 37, 100, 5], np.int32)
        self.chunks = np.array([21, 50, 1, 30], np.int32)
        spec = Spec("layers", 8, 2, 64, 16, list(self.ctx + self.chunks), 6100 + 10 * ke + ve, 1.0, 1.0)
        self.w = w = Workload("layers", spec=spec)
        self.ks = [np.float32(0.02 * (l + 1)) if ke == E else np.float32(1.0) for l in range(layers)]
        self.vs = [np.float32(0.015 * (l + 2)) if ve == E else np.float32(1.0) for l in range(layers)]
        n = w.NB * w.Hkv * w.BS * w.D
        self.k_pool = torch.zeros(layers * n * EB[ke], dtype=torch.uint8, device=DEV)
        self.v_pool = torch.zeros(layers * n * EB[ve], dtype=torch.uint8, device=DEV)
        self.handle = kv.kv_cache_alloc_typed(layers, w.NB, w.BS, w.Hkv, w.D, ke, ve, [float(x) for x in self.ks],
                                              [float(x) for x in self.vs], kv.DTYPE_F32, self.k_pool, self.v_pool)
        shape = (w.NB, w.Hkv, w.BS * w.D)
        self.ok = [np.zeros(shape, NP[ke]) for _ in range(layers)]
        self.ov = [np.zeros(shape, NP[ve]) for _ in range(layers)]
        self.row = w.Hkv * w.D

    def inputs(self, layer, b, lo, n):
        """Layer-specific K/V: the workload's values scaled by (layer + 1) and flipped in sign
        on odd layers (still bf16-exact), so every layer stores different codes."""
        k, v = self.w.kv(b, lo, n)
        f = float(layer + 1) * (-1.0 if layer % 2 else 1.0)
        return (k.float() * f).to(torch.bfloat16), (v.float() * f).to(torch.bfloat16)

    def store(self, layer, b, lo, n):
        k, v = self.inputs(layer, b, lo, n)
        s = self.w.slots(b, lo, n)
        kv.kv_store_fp8(self.handle, layer, k.to(DEV).reshape(n, self.row), v.to(DEV).reshape(n, self.row),
                        self.row, self.row, t_dev(s), n)
        oracle.store(bf16_bits(k), bf16_bits(v), s, self.ok[layer], self.ov[layer], Hkv=self.w.Hkv, D=self.w.D,
                     BS=self.w.BS, k_scale=self.ks[layer], v_scale=self.vs[layer])

    def pools(self, layer):
        torch.cuda.synchronize()
        w = self.w
        n = w.NB * w.Hkv * w.BS * w.D
        gk = self.k_pool.cpu().numpy().view(NP[self.ke]).reshape(self.L, -1)[layer].reshape(self.ok[layer].shape)
        gv = self.v_pool.cpu().numpy().view(NP[self.ve]).reshape(self.L, -1)[layer].reshape(self.ov[layer].shape)
        assert gk.size == n
        return gk, gv

    def check(self, layer):
        gk, gv = self.pools(layer)
        assert np.array_equal(gk, self.ok[layer]), f"layer {layer}: K differs"
        assert np.array_equal(gv, self.ov[layer]), f"layer {layer}: V differs"

    def close(self):
        kv.kv_cache_free(self.handle)


@pytest.mark.parametrize("ke,ve", [(E, E), (B, E), (B, B)])
def test_layers_store_decode_prefill_shift(ke, ve):
    c = Layered(ke, ve)
    w = c.w
    log(f"layers k={ke} v={ve}")
    try:
        total = (c.ctx + c.chunks).astype(np.int32)
        for layer in range(c.L):
            for b in range(w.B):
                c.store(layer, b, 0, int(total[b]))
        for layer in range(c.L):
            c.check(layer)
        tables = t_dev(w.block_tables.astype(np.int32))
        # decode of every layer
        q = w.q_decode()
        for layer in range(c.L):
            out = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device=DEV)
            ws_bytes = kv.paged_attn_decode_workspace(c.handle, w.B, w.Hq, int(total.max()))
            ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=DEV)
            kv.paged_attn_decode(c.handle, layer, q.to(DEV), w.Hq, tables, w.max_blocks, t_dev(total), w.B,
                                 int(total.max()), w.sm_scale(), out, kv.DTYPE_F32, ws, ws_bytes)
            torch.cuda.synchronize()
            want = oracle.decode_attn(bf16_bits(q), c.ok[layer], c.ov[layer], w.block_tables, total, Hq=w.Hq,
                                      Hkv=w.Hkv, D=w.D, BS=w.BS, k_scale=c.ks[layer], v_scale=c.vs[layer],
                                      sm_scale=w.sm_scale())
            got = out.cpu().numpy()
            assert_close(got, want, f"decode layer {layer}")
            assert float(np.max(np.abs(got - want))) <= ATOL
        # prefill of the middle layer
        cu = np.concatenate([[0], np.cumsum(c.chunks)]).astype(np.int32)
        qc = torch.randn((int(cu[-1]), w.Hq, w.D), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
        out = torch.full((int(cu[-1]), w.Hq, w.D), float("nan"), dtype=torch.float32, device=DEV)
        kv.paged_attn_prefill_chunk(c.handle, 1, qc.to(DEV), w.Hq, t_dev(cu), t_dev(c.ctx), tables, w.max_blocks,
                                    w.B, int(cu[-1]), int(c.chunks.max()), int(c.ctx.max()), w.sm_scale(), out,
                                    kv.DTYPE_F32)
        torch.cuda.synchronize()
        want = oracle.prefill_attn(bf16_bits(qc), c.ok[1], c.ov[1], cu, c.ctx, w.block_tables, Hq=w.Hq, Hkv=w.Hkv,
                                   D=w.D, BS=w.BS, k_scale=c.ks[1], v_scale=c.vs[1], sm_scale=w.sm_scale())
        assert_close(out.cpu().numpy(), want, "prefill layer 1")
        # K-shift of layer 2 only
        slots = np.concatenate([w.slots(b, 0, int(total[b])) for b in range(w.B)])
        kv.kv_shift_rope(c.handle, 2, t_dev(slots), slots.size, -5, 1e4, w.D, kv.ROPE_NEOX)
        oracle.kshift(c.ok[2], slots, Hkv=w.Hkv, D=w.D, BS=w.BS, delta=-5, theta=1e4, rot_dim=w.D, neox=True)
        for layer in range(c.L):
            c.check(layer)
        # new scales on layer 0 (E4M3 sides only) change what layer 0 stores next, nothing else
        if ke == E or ve == E:
            nks = np.float32(0.5) if ke == E else None
            nvs = np.float32(0.25) if ve == E else None
            kv.kv_cache_set_scales(c.handle, 0, None if nks is None else float(nks),
                                   None if nvs is None else float(nvs))
            if nks is not None:
                c.ks[0] = nks
            if nvs is not None:
                c.vs[0] = nvs
            c.store(0, 1, 0, int(total[1]))
            for layer in range(c.L):
                c.check(layer)
    finally:
        c.close()
