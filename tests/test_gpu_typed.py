"""GPU parity of caches whose K and V pools have their own element types
(E4M3 codes or bf16 values as given): every stored element bit-exact against
the oracle for all four type combinations, and the decode within the
attention tolerance, including ragged lengths, group sizes, bf16 outputs and
split-K with the reduce."""
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
COMBOS = [(E, B), (B, E), (B, B), (E, E)]
NP = {E: np.uint8, B: np.uint16}
EB = {E: 1, B: 2}


class TypedCache:
    """A one-layer typed cache over torch-owned zeroed pools, with the oracle's twin."""

    def __init__(self, w: Workload, ke, ve, ks, vs, store_lens=None):
        self.w, self.ke, self.ve = w, ke, ve
        self.ks = np.float32(ks if ke == E else 1.0)
        self.vs = np.float32(vs if ve == E else 1.0)
        n = w.NB * w.Hkv * w.BS * w.D
        self.k_pool = torch.zeros(n * EB[ke], dtype=torch.uint8, device=DEV)
        self.v_pool = torch.zeros(n * EB[ve], dtype=torch.uint8, device=DEV)
        self.handle = kv.kv_cache_alloc_typed(1, w.NB, w.BS, w.Hkv, w.D, ke, ve, [float(self.ks)],
                                              [float(self.vs)], kv.DTYPE_F32, self.k_pool, self.v_pool)
        shape = (w.NB, w.Hkv, w.BS * w.D)
        self.ok = np.zeros(shape, NP[ke])
        self.ov = np.zeros(shape, NP[ve])
        self.lens = np.asarray(w.total_lengths if store_lens is None else store_lens, np.int64)
        row = w.Hkv * w.D
        for b in range(w.B):
            L = int(self.lens[b])
            if L == 0:
                continue
            k, v = w.kv(b, 0, L)
            s = w.slots(b, 0, L)
            kv.kv_store_fp8(self.handle, 0, k.to(DEV).reshape(L, row), v.to(DEV).reshape(L, row), row, row,
                            t_dev(s), L)
            oracle.store(bf16_bits(k), bf16_bits(v), s, self.ok, self.ov, Hkv=w.Hkv, D=w.D, BS=w.BS,
                         k_scale=self.ks, v_scale=self.vs)

    def check_bytes(self):
        torch.cuda.synchronize()
        gk = self.k_pool.cpu().numpy().view(NP[self.ke]).reshape(self.ok.shape)
        gv = self.v_pool.cpu().numpy().view(NP[self.ve]).reshape(self.ov.shape)
        assert np.array_equal(gk, self.ok), f"{int((gk != self.ok).sum())} K elements differ"
        assert np.array_equal(gv, self.ov), f"{int((gv != self.ov).sum())} V elements differ"

    def decode(self, q, lens, out_dtype=kv.DTYPE_F32):
        w = self.w
        lens = np.asarray(lens, np.int32)
        max_len = int(lens.max())
        ws_bytes = kv.paged_attn_decode_workspace(self.handle, w.B, w.Hq, max_len)
        ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=DEV)
        dt = torch.float32 if out_dtype == kv.DTYPE_F32 else torch.bfloat16
        out = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=dt, device=DEV)
        kv.paged_attn_decode(self.handle, 0, q.to(DEV), w.Hq, t_dev(w.block_tables.astype(np.int32)),
                             w.max_blocks, t_dev(lens), w.B, max_len, w.sm_scale(), out, out_dtype, ws,
                             ws_bytes)
        torch.cuda.synchronize()
        return out.float().cpu().numpy(), ws_bytes

    def oracle_decode(self, q, lens, sel=None):
        w = self.w
        return oracle.decode_attn(bf16_bits(q), self.ok, self.ov, w.block_tables, np.asarray(lens, np.int32),
                                  Hq=w.Hq, Hkv=w.Hkv, D=w.D, BS=w.BS, k_scale=self.ks, v_scale=self.vs,
                                  sm_scale=w.sm_scale(), sel=sel)

    def close(self):
        if self.handle:
            kv.kv_cache_free(self.handle)
            self.handle = None


@pytest.mark.parametrize("ke,ve", COMBOS)
@pytest.mark.parametrize("Hq,Hkv,D,BS", [(4, 2, 64, 16), (32, 8, 128, 16), (16, 2, 128, 32), (8, 8, 64, 32)])
def test_typed_store_and_decode(ke, ve, Hq, Hkv, D, BS):
    lengths = [0, 1, 3, 16, 17, 33, 129, 300, 777]
    spec = Spec("typed", Hq, Hkv, D, BS, lengths, 5000 + Hq + D + BS + 10 * ke + ve, 0.05, 0.02, outliers=2)
    w = Workload("typed", spec=spec)
    log(f"typed k={ke} v={ve} Hq={Hq} Hkv={Hkv} D={D} BS={BS}")
    c = TypedCache(w, ke, ve, 0.05, 0.02)
    try:
        c.check_bytes()
        q = w.q_decode()
        want = c.oracle_decode(q, c.lens)
        got, _ = c.decode(q, c.lens)
        assert_close(got, want, f"typed decode k={ke} v={ve}")
        assert float(np.nanmax(np.abs(got - want))) <= ATOL
        gotb, _ = c.decode(q, c.lens, kv.DTYPE_BF16)
        assert_close(gotb, want, f"typed decode bf16 out k={ke} v={ve}")
    finally:
        c.close()


@pytest.mark.parametrize("ke,ve", COMBOS[:3])
def test_typed_decode_split_with_reduce(ke, ve):
    spec = Spec("typedsplit", 16, 2, 128, 16, [9000, 4097, 131], 5100 + 10 * ke + ve, 0.03, 0.03)
    w = Workload("typedsplit", spec=spec)
    c = TypedCache(w, ke, ve, 0.03, 0.03)
    try:
        q = w.q_decode()
        got, ws = c.decode(q, c.lens)
        assert ws > 0
        assert_close(got, c.oracle_decode(q, c.lens), f"typed split k={ke} v={ve}")
    finally:
        c.close()


def test_single_token_appends_into_bf16_pools():
    """The decode-step store of one token per sequence (the V path that writes
    each token on its own) into bf16 pools, then a decode over the new length."""
    spec = Spec("typedappend", 8, 2, 128, 16, [5, 16, 37, 100], 5200, None, None, new_tokens=1)
    w = Workload("typedappend", spec=spec)
    c = TypedCache(w, B, B, 1.0, 1.0, store_lens=w.lengths)
    try:
        row = w.Hkv * w.D
        for b in range(w.B):
            L = int(w.lengths[b])
            k, v = w.kv(b, L, 1)
            s = w.slots(b, L, 1)
            kv.kv_store_fp8(c.handle, 0, k.to(DEV).reshape(1, row), v.to(DEV).reshape(1, row), row, row,
                            t_dev(s), 1)
            oracle.store(bf16_bits(k), bf16_bits(v), s, c.ok, c.ov, Hkv=w.Hkv, D=w.D, BS=w.BS,
                         k_scale=1.0, v_scale=1.0)
        c.check_bytes()
        q = w.q_decode()
        got, _ = c.decode(q, w.total_lengths)
        assert_close(got, c.oracle_decode(q, w.total_lengths), "bf16 append + decode")
    finally:
        c.close()


@pytest.mark.parametrize("ke,ve", COMBOS[:3])
@pytest.mark.parametrize("Hq,Hkv,D,BS", [(4, 2, 64, 16), (32, 8, 128, 16), (16, 2, 128, 32), (12, 4, 64, 32)])
def test_typed_prefill(ke, ve, Hq, Hkv, D, BS):
    """Chunked prefill over bf16 and mixed pools: contexts of 0 and ragged
    lengths, chunks of 1, straddling and empty, a ragged last key step, fp32
    and bf16 outputs, against the oracle's attention over the same pools."""
    ctx = np.array([0, 37, 100, 5, 64], np.int32)
    chunks = np.array([21, 50, 1, 0, 160], np.int32)
    spec = Spec("typedpf", Hq, Hkv, D, BS, list(ctx + chunks), 5300 + Hq + D + BS + 10 * ke + ve, 0.04, 0.03)
    w = Workload("typedpf", spec=spec)
    log(f"typed prefill k={ke} v={ve} Hq={Hq} Hkv={Hkv} D={D} BS={BS}")
    c = TypedCache(w, ke, ve, 0.04, 0.03)
    try:
        c.check_bytes()
        cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
        g = torch.Generator().manual_seed(77 + D)
        q = torch.randn((int(cu[-1]), Hq, D), generator=g).to(torch.bfloat16)
        want = oracle.prefill_attn(bf16_bits(q), c.ok, c.ov, cu, ctx, w.block_tables, Hq=Hq, Hkv=Hkv, D=D, BS=BS,
                                   k_scale=c.ks, v_scale=c.vs, sm_scale=w.sm_scale())
        tables = t_dev(w.block_tables.astype(np.int32))
        for out_dtype in (kv.DTYPE_F32, kv.DTYPE_BF16):
            dt = torch.float32 if out_dtype == kv.DTYPE_F32 else torch.bfloat16
            out = torch.full((int(cu[-1]), Hq, D), float("nan"), dtype=dt, device=DEV)
            kv.paged_attn_prefill_chunk(c.handle, 0, q.to(DEV), Hq, t_dev(cu), t_dev(ctx), tables, w.max_blocks,
                                        w.B, int(cu[-1]), int(chunks.max()), int(ctx.max()), w.sm_scale(), out,
                                        out_dtype)
            torch.cuda.synchronize()
            got = out.float().cpu().numpy()
            assert_close(got, want, f"typed prefill k={ke} v={ve} out={out_dtype}")
            if out_dtype == kv.DTYPE_F32:
                assert float(np.max(np.abs(got - want))) <= ATOL
    finally:
        c.close()
