"""GPU parity on inputs with non-finite values and extreme query rows.

NaN is a storable E4M3 code (the encoder maps NaN to sign|0x7F), and a bf16
pool keeps infinities and NaNs as given.  The definition sums, for each query
row, over the keys the row sees and only those, so:
  * a NaN V value at a key past a row's position (inside the prefill's
    diagonal 32-key step) must not reach that row; rows that see it are NaN in
    that dim;
  * a seen +-Inf V value (bf16 pools) makes the dim an infinity of its sign,
    NaN with both signs, whatever the key's probability;
  * a NaN K code makes every row that sees its key NaN.
Outputs are compared element by element with the fp64 oracle: NaN where it is
NaN, the same infinity where it is infinite, and the attention tolerance on
every finite element.  Covered for the prefill and the decode (with split-K),
all four K/V element-type combinations, fp32 and bf16 outputs.

Extreme query rows exercise the prefill's two-term E4M3 split of Q: a
dominant element with the rest 2^-9 .. 2^-24 below it, all-subnormal bf16
rows, rows with max |q| between 2^-133 and 2^-118, and rows holding +-Inf or
NaN, against K codes at and near +-448.
"""
import numpy as np
import pytest
import torch

import fp8_e4m3_scaled_amd as kv
import oracle
from synth import bf16_bits
from tests.gpu_util import DEV, log, t_dev
from tests.test_gpu_decode import ATOL, assert_close

pytestmark = pytest.mark.gpu

E, B = kv.ELEM_E4M3, kv.ELEM_BF16
NP = {E: np.uint8, B: np.uint16}
EB = {E: 1, B: 2}
COMBOS = [(E, E), (E, B), (B, E), (B, B)]


def assert_match(got, want, what, f32):
    """NaN where the oracle is NaN, the same infinity where it is infinite, and
    the attention tolerance on every finite element (plus max |d| <= 2e-3 for
    fp32 outputs)."""
    got = np.asarray(got, np.float64)
    nan_w, nan_g = np.isnan(want), np.isnan(got)
    assert np.array_equal(nan_w, nan_g), (f"{what}: NaN pattern differs: {int((nan_w & ~nan_g).sum())} missing, "
                                          f"{int((nan_g & ~nan_w).sum())} extra")
    inf_w, inf_g = np.isinf(want), np.isinf(got)
    assert np.array_equal(inf_w, inf_g), (f"{what}: infinity pattern differs: {int((inf_w & ~inf_g).sum())} "
                                          f"missing, {int((inf_g & ~inf_w).sum())} extra")
    assert np.array_equal(np.sign(got[inf_w]), np.sign(want[inf_w])), f"{what}: infinities of the wrong sign"
    fin = ~nan_w & ~inf_w
    assert_close(got[fin], want[fin], what)
    if f32 and fin.any():
        err = float(np.max(np.abs(got[fin] - want[fin])))
        assert err <= ATOL, f"{what}: fp32 max |d| {err:.3g} > {ATOL}"


class Cache:
    """A one-layer cache with explicit bf16 K/V rows per sequence ([L][Hkv][D]),
    stored through kv_store_fp8 on the GPU and through the oracle's store."""

    def __init__(self, ke, ve, Hkv, D, BS, ks_vs, k_rows, v_rows, seed):
        self.ke, self.ve, self.Hkv, self.D, self.BS = ke, ve, Hkv, D, BS
        self.lens = np.array([r.shape[0] for r in k_rows], np.int64)
        self.B = len(k_rows)
        self.max_blocks = int((self.lens.max() + BS - 1) // BS)
        self.NB = self.B * self.max_blocks + 3
        rng = np.random.default_rng(seed)
        self.tables = rng.permutation(self.NB)[:self.B * self.max_blocks].reshape(self.B, self.max_blocks)
        self.tables = self.tables.astype(np.int32)
        self.ks = np.float32(ks_vs[0] if ke == E else 1.0)
        self.vs = np.float32(ks_vs[1] if ve == E else 1.0)
        n = self.NB * Hkv * BS * D
        self.k_pool = torch.zeros(n * EB[ke], dtype=torch.uint8, device=DEV)
        self.v_pool = torch.zeros(n * EB[ve], dtype=torch.uint8, device=DEV)
        self.handle = kv.kv_cache_alloc_typed(1, self.NB, BS, Hkv, D, ke, ve, [float(self.ks)], [float(self.vs)],
                                              kv.DTYPE_F32, self.k_pool, self.v_pool)
        shape = (self.NB, Hkv, BS * D)
        self.ok = np.zeros(shape, NP[ke])
        self.ov = np.zeros(shape, NP[ve])
        row = Hkv * D
        for b in range(self.B):
            L = int(self.lens[b])
            pos = np.arange(L)
            slots = (self.tables[b, pos // BS].astype(np.int64) * BS + pos % BS).astype(np.int64)
            k, v = k_rows[b], v_rows[b]
            kv.kv_store_fp8(self.handle, 0, k.to(DEV).reshape(L, row), v.to(DEV).reshape(L, row), row, row,
                            t_dev(slots), L)
            oracle.store(bf16_bits(k), bf16_bits(v), slots, self.ok, self.ov, Hkv=Hkv, D=D, BS=BS,
                         k_scale=self.ks, v_scale=self.vs)
        torch.cuda.synchronize()
        gk = self.k_pool.cpu().numpy().view(NP[ke]).reshape(shape)
        gv = self.v_pool.cpu().numpy().view(NP[ve]).reshape(shape)
        assert np.array_equal(gk, self.ok) and np.array_equal(gv, self.ov), "stored elements differ"

    def prefill(self, q, Hq, ctx, chunks, sm_scale, out_dtype):
        cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
        T = int(cu[-1])
        dt = torch.float32 if out_dtype == kv.DTYPE_F32 else torch.bfloat16
        out = torch.full((T, Hq, self.D), 7.0, dtype=dt, device=DEV)
        kv.paged_attn_prefill_chunk(self.handle, 0, q.to(DEV), Hq, t_dev(cu), t_dev(np.asarray(ctx, np.int32)),
                                    t_dev(self.tables), self.max_blocks, self.B, T, int(max(chunks)),
                                    int(max(ctx)), sm_scale, out, out_dtype)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        want = oracle.prefill_attn(bf16_bits(q), self.ok, self.ov, cu, np.asarray(ctx, np.int32), self.tables,
                                   Hq=Hq, Hkv=self.Hkv, D=self.D, BS=self.BS, k_scale=self.ks, v_scale=self.vs,
                                   sm_scale=sm_scale)
        return got, want

    def decode(self, q, Hq, lens, sm_scale, out_dtype):
        lens = np.asarray(lens, np.int32)
        max_len = int(lens.max())
        ws_bytes = kv.paged_attn_decode_workspace(self.handle, self.B, Hq, max_len)
        ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=DEV)
        dt = torch.float32 if out_dtype == kv.DTYPE_F32 else torch.bfloat16
        out = torch.full((self.B, Hq, self.D), 7.0, dtype=dt, device=DEV)
        kv.paged_attn_decode(self.handle, 0, q.to(DEV), Hq, t_dev(self.tables), self.max_blocks, t_dev(lens),
                             self.B, max_len, sm_scale, out, out_dtype, ws, ws_bytes)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        want = oracle.decode_attn(bf16_bits(q), self.ok, self.ov, self.tables, lens, Hq=Hq, Hkv=self.Hkv,
                                  D=self.D, BS=self.BS, k_scale=self.ks, v_scale=self.vs, sm_scale=sm_scale)
        return got, want, ws_bytes

    def close(self):
        if self.handle:
            kv.kv_cache_free(self.handle)
            self.handle = None


def _rows(lens, Hkv, D, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return [(torch.randn((int(L), Hkv, D), generator=g) * scale).to(torch.bfloat16) for L in lens]


NAN, INF = float("nan"), float("inf")

# (sequence, position, kv-head, dim, value) placed in V, and in K: keys inside
# the diagonal steps of the chunks below (context 40 / 0 / 100, chunks of
# 70 / 45 / 33 tokens), and one past the shorter decode length.
V_SPECIALS = [
    (0, 45, 0, 3, NAN), (0, 47, 1, 100, NAN), (0, 61, 0, 7, INF), (0, 66, 0, 7, -INF),
    (0, 102, 1, 9, INF), (1, 2, 0, 0, NAN), (1, 14, 1, 31, -INF), (1, 33, 0, 64, INF),
    (2, 101, 1, 5, NAN), (2, 110, 0, 90, INF), (2, 110, 1, 90, -INF), (2, 131, 0, 11, NAN),
]
K_SPECIALS = [(0, 52, 1, 17, NAN), (1, 20, 0, 40, NAN), (2, 120, 1, 2, NAN)]
K_INF = [(1, 9, 1, 60, INF), (2, 104, 0, 33, -INF)]       # bf16 K pools only (E4M3 saturates them)


def _place(rows, specials, D):
    for b, pos, h, d, val in specials:
        if pos < rows[b].shape[0] and d < D:
            rows[b][pos, h, d] = val


@pytest.mark.parametrize("ke,ve", COMBOS, ids=["e4m3", "e4m3K_bf16V", "bf16K_e4m3V", "bf16"])
@pytest.mark.parametrize("D", [128, 64])
def test_nonfinite_values_inside_diagonal_steps(ke, ve, D):
    Hq, Hkv, BS = 8, 2, 16
    ctx, chunks = [40, 0, 100], [70, 45, 33]
    lens = [c + n for c, n in zip(ctx, chunks)]
    k_rows = _rows(lens, Hkv, D, 71 + D)
    v_rows = _rows(lens, Hkv, D, 72 + D)
    _place(v_rows, V_SPECIALS, D)
    _place(k_rows, K_SPECIALS, D)
    if ke == B:
        _place(k_rows, K_INF, D)
    c = Cache(ke, ve, Hkv, D, BS, (0.02, 0.015), k_rows, v_rows, 700 + D)
    try:
        g = torch.Generator().manual_seed(73 + D)
        q = torch.randn((sum(chunks), Hq, D), generator=g).to(torch.bfloat16)
        sm = 1.0 / np.sqrt(D)
        for out_dtype in (kv.DTYPE_F32, kv.DTYPE_BF16):
            f32 = out_dtype == kv.DTYPE_F32
            log(f"non-finite prefill ke={ke} ve={ve} D={D} out={'f32' if f32 else 'bf16'}")
            got, want = c.prefill(q, Hq, ctx, chunks, sm, out_dtype)
            # the placed values must matter: some rows NaN or infinite, others finite
            nonfin = ~np.isfinite(want)
            assert nonfin.any() and (~nonfin).any()
            if ve == E:
                # a NaN V at position 45 of sequence 0 (chunk token 5): chunk
                # rows 0..4 of head group 0 stay finite, rows 5.. are NaN in dim 3
                assert np.isfinite(want[0:5, 0:4, 3]).all() and np.isnan(want[5:20, 0:4, 3]).all()
            assert_match(got, want, "prefill", f32)

            log(f"non-finite decode ke={ke} ve={ve} D={D}")
            qd = q[np.cumsum(chunks) - 1].contiguous()
            for dl in (lens, [41, 30, 104]):
                got, want, ws = c.decode(qd, Hq, dl, sm, out_dtype)
                assert ws > 0 or dl != lens                   # full lengths: split-K and the reduce
                assert_match(got, want, f"decode lens {dl}", f32)
    finally:
        c.close()


def _extreme_q(T, Hq, D, seed):
    """Query rows of several kinds, as float32 before the bf16 rounding."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, Hq, D)).astype(np.float32)
    kinds = []
    for t in range(T):
        for h in range(Hq):
            kind = (t * Hq + h) % 8
            kinds.append(kind)
            if kind == 0:      # one dominant element, the rest 2^-9 .. 2^-24 of it, random signs
                r = np.exp2(-rng.uniform(9, 24, D)) * rng.choice([-1.0, 1.0], D)
                r[rng.integers(D)] = rng.choice([-1.0, 1.0]) * rng.uniform(1, 4)
                q[t, h] = r
            elif kind == 1:    # a dominant element and a tail just under 2^-10 of it
                r = rng.uniform(0.5, 1.0, D) * 2.0 ** -11 * rng.choice([-1.0, 1.0], D)
                r[rng.integers(D)] = 1.9
                q[t, h] = r
            elif kind == 2:    # all bf16 subnormals
                q[t, h] = rng.integers(-127, 128, D) * 2.0 ** -133
            elif kind == 3:    # max |q| between 2^-126 and 2^-118
                q[t, h] = rng.standard_normal(D) * 2.0 ** rng.uniform(-126, -118)
            elif kind == 4:    # two large elements of opposite sign, the rest tiny
                r = rng.standard_normal(D) * 2.0 ** -15
                r[0], r[-1] = 3.0, -2.5
                q[t, h] = r
            elif kind == 5 and t % 3 == 0:
                q[t, h, rng.integers(D)] = np.inf
            elif kind == 6 and t % 3 == 1:
                q[t, h, rng.integers(D)] = np.nan
            # kind 7 (and 5, 6 otherwise): ordinary N(0, 1)
    return torch.from_numpy(q).to(torch.bfloat16), np.array(kinds).reshape(T, Hq)


@pytest.mark.parametrize("ke,ve", COMBOS, ids=["e4m3", "e4m3K_bf16V", "bf16K_e4m3V", "bf16"])
@pytest.mark.parametrize("G", [4, 1])
def test_extreme_query_rows(ke, ve, G):
    Hkv, D, BS = 2, 128, 16
    Hq = Hkv * G
    ctx, chunks = [90, 0, 300], [70, 129, 40]
    lens = [c + n for c, n in zip(ctx, chunks)]
    ks, vs = 0.02, 0.015
    # K at and near the code maximum: +-448 and +-416 times the scale
    g = torch.Generator().manual_seed(91 + G)
    k_rows = []
    for L in lens:
        mag = torch.where(torch.rand((L, Hkv, D), generator=g) < 0.5, 448.0, 416.0)
        sign = torch.where(torch.rand((L, Hkv, D), generator=g) < 0.5, -1.0, 1.0)
        k = mag * sign * ks
        k[torch.rand((L, Hkv, D), generator=g) < 0.5] *= 0.01     # and ordinary small codes
        k_rows.append(k.to(torch.bfloat16))
    v_rows = _rows(lens, Hkv, D, 92 + G)
    c = Cache(ke, ve, Hkv, D, BS, (ks, vs), k_rows, v_rows, 800 + G)
    try:
        q, kinds = _extreme_q(sum(chunks), Hq, D, 93 + G)
        sm = 1.0 / np.sqrt(D)
        for out_dtype in (kv.DTYPE_F32, kv.DTYPE_BF16):
            f32 = out_dtype == kv.DTYPE_F32
            log(f"extreme Q prefill ke={ke} ve={ve} G={G} out={'f32' if f32 else 'bf16'}")
            got, want = c.prefill(q, Hq, ctx, chunks, sm, out_dtype)
            assert np.isnan(want[kinds == 5]).any() and np.isfinite(want[kinds == 0]).all()
            assert_match(got, want, "prefill, extreme Q rows", f32)
    finally:
        c.close()
