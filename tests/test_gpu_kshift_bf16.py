"""GPU parity of the K-shift over bf16 K pools (the bf16 twin of the cache):
every stored bf16 value bit-exact against the oracle, for one delta and for a
delta per slot, both pairings, the 16-byte-run path and the one-pair path,
with subnormal, zero, huge, infinite and NaN values and skipped slots."""
import numpy as np
import pytest
import torch

import fp8_e4m3_scaled_amd as kv
import oracle
from tests.gpu_util import DEV, log, t_dev

pytestmark = pytest.mark.gpu

DELTAS = np.array([-4096, -1, 0, 3, 17, 100000], np.int32)


def _bf16_values(rng, n):
    x = (rng.standard_normal(n) * np.exp(rng.uniform(-30, 30, n))).astype(np.float32)
    x[rng.random(n) < 0.01] = 0.0
    b = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    special = rng.random(n)
    b[special < 0.003] = 0x7F80                      # +inf
    b[(special >= 0.003) & (special < 0.006)] = 0xFFC3   # NaN
    b[(special >= 0.006) & (special < 0.01)] = 0x0005    # subnormal
    return b


@pytest.mark.parametrize("per_slot", [False, True])
@pytest.mark.parametrize("BS,Hkv,D,rot,neox", [
    (16, 2, 64, 64, True), (16, 2, 64, 64, False), (32, 8, 128, 128, True), (16, 3, 128, 48, False),
    (16, 2, 128, 40, True), (32, 1, 64, 2, False), (16, 2, 128, 96, True),
])
def test_bf16_kshift_matches_oracle(per_slot, BS, Hkv, D, rot, neox):
    rng = np.random.default_rng(BS + 7 * Hkv + D + rot + 2 * neox + per_slot)
    NB, theta = 11, 1e4
    n = NB * Hkv * BS * D
    kbits = _bf16_values(rng, n).reshape(NB, Hkv, BS * D)
    vbits = rng.integers(0, 1 << 16, size=n, dtype=np.uint16).reshape(NB, Hkv, BS * D)
    k_dev = torch.from_numpy(kbits.view(np.int16)).to(DEV)
    v_dev = torch.from_numpy(vbits.view(np.int16)).to(DEV)
    slots = rng.choice(NB * BS, size=NB * BS * 2 // 3, replace=False).astype(np.int64)
    slots = np.concatenate([slots, [-1, NB * BS, NB * BS + 3]])
    rng.shuffle(slots)
    log(f"bf16 kshift per_slot={per_slot} BS={BS} Hkv={Hkv} D={D} rot={rot} neox={neox}")
    h = kv.kv_cache_alloc_typed(1, NB, BS, Hkv, D, kv.ELEM_BF16, kv.ELEM_BF16, None, None, kv.DTYPE_F32,
                                k_dev, v_dev)
    style = kv.ROPE_NEOX if neox else kv.ROPE_NORM
    want = kbits.copy()
    try:
        if per_slot:
            rows = rng.integers(0, DELTAS.size, slots.size).astype(np.int32)
            table = kv.kv_rope_table(DELTAS, theta, rot)
            kv.kv_shift_rope_per_slot(h, 0, t_dev(slots), t_dev(rows), slots.size, t_dev(table), DELTAS.size,
                                      rot, style)
            oracle.kshift_per_slot(want, slots, DELTAS[rows], Hkv=Hkv, D=D, BS=BS, theta=theta, rot_dim=rot,
                                   neox=neox)
        else:
            kv.kv_shift_rope(h, 0, t_dev(slots), slots.size, -7, theta, rot, style)
            oracle.kshift(want, slots, Hkv=Hkv, D=D, BS=BS, delta=-7, theta=theta, rot_dim=rot, neox=neox)
        torch.cuda.synchronize()
        gk = k_dev.cpu().numpy().view(np.uint16)
        gv = v_dev.cpu().numpy().view(np.uint16)
    finally:
        kv.kv_cache_free(h)
    assert np.array_equal(gk, want), f"{int((gk != want).sum())} K values differ"
    assert np.array_equal(gv, vbits), "V must not change"
    assert not np.array_equal(gk, kbits)
