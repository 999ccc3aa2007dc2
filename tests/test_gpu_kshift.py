"""GPU parity of kv_shift_rope: the shifted K bytes must equal the oracle's bit for bit.

Random pools carry every code class (normal, subnormal, both zeros, NaN),
both rotary pairings are covered on the 16-pair run path (NEOX rot % 32 == 0,
NORM rot % 16 == 0) and on the one-pair path (other even rot), as are skipped
slots (negative or past the pool), delta 0, and the long-context chain
store -> decode -> shift -> decode against the oracle's own chain.
"""
import numpy as np
import pytest
import torch

import fp8_e4m3_scaled_amd as kv
import oracle
from synth import Spec, Workload, bf16_bits
from tests.gpu_util import DEV, GpuCache, log, t_dev
from tests.test_gpu_decode import Filled, assert_close

pytestmark = pytest.mark.gpu


def _random_codes(rng, shape, nan_frac=0.01):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    nan = rng.random(shape) < nan_frac
    c[nan] = np.where(rng.random(int(nan.sum())) < 0.5, 0x7F, 0xFF).astype(np.uint8)
    c[~nan & ((c & 0x7F) == 0x7F)] &= 0xFE          # other 0x7F/0xFF become finite
    return c


@pytest.mark.parametrize("BS,Hkv,D,rot,neox,delta,theta", [
    (16, 2, 64, 64, True, -1, 1e4),
    (16, 2, 64, 64, False, 3, 1e4),
    (32, 2, 256, 256, True, -4096, 1e6),
    (32, 2, 256, 256, False, -4096, 1e6),
    (16, 8, 128, 128, True, 17, 5e5),
    (16, 8, 128, 64, True, -33, 1e4),      # partial rotary, run path
    (16, 3, 128, 96, True, 7, 1e4),        # rot % 32 != 0: one-pair path
    (32, 1, 64, 40, False, -5, 1e4),       # rot % 16 != 0: one-pair path
    (16, 2, 128, 2, True, 9, 1e4),
])
def test_kshift_matches_oracle(BS, Hkv, D, rot, neox, delta, theta):
    rng = np.random.default_rng(BS * 1000 + D + rot + (1 if neox else 0))
    NB = 11
    pool = _random_codes(rng, (NB, Hkv, BS * D))
    slots = rng.choice(NB * BS, size=NB * BS // 2, replace=False).astype(np.int64)
    slots = np.concatenate([slots, [-1, -7, NB * BS, NB * BS + 100]])     # skipped slots
    rng.shuffle(slots)
    log(f"kshift BS={BS} Hkv={Hkv} D={D} rot={rot} neox={neox} delta={delta}")
    with GpuCache(NB, BS, Hkv, D) as c:
        c.k_pool[0].copy_(torch.from_numpy(pool).to(DEV))
        c.v_pool[0].copy_(torch.from_numpy(pool[::-1].copy()).to(DEV))
        kv.kv_shift_rope(c.handle, 0, t_dev(slots), slots.size, delta, theta, rot,
                         kv.ROPE_NEOX if neox else kv.ROPE_NORM)
        gk, gv = c.pools()
    want = pool.copy()
    oracle.kshift(want, slots, Hkv=Hkv, D=D, BS=BS, delta=delta, theta=theta, rot_dim=rot, neox=neox)
    assert np.array_equal(gk, want), f"{int((gk != want).sum())} K bytes differ"
    assert np.array_equal(gv, pool[::-1]), "V must not change"
    assert not np.array_equal(gk, pool)


def test_kshift_delta_zero():
    rng = np.random.default_rng(9)
    BS, Hkv, D, NB = 16, 2, 128, 4
    pool = _random_codes(rng, (NB, Hkv, BS * D), nan_frac=0.0)   # a NaN partner would turn a code into 0x7F
    slots = np.arange(NB * BS, dtype=np.int64)
    with GpuCache(NB, BS, Hkv, D) as c:
        c.k_pool[0].copy_(torch.from_numpy(pool).to(DEV))
        kv.kv_shift_rope(c.handle, 0, t_dev(slots), slots.size, 0, 1e4, D, kv.ROPE_NEOX)
        gk, _ = c.pools()
    want = pool.copy()
    oracle.kshift(want, slots, Hkv=Hkv, D=D, BS=BS, delta=0, theta=1e4, rot_dim=D, neox=True)
    assert np.array_equal(gk, want)
    assert not np.any((pool & 0x7F) == 0x7F)
    same = (gk == pool) | (((gk & 0x7F) == 0) & ((pool & 0x7F) == 0))   # zeros may change sign
    assert np.all(same)


def test_long_context_decode_shift_decode():
    """The long-context chain at reduced size: head_dim 256, block 32, 16 q / 2 kv
    heads, scales 0.03; decode, shift all cached K by -4096 (theta 1e6, NEOX),
    decode again -- every step against the oracle's own chain."""
    w = Workload("longctx", scale_down=128)          # 1 sequence x 1024 tokens
    f = Filled(w)
    try:
        f.check_bytes()
        q = w.q_decode()
        qb = bf16_bits(q)
        got1 = f.decode(q.to(DEV), f.lens)
        assert_close(got1, f.oracle_decode(qb, f.lens), "decode before shift")
        slots = np.concatenate([w.slots(b, 0, int(f.lens[b])) for b in range(w.B)])
        kv.kv_shift_rope(f.cache.handle, 0, t_dev(slots), slots.size, w.spec.delta, w.spec.theta,
                         w.D, kv.ROPE_NEOX)
        oracle.kshift(f.ok, slots, Hkv=w.Hkv, D=w.D, BS=w.BS, delta=w.spec.delta,
                      theta=w.spec.theta, rot_dim=w.D, neox=True)
        f.check_bytes()
        got2 = f.decode(q.to(DEV), f.lens)
        want2 = f.oracle_decode(qb, f.lens)
        assert_close(got2, want2, "decode after shift")
        assert not np.allclose(got1, got2)
    finally:
        f.close()
