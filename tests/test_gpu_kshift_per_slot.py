"""GPU parity of kv_shift_rope_per_slot: every slot turned by its own delta,
bit-exact against the oracle's per-slot K-shift.

The table comes from kv_rope_table on the host (its values are checked
against the oracle's own angle table on the CPU); each slot names a row.
Covered: both pairings on the run path and the one-pair path, partial rotary
widths, several kv-head counts (odd too), skipped slots, rows outside the
table, repeated deltas in scattered order, and the long-context pool (8 x
131,072 tokens, head_dim 256) with a different delta per sequence, checked
over every byte.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import fp8_e4m3_scaled_amd as kv
import oracle
from synth import Workload
from tests.gpu_util import DEV, GpuCache, log, t_dev
from tests.test_gpu_kshift import _random_codes

pytestmark = pytest.mark.gpu

DELTAS = np.array([-4096, -1, 0, 3, 17, 100000], np.int32)


def _shift(c, slots, rows, table, rot, neox):
    kv.kv_shift_rope_per_slot(c.handle, 0, t_dev(slots), t_dev(rows), slots.size, t_dev(table),
                              table.shape[0], rot, kv.ROPE_NEOX if neox else kv.ROPE_NORM)


@pytest.mark.parametrize("BS,Hkv,D,rot,neox,theta", [
    (16, 2, 64, 64, True, 1e4),
    (16, 2, 64, 64, False, 1e4),
    (32, 2, 256, 256, True, 1e6),
    (32, 2, 256, 256, False, 1e6),
    (16, 8, 128, 128, True, 5e5),
    (16, 3, 128, 64, False, 1e4),       # odd head count, partial rotary, run path
    (16, 3, 128, 96, True, 1e4),        # one-pair path
    (32, 1, 64, 40, False, 1e4),        # one-pair path
])
def test_per_slot_matches_oracle(BS, Hkv, D, rot, neox, theta):
    rng = np.random.default_rng(BS * 100 + D + rot + Hkv + (1 if neox else 0))
    NB = 13
    pool = _random_codes(rng, (NB, Hkv, BS * D))
    slots = rng.choice(NB * BS, size=NB * BS * 3 // 4, replace=False).astype(np.int64)
    slots = np.concatenate([slots, [-1, NB * BS, NB * BS + 9]])
    rng.shuffle(slots)
    rows = rng.integers(0, DELTAS.size, slots.size).astype(np.int32)
    rows[rng.random(slots.size) < 0.05] = -1           # rows outside the table skip the slot
    rows[rng.random(slots.size) < 0.05] = DELTAS.size
    table = kv.kv_rope_table(DELTAS, theta, rot)
    log(f"kshift per slot BS={BS} Hkv={Hkv} D={D} rot={rot} neox={neox}")
    with GpuCache(NB, BS, Hkv, D) as c:
        c.k_pool[0].copy_(torch.from_numpy(pool).to(DEV))
        c.v_pool[0].copy_(torch.from_numpy(pool[::-1].copy()).to(DEV))
        _shift(c, slots, rows, table, rot, neox)
        gk, gv = c.pools()
    ok = (rows >= 0) & (rows < DELTAS.size)
    want = pool.copy()
    oracle.kshift_per_slot(want, np.where(ok, slots, -1), DELTAS[np.clip(rows, 0, DELTAS.size - 1)],
                           Hkv=Hkv, D=D, BS=BS, theta=theta, rot_dim=rot, neox=neox)
    assert np.array_equal(gk, want), f"{int((gk != want).sum())} K bytes differ"
    assert np.array_equal(gv, pool[::-1]), "V must not change"


def test_per_slot_single_row_equals_kv_shift_rope():
    """A one-row table equals kv_shift_rope with that delta, byte for byte."""
    rng = np.random.default_rng(41)
    BS, Hkv, D, NB, rot = 32, 2, 256, 9, 256
    pool = _random_codes(rng, (NB, Hkv, BS * D))
    slots = rng.permutation(NB * BS).astype(np.int64)
    outs = []
    for per_slot in (False, True):
        with GpuCache(NB, BS, Hkv, D) as c:
            c.k_pool[0].copy_(torch.from_numpy(pool).to(DEV))
            if per_slot:
                _shift(c, slots, np.zeros(slots.size, np.int32), kv.kv_rope_table([-4096], 1e6, rot), rot, True)
            else:
                kv.kv_shift_rope(c.handle, 0, t_dev(slots), slots.size, -4096, 1e6, rot, kv.ROPE_NEOX)
            outs.append(c.pools()[0])
    assert np.array_equal(outs[0], outs[1])
    assert not np.array_equal(outs[0], pool)


def test_per_slot_long_context_pool():
    """The long-context pool (8 sequences x 131,072 tokens, 2 kv-heads x 256,
    block 32, NEOX over all 256 dims, theta 1e6), each sequence shifted by its
    own delta in one call; every K byte against the oracle."""
    w = Workload("longctx")
    rng = np.random.default_rng(77)
    shape = (w.NB, w.Hkv, w.BS * w.D)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(77)
    k_dev = torch.randint(0, 256, shape, dtype=torch.uint8, device=DEV, generator=gen)
    pool = k_dev.cpu().numpy()
    deltas = np.array([-4096, -1, 1, 4096, -131072, 7, -2048, 0], np.int32)[:w.B]
    slots = np.concatenate([w.slots(b, 0, int(w.lengths[b])) for b in range(w.B)])
    rows = np.repeat(np.arange(w.B, dtype=np.int32), w.lengths.astype(np.int64))
    table = kv.kv_rope_table(deltas, w.spec.theta, w.D)
    v_dev = torch.zeros(shape, dtype=torch.uint8, device=DEV)
    h = kv.kv_cache_alloc(1, w.NB, w.BS, w.Hkv, w.D, [0.03], [0.03], kv.DTYPE_F32, k_dev, v_dev)
    try:
        log(f"per-slot shift of {slots.size} slots")
        kv.kv_shift_rope_per_slot(h, 0, t_dev(slots), t_dev(rows), slots.size, t_dev(table), w.B, w.D,
                                  kv.ROPE_NEOX)
        torch.cuda.synchronize()
        got = k_dev.cpu().numpy()
    finally:
        kv.kv_cache_free(h)
    want = pool.copy()
    bounds = np.concatenate([[0], np.cumsum(w.lengths.astype(np.int64))])

    def one(b):
        s = slots[bounds[b]:bounds[b + 1]]
        oracle.kshift_per_slot(want, s, np.full(s.size, deltas[b], np.int32), Hkv=w.Hkv, D=w.D, BS=w.BS,
                               theta=w.spec.theta, rot_dim=w.D, neox=True)

    oracle._load()
    n = max(1, min(16, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(max_workers=n) as ex:
        list(ex.map(one, range(w.B)))
    assert np.array_equal(got, want), f"{int((got != want).sum())} K bytes differ"
