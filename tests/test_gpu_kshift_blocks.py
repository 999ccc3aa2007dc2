"""GPU parity of both K-shift entry points on slot lists built from whole and
broken blocks, bit-exact against the oracle.

A shift of whole sequences hands the kernels runs of block_size slots that
fill one block in order; other callers pass anything.  The list here mixes
whole blocks in order, a block in reverse order, a block with one skipped
entry, a run of block_size slots that straddles two blocks, an aligned run
past the end of the pool, a whole block with one row outside the table
(per-slot), and a short final run; blocks that no slot names must keep their
bytes.
"""
import numpy as np
import pytest
import torch

import fp8_e4m3_scaled_amd as kv
import oracle
from tests.gpu_util import DEV, GpuCache, log, t_dev
from tests.test_gpu_kshift import _random_codes

pytestmark = pytest.mark.gpu

DELTAS = np.array([-4096, -1, 0, 3, 17, 100000], np.int32)
NB = 12


def _groups(BS):
    """The slot list and, per entry, whether the per-slot test gives it a row outside the table."""
    blk = lambda b: np.arange(b * BS, (b + 1) * BS, dtype=np.int64)    # noqa: E731
    holed = blk(1).copy()
    holed[BS // 3] = -1
    groups = [blk(3), blk(7), blk(5)[::-1].copy(), holed,
              np.arange(8 * BS + BS // 2, 9 * BS + BS // 2, dtype=np.int64),   # straddles blocks 8 and 9
              blk(10), np.arange(NB * BS, (NB + 1) * BS, dtype=np.int64),      # aligned, past the pool
              blk(0)[:BS - 3]]                                                  # short final group
    bad_row = [np.zeros(g.size, bool) for g in groups]
    bad_row[5][BS - 2] = True                                                   # block 10: one row outside
    return np.concatenate(groups), np.concatenate(bad_row)


@pytest.mark.parametrize("BS,Hkv,D,rot,neox", [
    (16, 2, 64, 64, True),
    (16, 2, 64, 64, False),
    (16, 1, 64, 32, True),         # one run per row
    (32, 2, 256, 256, True),
    (32, 2, 256, 256, False),
    (16, 8, 128, 128, True),
    (16, 3, 128, 64, False),       # partial rotary
    (16, 2, 128, 96, False),       # NORM runs over three column quarters
    (32, 1, 128, 64, True),
])
@pytest.mark.parametrize("per_slot", [False, True])
def test_whole_and_broken_blocks(BS, Hkv, D, rot, neox, per_slot):
    rng = np.random.default_rng(BS * 7 + Hkv * 11 + D + rot + (1 if neox else 0) + (100 if per_slot else 0))
    pool = _random_codes(rng, (NB, Hkv, BS * D))
    slots, bad = _groups(BS)
    mode = kv.ROPE_NEOX if neox else kv.ROPE_NORM
    theta = 1e4 if D < 256 else 1e6
    log(f"kshift blocks BS={BS} Hkv={Hkv} D={D} rot={rot} neox={neox} per_slot={per_slot}")
    want = pool.copy()
    with GpuCache(NB, BS, Hkv, D) as c:
        c.k_pool[0].copy_(torch.from_numpy(pool).to(DEV))
        c.v_pool[0].copy_(torch.from_numpy(pool[::-1].copy()).to(DEV))
        if per_slot:
            rows = rng.integers(0, DELTAS.size, slots.size).astype(np.int32)
            rows[bad] = DELTAS.size
            table = kv.kv_rope_table(DELTAS, theta, rot)
            kv.kv_shift_rope_per_slot(c.handle, 0, t_dev(slots), t_dev(rows), slots.size, t_dev(table),
                                      table.shape[0], rot, mode)
            oracle.kshift_per_slot(want, np.where(bad, -1, slots), DELTAS[np.clip(rows, 0, DELTAS.size - 1)],
                                   Hkv=Hkv, D=D, BS=BS, theta=theta, rot_dim=rot, neox=neox)
        else:
            kv.kv_shift_rope(c.handle, 0, t_dev(slots), slots.size, -37, theta, rot, mode)
            oracle.kshift(want, slots, Hkv=Hkv, D=D, BS=BS, delta=-37, theta=theta, rot_dim=rot, neox=neox)
        gk, gv = c.pools()
    assert np.array_equal(gk, want), f"{int((gk != want).sum())} K bytes differ"
    assert np.array_equal(gv, pool[::-1]), "V must not change"
    for b in (2, 4, 6, 11):
        assert np.array_equal(gk[b], pool[b]), f"untouched block {b} changed"
