"""Pins of the oracle's K-shift (dequantize -> rotate -> requantize, scale-free).

[P1, tests/test-fp8.cpp check_fp8_context_shift: the expected cache bytes are
quantize(rope(to_float(bytes), shift)) with no scale; src/llama-kv-cache.cpp
build_rope_shift keeps F8_E4M3 out of the in-place rope.]

* the rotation equals a complex multiplication (x0 + i x1) * (c + i s) done
  by NumPy in complex128, rounded to fp32 and encoded by the independent
  NumPy codec, for the NEOX pairing (i, i + rot/2) and the NORM pairing
  (2i, 2i+1);
* the angle table: pair 0 turns by exactly delta radians (theta^0 = 1),
  c^2 + s^2 = 1 to fp32 accuracy, angles fall geometrically with the pair index;
* delta = 0 leaves every value unchanged (a zero may change sign); dims at or beyond rot_dim are untouched;
* shifting by +delta then -delta comes back within two rounding envelopes.
"""
import math

import numpy as np
import pytest

from oracle import np_codec


def _random_pool(rng, NB, Hkv, BS, D):
    # codes of magnitude below NaN, both signs, including subnormal codes
    mag = rng.integers(0, 0x7F, size=(NB, Hkv, BS * D), dtype=np.uint8)
    return (mag | (rng.integers(0, 2, size=mag.shape, dtype=np.uint8) << 7)).astype(np.uint8)


def _expected(orc, pool, slots, Hkv, D, BS, delta, theta, rot, neox):
    c, s = orc.rope_table(rot, delta, theta)
    out = pool.copy()
    for slot in slots:
        if slot < 0:
            continue
        blk, t = divmod(int(slot), BS)
        for h in range(Hkv):
            ko = np.array([orc.k_tile_offset(t, d, BS, D) for d in range(D)])
            x = np_codec.decode(pool[blk, h, ko]).astype(np.float64)
            half = rot // 2
            i0 = np.arange(half) if neox else 2 * np.arange(half)
            i1 = i0 + half if neox else i0 + 1
            a = np.empty(half, np.complex128)      # built field by field: keeps signed zeros
            a.real, a.imag = x[i0], x[i1]
            r = np.empty(half, np.complex128)
            r.real, r.imag = c, s
            z = a * r
            y = x.astype(np.float32)
            y[i0] = z.real.astype(np.float32)
            y[i1] = z.imag.astype(np.float32)
            codes = pool[blk, h, ko].copy()
            codes[i0] = np_codec.encode(y[i0])
            codes[i1] = np_codec.encode(y[i1])
            out[blk, h, ko] = codes
    return out


@pytest.mark.parametrize("neox", [True, False])
@pytest.mark.parametrize("BS,Hkv,D,rot,delta", [(16, 2, 64, 64, -1), (32, 2, 256, 256, -4096),
                                                 (16, 2, 128, 96, 7)])
def test_kshift_matches_complex_rotation(orc, neox, BS, Hkv, D, rot, delta):
    rng = np.random.default_rng(abs(delta) + rot)
    pool = _random_pool(rng, 6, Hkv, BS, D)
    slots = np.concatenate([rng.choice(6 * BS, size=40, replace=False), [-1]]).astype(np.int64)
    want = _expected(orc, pool, slots, Hkv, D, BS, delta, 1e6, rot, neox)
    got = pool.copy()
    orc.kshift(got, slots, Hkv=Hkv, D=D, BS=BS, delta=delta, theta=1e6, rot_dim=rot, neox=neox)
    assert np.array_equal(got, want)
    assert not np.array_equal(got, pool)


def test_rope_table_pins(orc):
    for delta in [-4096, -1, 3]:
        c, s = orc.rope_table(256, delta, 1e6)
        assert c[0] == np.float32(math.cos(delta)) and s[0] == np.float32(math.sin(delta))
        assert np.all(np.abs(c.astype(np.float64) ** 2 + s.astype(np.float64) ** 2 - 1) < 3e-7)
        ang = np.arctan2(s.astype(np.float64), c.astype(np.float64))
        # the last pair turns by delta * theta^(-254/256): tiny, so the angle is direct
        assert abs(ang[-1] - delta * 1e6 ** (-254 / 256)) < 1e-6 * max(1, abs(delta))


@pytest.mark.parametrize("rot", [256, 128, 96, 64, 2])
@pytest.mark.parametrize("theta", [1e4, 1e6])
@pytest.mark.parametrize("delta", [-4096, -1, 3, 7, 100000])
def test_rope_table_every_pair(orc, rot, theta, delta):
    """Every pair i of the table, for rotary widths equal to and below the head
    dim: cos and sin of delta * theta^(-2i/rot), taken here by another route
    (exp of a logarithm, numpy's fp64 cos/sin) and rounded to fp32, are the
    table's values to within half an fp32 step (the two fp64 angles differ by a
    few units of their last place).  An exponent over the head dim instead of
    rot, over rot - 2, or a pair index off by one fails this at every rot."""
    c, s = orc.rope_table(rot, delta, theta)
    i = np.arange(rot // 2, dtype=np.float64)
    ang = delta * np.exp(-2.0 * i / rot * np.log(np.float64(np.float32(theta))))
    for got, ref in ((c, np.cos(ang)), (s, np.sin(ang))):
        half_ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64) / 2
        assert np.all(np.abs(got.astype(np.float64) - ref) <= half_ulp + 1e-11), (rot, theta, delta)


def test_kshift_delta_zero_and_untouched_dims(orc):
    rng = np.random.default_rng(3)
    BS, Hkv, D = 16, 2, 128
    pool = _random_pool(rng, 4, Hkv, BS, D)
    slots = np.arange(4 * BS, dtype=np.int64)
    same = pool.copy()
    orc.kshift(same, slots, Hkv=Hkv, D=D, BS=BS, delta=0, theta=1e4, rot_dim=128, neox=True)
    # values are unchanged; only the sign of a zero may change, as IEEE arithmetic gives
    # (-0) - (-0) = +0 for x0*1 - x1*0 with x0 = -0 and x1 < 0
    nz = (pool & 0x7F) != 0
    assert np.array_equal(same[nz], pool[nz])
    assert np.all((same[~nz] & 0x7F) == 0)
    part = pool.copy()
    orc.kshift(part, slots, Hkv=Hkv, D=D, BS=BS, delta=-9, theta=1e4, rot_dim=64, neox=True)
    for t in range(BS):
        for d in range(64, D):
            o = orc.k_tile_offset(t, d, BS, D)
            assert np.array_equal(part[:, :, o], pool[:, :, o])


def test_kshift_nan_code_pairs(orc):
    BS, Hkv, D = 16, 1, 64
    pool = np.full((1, Hkv, BS * D), 0x38, np.uint8)
    pool[0, 0, orc.k_tile_offset(0, 0, BS, D)] = 0xFF
    orc.kshift(pool, np.array([0]), Hkv=Hkv, D=D, BS=BS, delta=5, theta=1e4, rot_dim=64, neox=True)
    assert pool[0, 0, orc.k_tile_offset(0, 0, BS, D)] == 0x7F
    assert pool[0, 0, orc.k_tile_offset(0, 32, BS, D)] == 0x7F


def test_kshift_there_and_back_within_envelope(orc):
    rng = np.random.default_rng(11)
    BS, Hkv, D = 32, 2, 256
    # normal-range codes only (exponent field 4..13), so the relative envelope applies
    e = rng.integers(4, 14, size=(3, Hkv, BS * D))
    m = rng.integers(0, 8, size=e.shape)
    pool = ((e << 3) | m | (rng.integers(0, 2, size=e.shape) << 7)).astype(np.uint8)
    slots = np.arange(3 * BS, dtype=np.int64)
    x0 = np_codec.decode(pool).astype(np.float64)
    p = pool.copy()
    orc.kshift(p, slots, Hkv=Hkv, D=D, BS=BS, delta=-4096, theta=1e6, rot_dim=256, neox=True)
    orc.kshift(p, slots, Hkv=Hkv, D=D, BS=BS, delta=4096, theta=1e6, rot_dim=256, neox=True)
    x1 = np_codec.decode(p).astype(np.float64)
    # per pair: |r(x) - x| <= 2 * 2^-4 * |pair| (+ subnormal grid), norm-preserving rotation
    half = D // 2
    for blk in range(3):
        for h in range(Hkv):
            for t in range(BS):
                ko = np.array([orc.k_tile_offset(t, d, BS, D) for d in range(D)])
                a, b = x0[blk, h, ko], x1[blk, h, ko]
                na = np.hypot(a[:half], a[half:])
                err = np.hypot(b[:half] - a[:half], b[half:] - a[half:])
                assert np.all(err <= 2 * (2 ** -4 * np.sqrt(2) * na * 1.07 + 2 ** -10 * 2))


@pytest.mark.parametrize("neox", [True, False])
def test_per_slot_deltas(orc, neox):
    """Each slot turns by its own delta [P1, tests/test-fp8.cpp
    check_fp8_context_shift: one shift value per cache cell]: one delta
    everywhere equals kshift; distinct deltas equal the NumPy complex rotation
    of each slot by its own delta, and equal kshift run on each slot alone;
    skipped slots stay untouched."""
    rng = np.random.default_rng(5 + neox)
    NB, Hkv, BS, D, rot, theta = 6, 2, 16, 64, 64, 10000.0
    pool = _random_pool(rng, NB, Hkv, BS, D)
    slots = rng.permutation(NB * BS)[:40].astype(np.int64)
    slots[3] = -1
    slots[9] = NB * BS + 5
    # one delta everywhere
    a, b = pool.copy(), pool.copy()
    orc.kshift(a, slots, Hkv=Hkv, D=D, BS=BS, delta=-3, theta=theta, rot_dim=rot, neox=neox)
    orc.kshift_per_slot(b, slots, np.full(slots.shape, -3, np.int32), Hkv=Hkv, D=D, BS=BS, theta=theta,
                        rot_dim=rot, neox=neox)
    assert np.array_equal(a, b)
    # distinct deltas, repeats not adjacent
    deltas = rng.choice(np.array([-4096, -1, 0, 5, 77], np.int32), size=slots.shape)
    got = pool.copy()
    orc.kshift_per_slot(got, slots, deltas, Hkv=Hkv, D=D, BS=BS, theta=theta, rot_dim=rot, neox=neox)
    want = pool.copy()
    alone = pool.copy()
    for sl, dl in zip(slots, deltas):
        if 0 <= sl < NB * BS:
            want = _expected(orc, want, [sl], Hkv, D, BS, int(dl), theta, rot, neox)
        orc.kshift(alone, np.array([sl]), Hkv=Hkv, D=D, BS=BS, delta=int(dl), theta=theta, rot_dim=rot,
                   neox=neox)
    assert np.array_equal(got, want)
    assert np.array_equal(got, alone)
    assert not np.array_equal(got, pool)


def _bf16_pool(rng, NB, Hkv, BS, D):
    import torch
    x = (rng.standard_normal((NB, Hkv, BS * D)) * np.exp(rng.uniform(-20, 20, (NB, Hkv, BS * D)))).astype(np.float32)
    x[rng.random(x.shape) < 0.01] = 0.0
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    bits[rng.random(bits.shape) < 0.01] = 0x0003          # subnormal bf16
    return bits


@pytest.mark.parametrize("neox", [True, False])
@pytest.mark.parametrize("per_slot", [False, True])
def test_bf16_pool_rotation(orc, neox, per_slot):
    """K-shift of a bf16 K pool (the bf16 twin of the cache): each pair is the
    NumPy complex128 rotation of the stored values, rounded to fp32 and then to
    bf16 by torch (independent of the oracle); delta 0 leaves finite values as
    they are; a NaN in a pair makes both the quiet NaN 0x7FC0."""
    import torch
    rng = np.random.default_rng(31 + neox + 2 * per_slot)
    NB, Hkv, BS, D, rot, theta = 4, 2, 16, 64, 48, 10000.0
    pool = _bf16_pool(rng, NB, Hkv, BS, D)
    slots = rng.permutation(NB * BS)[:30].astype(np.int64)
    deltas = rng.choice(np.array([-4096, -7, 0, 3, 100], np.int32), size=slots.shape)
    got = pool.copy()
    if per_slot:
        orc.kshift_per_slot(got, slots, deltas, Hkv=Hkv, D=D, BS=BS, theta=theta, rot_dim=rot, neox=neox)
    else:
        deltas[:] = -7
        orc.kshift(got, slots, Hkv=Hkv, D=D, BS=BS, delta=-7, theta=theta, rot_dim=rot, neox=neox)
    want = pool.copy()
    half = rot // 2
    i0 = np.arange(half) if neox else 2 * np.arange(half)
    i1 = i0 + half if neox else i0 + 1
    for slot, dl in zip(slots, deltas):
        blk, t = divmod(int(slot), BS)
        c, s = orc.rope_table(rot, int(dl), theta)
        for h in range(Hkv):
            ko = np.array([orc.k_tile_offset(t, d, BS, D) for d in range(D)])
            x = orc.bf16_to_f32(pool[blk, h, ko]).astype(np.float64)
            a = np.empty(half, np.complex128)
            a.real, a.imag = x[i0], x[i1]
            r = np.empty(half, np.complex128)
            r.real, r.imag = c, s
            z = a * r
            row = pool[blk, h, ko].copy()
            for idx, val in ((i0, z.real), (i1, z.imag)):
                row[idx] = torch.from_numpy(val.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            want[blk, h, ko] = row
    assert np.array_equal(got, want), int((got != want).sum())
    # delta 0 keeps finite values
    z0 = pool.copy()
    orc.kshift(z0, slots, Hkv=Hkv, D=D, BS=BS, delta=0, theta=theta, rot_dim=rot, neox=neox)
    assert np.array_equal(z0, pool)
    # NaN pairs
    nanp = pool.copy()
    blk, t = divmod(int(slots[0]), BS)
    e0 = orc.k_tile_offset(t, int(i0[1]), BS, D)
    e1 = orc.k_tile_offset(t, int(i1[1]), BS, D)
    nanp[blk, 0, e0] = 0xFFC1
    orc.kshift(nanp, slots[:1], Hkv=Hkv, D=D, BS=BS, delta=5, theta=theta, rot_dim=rot, neox=neox)
    assert nanp[blk, 0, e0] == 0x7FC0 and nanp[blk, 0, e1] == 0x7FC0
