"""Pins of the oracle's store (quantize -> byte pools) and tile layout.

* the tile layout is a bijection of every (block, kv-head) tile;
* store followed by the dequantizing gather returns fl32(decode(encode(fl32(x*fl32(1/s))))*s)
  computed with the independent NumPy codec, every untouched byte stays 0, and
  negative slots are skipped;
* the rounding envelope |s*decode(store(x)) - x| <= 2^-4|x| + 2^-10|s| (+ fp32 slack)
  read off the format [P3, "What the THIRD fresh review found"], with the
  pages' anti-vacuity conditions, and a planted scale mistake leaves it;
* power-of-two scale invariance [P3, "Round 4"]: s*D(Q(x/s)) == s'*D(Q(x/s'))
  bitwise when every value is normal and unsaturated at both scales;
* multiply-by-inverse equals divide for power-of-two scales;
* KVBytesPerBlock for one-byte elements is exactly half the bf16 figure
  [P3, W3 summary "KVBytesPerBlock exactly halved"].
"""
import numpy as np
import pytest
import torch

from oracle import np_codec
from synth import Workload, bf16_bits


LAYOUTS = [(16, 64), (16, 128), (32, 256), (16, 256), (32, 128), (32, 64)]


@pytest.mark.parametrize("BS,D", LAYOUTS)
def test_tile_layout_is_a_bijection(orc, BS, D):
    ko = sorted(orc.k_tile_offset(t, d, BS, D) for t in range(BS) for d in range(D))
    vo = sorted(orc.v_tile_offset(t, d, BS, D) for t in range(BS) for d in range(D))
    assert ko == list(range(BS * D))
    assert vo == list(range(BS * D))


@pytest.mark.parametrize("BS,D", [(16, 128), (32, 256)])
def test_tile_layout_structure(orc, BS, D):
    """K: each token's quarter-row of D/4 dims is one contiguous run; V: within a
    group of four tokens, the four tokens of one dim are four consecutive bytes."""
    q = D // 4
    for t in range(BS):
        for c in range(4):
            offs = [orc.k_tile_offset(t, c * q + i, BS, D) for i in range(q)]
            assert offs == list(range(offs[0], offs[0] + q))
    for g in range(BS // 4):
        for d in range(D):
            offs = [orc.v_tile_offset(4 * g + i, d, BS, D) for i in range(4)]
            assert offs == list(range(offs[0], offs[0] + 4))


def _expected_dequant(x_bits, scale):
    x = (x_bits.astype(np.uint32) << 16).view(np.float32)
    inv = np.float32(1.0) / np.float32(scale)
    y = (x * inv).astype(np.float32)
    return (np_codec.decode(np_codec.encode(y)) * np.float32(scale)).astype(np.float32)


def _store_tiny(orc, k_scale=0.02, v_scale=0.015):
    w = Workload("tiny")
    Hkv, D, BS = w.Hkv, w.D, w.BS
    kp = np.zeros((w.NB, Hkv, BS * D), np.uint8)
    vp = np.zeros_like(kp)
    kvs = []
    for b in range(w.B):
        L = int(w.lengths[b])
        k, v = w.kv(b, 0, L)
        kb, vb = bf16_bits(k), bf16_bits(v)
        orc.store(kb, vb, w.slots(b, 0, L), kp, vp, Hkv=Hkv, D=D, BS=BS,
                  k_scale=k_scale, v_scale=v_scale)
        kvs.append((kb, vb))
    return w, kp, vp, kvs


def test_store_then_gather_roundtrip(orc):
    w, kp, vp, kvs = _store_tiny(orc)
    for b in range(w.B):
        L = int(w.lengths[b])
        for h in range(w.Hkv):
            kd, vd = orc.gather_dequant(kp, vp, w.block_tables[b], L, h, Hkv=w.Hkv, D=w.D, BS=w.BS,
                                        k_scale=0.02, v_scale=0.015)
            ek = _expected_dequant(kvs[b][0][:, h, :], 0.02)
            ev = _expected_dequant(kvs[b][1][:, h, :], 0.015)
            assert np.array_equal(kd.view(np.uint32), ek.view(np.uint32))
            assert np.array_equal(vd.view(np.uint32), ev.view(np.uint32))


def test_store_touches_only_its_slots(orc):
    w, kp, vp, _ = _store_tiny(orc)
    used = np.zeros(w.NB * w.BS, bool)
    for b in range(w.B):
        used[w.slots(b, 0, int(w.lengths[b]))] = True
    assert used.sum() == int(w.lengths.sum())
    # every unused slot's bytes are still zero (slots are whole rows in every tile)
    for s in np.flatnonzero(~used):
        blk, t = divmod(int(s), w.BS)
        for h in range(w.Hkv):
            for d in range(w.D):
                assert kp[blk, h, orc.k_tile_offset(t, d, w.BS, w.D)] == 0
                assert vp[blk, h, orc.v_tile_offset(t, d, w.BS, w.D)] == 0


def test_negative_slots_are_skipped(orc):
    Hkv, D, BS = 2, 64, 16
    kp = np.zeros((2, Hkv, BS * D), np.uint8)
    vp = np.zeros_like(kp)
    x = bf16_bits(torch.ones((3, Hkv, D), dtype=torch.bfloat16))
    orc.store(x, x, np.array([-1, 5, -7]), kp, vp, Hkv=Hkv, D=D, BS=BS, k_scale=1.0, v_scale=1.0)
    assert np.count_nonzero(kp) == Hkv * D and np.count_nonzero(vp) == Hkv * D
    assert set(np.unique(kp)) == {0, 0x38}


def test_inf_and_nan_inputs(orc):
    Hkv, D, BS = 1, 64, 16
    kp = np.zeros((1, Hkv, BS * D), np.uint8)
    vp = np.zeros_like(kp)
    vals = np.array([np.inf, -np.inf, np.nan, -np.nan, 1e30, -1e30, 0.0, -0.0], np.float32)
    row = np.zeros(D, np.float32)
    row[:8] = vals
    bits = (row.view(np.uint32) >> 16).astype(np.uint16).reshape(1, 1, D)
    orc.store(bits, bits, np.array([0]), kp, vp, Hkv=Hkv, D=D, BS=BS, k_scale=0.5, v_scale=-0.25)
    kc = [kp[0, 0, orc.k_tile_offset(0, d, BS, D)] for d in range(8)]
    vc = [vp[0, 0, orc.v_tile_offset(0, d, BS, D)] for d in range(8)]
    assert kc == [0x7E, 0xFE, 0x7F, 0xFF, 0x7E, 0xFE, 0x00, 0x80]
    # a negative scale flips the sign of every finite/infinite value; NaN keeps its own sign
    assert vc == [0xFE, 0x7E, 0x7F, 0xFF, 0xFE, 0x7E, 0x80, 0x00]


def _envelope_ok(x, kd, s):
    bound = 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * abs(s) + 2.0 ** -20 * np.abs(x)
    return np.abs(kd.astype(np.float64) - x.astype(np.float64)) <= bound


def test_store_rounding_envelope_with_anti_vacuity(orc):
    # non-unit, unequal scales as on the page; magnitudes that put most values in the
    # normal range and some in the subnormal range, never saturating
    w, kp, vp, kvs = _store_tiny(orc, k_scale=0.125, v_scale=0.25)
    n_norm = n_tot = 0
    for b in range(w.B):
        L = int(w.lengths[b])
        for h in range(w.Hkv):
            kd, vd = orc.gather_dequant(kp, vp, w.block_tables[b], L, h, Hkv=w.Hkv, D=w.D,
                                        BS=w.BS, k_scale=0.125, v_scale=0.25)
            xk = orc.bf16_to_f32(kvs[b][0][:, h, :])
            xv = orc.bf16_to_f32(kvs[b][1][:, h, :])
            assert np.all(np.abs(xk / 0.125) < 448) and np.all(np.abs(xv / 0.25) < 448)
            assert _envelope_ok(xk, kd, 0.125).all()
            assert _envelope_ok(xv, vd, 0.25).all()
            n_norm += int((np.abs(xk / 0.125) >= 2 ** -6).sum())
            n_tot += xk.size
            # planted mistake: reading with 8x the store scale must leave the envelope
            assert not _envelope_ok(xk, kd * 8, 0.125).all()
            # planted mistake: K read as V leaves the envelope
            assert not _envelope_ok(xk, vd, 0.125).all()
    assert n_norm > 0.9 * n_tot


@pytest.mark.parametrize("pair", [(2.0 ** -7, 2.0 ** -13), (2.0 ** -11, 2.0 ** -9)])
def test_power_of_two_scale_invariance(orc, pair):
    rng = np.random.default_rng(5)
    # magnitudes whose x/s is normal and unsaturated for every scale used
    mag = np.exp2(rng.uniform(-8.5, -5.5, size=4096))
    x = (mag * np.where(rng.random(4096) < 0.5, -1, 1)).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    x = (bits.astype(np.uint32) << 16).view(np.float32)
    outs = []
    for s in pair:
        inv = np.float32(1.0) / np.float32(s)
        y = (x * inv).astype(np.float32)
        assert np.all(np.abs(y) >= 2 ** -6) and np.all(np.abs(y) < 448)
        codes = orc.e4m3_encode(y)
        outs.append((codes, (orc.e4m3_decode(codes) * np.float32(s)).astype(np.float32)))
    assert not np.array_equal(outs[0][0], outs[1][0])            # bytes differ
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))


def test_multiply_by_inverse_equals_divide_for_power_of_two_scales(orc):
    x = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)
    x = x[np.isfinite(x)]
    for s in [2.0 ** -7, 0.125, 1.0, 4.0, 2.0 ** 20]:
        inv = orc.scale_inverse(s)
        with np.errstate(over="ignore"):
            a = orc.e4m3_encode((x * inv).astype(np.float32))
            b = orc.e4m3_encode((x / np.float32(s)).astype(np.float32))
        assert np.array_equal(a, b)


def test_scale_validation(orc):
    assert orc.scale_ok(0.02) and orc.scale_ok(-0.5) and orc.scale_ok(1e-38)
    for bad in [0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, 2.0 ** -130]:
        assert not orc.scale_ok(bad)


@pytest.mark.parametrize("BS,Hkv,D", [(16, 2, 64), (16, 8, 128), (32, 2, 256)])
def test_fp8_block_bytes_are_exactly_half(orc, BS, Hkv, D):
    fp8 = orc.kv_bytes_per_block(BS, Hkv, D, 1)
    bf16 = orc.kv_bytes_per_block(BS, Hkv, D, 2)
    assert 2 * fp8 == bf16
    assert fp8 == 2 * BS * Hkv * D      # K and V, one byte per element
    budget = 1 << 30
    assert budget // fp8 >= 2 * (budget // bf16)   # a byte budget at least doubles the block count


def test_slots_past_the_pool_are_skipped(orc):
    """Negative slots and slots at or past NB*BS are skipped by the store and the
    K-shift (the boundary's contract): nothing is written, nothing outside the pool."""
    Hkv, D, BS, NB = 2, 64, 16, 3
    kp = np.zeros((NB, Hkv, BS * D), np.uint8)
    vp = np.zeros_like(kp)
    x = bf16_bits(torch.ones((4, Hkv, D), dtype=torch.bfloat16))
    orc.store(x, x, np.array([NB * BS, NB * BS + 5, -3, 1 << 40]), kp, vp, Hkv=Hkv, D=D, BS=BS,
              k_scale=1.0, v_scale=1.0)
    assert not kp.any() and not vp.any()
    kp[:] = 0x38
    before = kp.copy()
    orc.kshift(kp, np.array([NB * BS, -1, 1 << 40]), Hkv=Hkv, D=D, BS=BS, delta=3, theta=1e4,
               rot_dim=D, neox=True)
    assert np.array_equal(kp, before)
