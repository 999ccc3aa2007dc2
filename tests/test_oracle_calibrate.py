"""Pins of the oracle's scale calibration: amax over bf16 tensors and the
per-tensor scale amax / 448 in fp32 or rounded to bf16.

The pages set per-tensor scales to amax / 448 for the benchmark tensors and
name runtime calibration as unbuilt [P3, "Unreached and owed"]; 448 is the
largest finite E4M3 value [P2, ggml_fp32_to_f8_e4m3].  Pinned by:
* amax equals torch's abs-max (a library reduction the oracle does not use),
  on random tensors, with planted maxima at the first and last element, with
  negative maxima, through row strides whose padding holds larger values, and
  propagates NaN as torch does; a running amax over parts equals the whole;
* amax = 448 * 2^k gives the scale 2^k exactly; the fp32 quotient equals the
  fp64 quotient rounded to fp32 (exact, since fp64 carries more than twice
  fp32's significand bits);
* the bf16 rounding equals torch's fp32 -> bf16 conversion on random values,
  on every constructed halfway point, at overflow and for NaN;
* with the calibrated scale (fp32 or bf16) the largest element encodes to the
  top finite E4M3 code 0x7E through the independent NumPy codec, and no
  element lands beyond 448 * (1 + 2^-8).
"""
import numpy as np
import pytest
import torch

from oracle import np_codec
from synth import bf16_bits


def _rand_bits(rng, shape, scale=1.0):
    x = torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32)).to(torch.bfloat16)
    return bf16_bits(x), x


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_amax_equals_torch_abs_max(orc, seed):
    rng = np.random.default_rng(seed)
    bits, x = _rand_bits(rng, (97, 136), scale=3.0)
    want = float(x.float().abs().max())
    assert float(orc.amax(bits)) == want
    # planted maxima: first element, last element, negative
    for pos, val in ((0, 77.5), (-1, 91.0), (500, -120.0)):
        b = bits.copy().reshape(-1)
        b[pos] = bf16_bits(torch.tensor([val], dtype=torch.bfloat16))[0]
        assert float(orc.amax(b.reshape(bits.shape))) == abs(val)


def test_amax_ignores_stride_padding_and_runs(orc):
    rng = np.random.default_rng(7)
    bits, x = _rand_bits(rng, (50, 64))
    padded = np.full((50, 72), bf16_bits(torch.tensor([1e4], dtype=torch.bfloat16))[0], np.uint16)
    padded[:, :64] = bits
    assert float(orc.amax(padded, row_elems=64)) == float(x.float().abs().max())
    # running over row ranges equals the whole
    a = orc.amax(bits[:13])
    a = orc.amax(bits[13:40], start=a)
    a = orc.amax(bits[40:], start=a)
    assert float(a) == float(x.float().abs().max())
    # empty input leaves the start value
    assert float(orc.amax(bits[:0], start=2.5)) == 2.5


def test_amax_special_values(orc):
    def b(vals):
        return bf16_bits(torch.tensor(vals, dtype=torch.bfloat16))
    assert float(orc.amax(b([0.0, -0.0]))) == 0.0
    assert np.isinf(orc.amax(b([1.0, -float("inf"), 2.0])))
    for vals in ([1.0, float("nan"), 2.0], [float("nan"), float("inf")], [float("inf"), float("nan")]):
        assert np.isnan(orc.amax(b(vals)))
        assert torch.isnan(torch.tensor(vals, dtype=torch.bfloat16).float().abs().max())
    # NaN start stays NaN
    assert np.isnan(orc.amax(b([1.0]), start=float("nan")))
    # subnormal bf16 magnitudes
    tiny = np.array([0x0001, 0x8003, 0x0002], np.uint16)
    assert orc.amax(tiny) == np.float32((np.array([3 << 16], np.uint32)).view(np.float32)[0])


def test_scale_powers_of_two_and_division(orc):
    for k in range(-30, 31):
        assert orc.scale_from_amax(np.float32(448.0) * np.float32(2.0 ** k)) == np.float32(2.0 ** k)
    rng = np.random.default_rng(11)
    a = np.concatenate([
        (rng.random(20000) * 1e3).astype(np.float32),
        np.ldexp(rng.random(20000), rng.integers(-140, 127, 20000)).astype(np.float32),
    ])
    want = (a.astype(np.float64) / 448.0).astype(np.float32)
    got = np.array([orc.scale_from_amax(v) for v in a], np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert orc.scale_from_amax(0.0) == 0.0 and not orc.scale_ok(orc.scale_from_amax(0.0))
    assert np.isinf(orc.scale_from_amax(np.inf)) and not orc.scale_ok(orc.scale_from_amax(np.inf))
    assert np.isnan(orc.scale_from_amax(np.nan))


def test_bf16_rounding_equals_torch(orc):
    rng = np.random.default_rng(3)
    u = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    # constructed halfway points: low half exactly 0x8000, both parities of the kept bit
    halves = ((rng.integers(0, 2 ** 16, 4000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    halves = halves[np.isfinite(halves)]
    edge = np.array([3.3895314e38, 3.3961776e38, np.finfo(np.float32).max, -np.finfo(np.float32).max,
                     1e-45, -1e-45, 0.0, -0.0, np.inf, -np.inf], np.float32)
    allx = np.concatenate([x, halves, edge])
    want = bf16_bits(torch.from_numpy(allx).to(torch.bfloat16))
    got = orc.f32_to_bf16(allx)
    assert np.array_equal(got, want), int((got != want).sum())
    assert int(orc.f32_to_bf16(np.float32(np.nan))) == 0x7FC0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_calibrated_max_lands_on_top_code(orc, dtype):
    rng = np.random.default_rng(21)
    for trial in range(200):
        scale = float(np.exp(rng.uniform(-12, 12)))
        bits, x = _rand_bits(rng, (16, 64), scale=scale)
        a = orc.amax(bits)
        (ks, _), (kb, _) = orc.calibrate_scales(a, a, dtype)
        assert orc.scale_ok(ks)
        inv = np.float32(1.0) / np.float32(ks)
        y = (x.float().numpy() * inv).astype(np.float32)
        assert float(np.abs(y).max()) <= 448.0 * (1 + 2 ** -8)
        top = np.unravel_index(np.argmax(np.abs(x.float().numpy())), x.shape)
        assert int(np_codec.encode(y[top])) & 0x7F == 0x7E, (trial, dtype)
        if dtype == "bf16":
            assert kb == orc.f32_to_bf16(orc.scale_from_amax(a))
        else:
            assert kb == np.array([ks], np.float32).view(np.uint32)[0]
    # NaN amax gives the canonical NaN bits in both dtypes
    (_, _), (nb, _) = orc.calibrate_scales(np.nan, 1.0, dtype)
    assert int(nb) == (0x7FC00000 if dtype == "f32" else 0x7FC0)
