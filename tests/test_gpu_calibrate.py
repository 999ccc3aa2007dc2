"""GPU parity of the on-device scale calibration: the running K/V maxima
bit-exact against the oracle's amax, and the scales amax / 448 bit-exact in
fp32 and in bf16, over ragged shapes, strided rows (K and V as slices of one
fused row), planted maxima, padding that must not count, infinities, NaN,
running calls over parts, one side only, and the full Llama-shaped and
variable-length fills (the latter one call per sequence, as a serving loop
would calibrate)."""
import numpy as np
import pytest
import torch

import fp8_e4m3_scaled_amd as kv
import oracle
from synth import Workload, bf16_bits
from tests.gpu_util import DEV, bits_dev, log

pytestmark = pytest.mark.gpu

QNAN = 0x7FC00000


def _u32(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.view(torch.int32).cpu().numpy().view(np.uint32)


def _f32_bits(x) -> int:
    x = np.float32(x)
    return QNAN if np.isnan(x) else int(np.array([x], np.float32).view(np.uint32)[0])


def _calibrate(k, v, ks, vs, T, row, amax=None, dtype=kv.DTYPE_F32):
    """One call; returns (amax tensor, scale bits as uint32 numpy [2])."""
    amax = torch.zeros(2, dtype=torch.float32, device=DEV) if amax is None else amax
    out = torch.full((2,), -1, dtype=torch.int32 if dtype == kv.DTYPE_F32 else torch.int16, device=DEV)
    kv.kv_calibrate_scales(k, v, ks, vs, T, row, amax, out, dtype)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    bits = o.view(np.uint32) if dtype == kv.DTYPE_F32 else o.view(np.uint16).astype(np.uint32)
    return amax, bits


def _check(amax_t, bits, want_k, want_v, dtype):
    got = _u32(amax_t)
    assert got[0] == _f32_bits(want_k), (hex(got[0]), want_k)
    assert got[1] == _f32_bits(want_v), (hex(got[1]), want_v)
    _, wb = oracle.calibrate_scales(want_k, want_v, "f32" if dtype == kv.DTYPE_F32 else "bf16")
    assert int(bits[0]) == int(wb[0]) and int(bits[1]) == int(wb[1]), (bits, wb)


def _fused(rng, T, row, pad, scale):
    """bf16 bits [T][2*row + pad]: K then V then padding (which must not count)."""
    x = (rng.standard_normal((T, 2 * row + pad)) * scale).astype(np.float32)
    b = bf16_bits(torch.from_numpy(x).to(torch.bfloat16))
    if pad:
        b[:, 2 * row:] = 0x7F00          # bf16 1.7e38: larger than any element
    return b


SHAPES = [(1, 8, 0), (3, 64, 8), (17, 136, 0), (257, 1024, 0), (1000, 2048, 16), (4099, 512, 24),
          (40000, 1024, 0)]


@pytest.mark.parametrize("T,row,pad", SHAPES)
@pytest.mark.parametrize("dtype", [kv.DTYPE_F32, kv.DTYPE_BF16])
def test_calibrate_matches_oracle(T, row, pad, dtype):
    rng = np.random.default_rng(T + row + pad + 7 * dtype)
    log(f"calibrate T={T} row={row} pad={pad} dtype={dtype}")
    for scale in (1.0, 37.0, 1e-38):
        b = _fused(rng, T, row, pad, scale)
        # planted maxima: V's at its last element of the last row, K's negative mid-way
        b[-1, 2 * row - 1] = 0x4F00 if scale == 1.0 else b[-1, 2 * row - 1]
        b[T // 2, row // 3] = 0xCF40 if scale == 1.0 else b[T // 2, row // 3]
        dev = bits_dev(b)
        stride = 2 * row + pad
        amax, bits = _calibrate(dev[:, :row], dev[:, row:2 * row], stride, stride, T, row, dtype=dtype)
        _check(amax, bits, oracle.amax(b[:, :row]), oracle.amax(b[:, row:2 * row]), dtype)


@pytest.mark.parametrize("dtype", [kv.DTYPE_F32, kv.DTYPE_BF16])
def test_calibrate_running_parts_one_side_and_specials(dtype):
    rng = np.random.default_rng(99)
    T, row = 3000, 256
    b = _fused(rng, T, row, 0, 3.0)
    dev = bits_dev(b)
    s = 2 * row
    # three calls over row ranges equal the whole
    amax = torch.zeros(2, dtype=torch.float32, device=DEV)
    for lo, hi in ((0, 1), (1, 1400), (1400, T)):
        amax, bits = _calibrate(dev[lo:, :row], dev[lo:, row:], s, s, hi - lo, row, amax=amax, dtype=dtype)
    _check(amax, bits, oracle.amax(b[:, :row]), oracle.amax(b[:, row:]), dtype)
    # one side only: V's maximum stays where it was
    amax = torch.tensor([0.0, 5.0], dtype=torch.float32, device=DEV)
    amax, bits = _calibrate(dev[:, :row], None, s, s, T, row, amax=amax, dtype=dtype)
    _check(amax, bits, oracle.amax(b[:, :row]), np.float32(5.0), dtype)
    # no tokens: scales from the state alone (448*3 -> 3; 0 -> 0)
    amax = torch.tensor([448.0 * 3, 0.0], dtype=torch.float32, device=DEV)
    amax, bits = _calibrate(dev, dev, s, s, 0, row, amax=amax, dtype=dtype)
    _check(amax, bits, np.float32(448.0 * 3), np.float32(0.0), dtype)
    # infinity in K, NaN in V (NaN stays NaN on a later clean call)
    b2 = b.copy()
    b2[1234, 17] = 0xFF80
    b2[2999, row + 255] = 0x7FA1
    d2 = bits_dev(b2)
    amax, bits = _calibrate(d2[:, :row], d2[:, row:], s, s, T, row, dtype=dtype)
    _check(amax, bits, np.float32(np.inf), np.float32(np.nan), dtype)
    amax, bits = _calibrate(dev[:, :row], dev[:, row:], s, s, T, row, amax=amax, dtype=dtype)
    _check(amax, bits, np.float32(np.inf), np.float32(np.nan), dtype)


def test_calibrate_full_llama8b_fill():
    """The Llama-shaped fill (64 x 4096 tokens, 8 x 128 per row, outlier
    channels): one call over the whole fill and a running call per sequence,
    both equal to the oracle's amax over the same bits; the fp32 scales also
    equal the ones the input generator derives for this workload."""
    w = Workload("llama8b", device=torch.device(DEV))
    row = w.Hkv * w.D
    T = int(w.total_lengths.sum())
    K = torch.empty((T, row), dtype=torch.bfloat16, device=DEV)
    V = torch.empty_like(K)
    run = torch.zeros(2, dtype=torch.float32, device=DEV)
    pos = 0
    for b in range(w.B):
        L = int(w.total_lengths[b])
        k, v = w.kv(b, 0, L)
        K[pos:pos + L] = k.reshape(L, row)
        V[pos:pos + L] = v.reshape(L, row)
        kv.kv_calibrate_scales(K[pos:], V[pos:], row, row, L, row, run)
        pos += L
    amax, bits = _calibrate(K, V, row, row, T, row)
    want_k, want_v = oracle.amax(bf16_bits(K)), oracle.amax(bf16_bits(V))
    _check(amax, bits, want_k, want_v, kv.DTYPE_F32)
    assert np.array_equal(_u32(run), _u32(amax))
    ks, vs, _ = w.scales()
    assert int(bits[0]) == _f32_bits(ks) and int(bits[1]) == _f32_bits(vs)


def test_calibrate_full_varlen_bf16_per_sequence():
    """The variable-length workload's 256 sequences (512..32768 tokens), one
    running call per sequence with bf16 scales out, against the oracle's amax
    over each sequence's bits."""
    w = Workload("varlen", device=torch.device(DEV))
    row = w.Hkv * w.D
    run = torch.zeros(2, dtype=torch.float32, device=DEV)
    wk = wv = np.float32(0.0)
    out = torch.zeros(2, dtype=torch.int16, device=DEV)
    for b in range(w.B):
        L = int(w.lengths[b])
        k, v = w.kv(b, 0, L)
        kv.kv_calibrate_scales(k, v, row, row, L, row, run, out, kv.DTYPE_BF16)
        wk = oracle.amax(bf16_bits(k).reshape(L, row), start=wk)
        wv = oracle.amax(bf16_bits(v).reshape(L, row), start=wv)
    torch.cuda.synchronize()
    bits = out.cpu().numpy().view(np.uint16).astype(np.uint32)
    _check(run, bits, wk, wv, kv.DTYPE_BF16)
    ks, vs, dt = w.scales()
    assert dt == "bf16"
    assert int(bits[0]) << 16 == _f32_bits(ks) and int(bits[1]) << 16 == _f32_bits(vs)
