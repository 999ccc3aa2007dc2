"""kvfp8 CPU oracle -- TEST INFRASTRUCTURE ONLY.

Thin ctypes/numpy wrapper around ``kvfp8_oracle.c``, a plain scalar C
implementation of the FP8-E4M3 scaled paged KV cache (codec, store, paged
decode and chunked-prefill attention in fp64, K-shift, block bytes).

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
CPU-baseline leg may import this package.  The HIP library never imports,
links or calls it, and the two share no code.

Parity status of each function (what pins it is in ``tests/test_oracle_*``):
  e4m3_decode / e4m3_encode   pinned (256-code closed form, brute-force nearest
                              value, pages' printed constants, NumPy codec)
  store                       pinned (rounding envelope, power-of-two scale
                              invariance, layout bijection and round trip)
  decode_attn / prefill_attn  pinned (fp64 SDPA on the dequantized values,
                              one-key and identical-key special cases)
  kshift                      pinned (complex rotation in NumPy, delta 0,
                              angle pins)
  kshift_per_slot             pinned (one delta everywhere = kshift; each slot
                              = kshift of that slot alone; NumPy complex
                              rotation per slot)
  kv_bytes_per_block          pinned (exact halving)
  amax / calibrate_scales     pinned (torch's abs-max, planted maxima and NaN,
                              power-of-two amax, fp64-then-fp32 division,
                              torch's bf16 rounding, the calibrated maximum
                              encodes to the top finite E4M3 code)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvfp8_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (no fast-math, no FP contraction)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    os.makedirs(_BUILD_DIR, exist_ok=True)
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
           "-Wall", "-Wextra", "-Werror", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f32, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double
    sig = {
        "orc_bf16_bits_to_f32": (f32, [ctypes.c_uint16]),
        "orc_e4m3_decode": (f32, [ctypes.c_uint8]),
        "orc_e4m3_encode": (ctypes.c_uint8, [f32]),
        "orc_e4m3_decode_n": (None, [P, P, i64]),
        "orc_e4m3_encode_n": (None, [P, P, i64]),
        "orc_scale_ok": (ctypes.c_int, [f32]),
        "orc_scale_inverse": (f32, [f32]),
        "orc_k_tile_offset": (i64, [ctypes.c_int] * 4),
        "orc_v_tile_offset": (i64, [ctypes.c_int] * 4),
        "orc_store": (None, [P, P, i64, i64, P, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                             i64, f32, f32, P, P]),
        "orc_gather_dequant": (None, [P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P,
                                      ctypes.c_int, ctypes.c_int, f32, f32, P, P]),
        "orc_decode_attn": (ctypes.c_int, [P, ctypes.c_int, P, P, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, P, ctypes.c_int, P, ctypes.c_int,
                                           f32, f32, f64, P, i64, P]),
        "orc_store_typed": (None, [P, P, i64, i64, P, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   i64, ctypes.c_int, ctypes.c_int, f32, f32, P, P]),
        "orc_gather_typed": (None, [P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, P, ctypes.c_int, ctypes.c_int, f32, f32, P, P]),
        "orc_decode_attn_typed": (ctypes.c_int, [P, ctypes.c_int, P, P, ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_int, ctypes.c_int, ctypes.c_int, P, ctypes.c_int,
                                                 P, ctypes.c_int, f32, f32, f64, P, i64, P]),
        "orc_prefill_attn": (ctypes.c_int, [P, ctypes.c_int, P, P, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, P, P, P, ctypes.c_int, ctypes.c_int,
                                            f32, f32, f64, P, i64, P]),
        "orc_prefill_attn_typed": (ctypes.c_int, [P, ctypes.c_int, P, P, ctypes.c_int, ctypes.c_int,
                                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P, ctypes.c_int,
                                                  ctypes.c_int, f32, f32, f64, P, i64, P]),
        "orc_rope_table": (None, [ctypes.c_int, ctypes.c_int, f32, P, P]),
        "orc_kshift": (ctypes.c_int, [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, i64, P, i64,
                                      ctypes.c_int, f32, ctypes.c_int, ctypes.c_int]),
        "orc_kv_bytes_per_block": (i64, [ctypes.c_int] * 4),
        "orc_kshift_typed": (ctypes.c_int, [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, i64, P,
                                            i64, ctypes.c_int, f32, ctypes.c_int, ctypes.c_int]),
        "orc_kshift_per_slot_typed": (ctypes.c_int, [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                     i64, P, P, i64, f32, ctypes.c_int, ctypes.c_int]),
        "orc_kshift_per_slot": (ctypes.c_int, [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, i64, P, P, i64,
                                               f32, ctypes.c_int, ctypes.c_int]),
        "orc_amax_bf16": (f32, [P, i64, i64, i64, f32]),
        "orc_scale_from_amax": (f32, [f32]),
        "orc_f32_to_bf16_rne": (ctypes.c_uint16, [f32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


# ---------------------------------------------------------------- codec
def e4m3_decode(codes) -> np.ndarray:
    """Decode E4M3 codes (any shape, uint8) to fp32."""
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float32)
    _load().orc_e4m3_decode_n(_ptr(c), _ptr(out), c.size)
    return out


def e4m3_encode(x) -> np.ndarray:
    """Encode fp32 values to saturating round-half-even E4M3 codes."""
    a = _c(x, np.float32)
    out = np.empty(a.shape, np.uint8)
    _load().orc_e4m3_encode_n(_ptr(a), _ptr(out), a.size)
    return out


def bf16_to_f32(bits) -> np.ndarray:
    b = _c(bits, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def scale_ok(s: float) -> bool:
    return bool(_load().orc_scale_ok(float(np.float32(s))))


def scale_inverse(s: float) -> np.float32:
    return np.float32(_load().orc_scale_inverse(float(np.float32(s))))


# ---------------------------------------------------------------- calibration
def amax(bits, row_elems: int | None = None, start: float = 0.0) -> np.float32:
    """Running amax of bf16 bits: 2-D [rows][stride] (only the first row_elems
    of each row count) or any shape (all elements count), from `start`."""
    b = np.asarray(bits, np.uint16)
    if b.ndim != 2:
        b = b.reshape(1, -1) if b.size else b.reshape(0, 1)
    b = np.ascontiguousarray(b)
    rows, stride = b.shape
    n = stride if row_elems is None else int(row_elems)
    assert 0 <= n <= stride
    return np.float32(_load().orc_amax_bf16(_ptr(b), rows, n, stride, float(np.float32(start))))


def scale_from_amax(a: float) -> np.float32:
    """fp32 scale amax / 448."""
    return np.float32(_load().orc_scale_from_amax(float(np.float32(a))))


def f32_to_bf16(x) -> np.ndarray:
    """Nearest-even bf16 bits of fp32 values (any shape)."""
    a = np.asarray(x, np.float32)
    f = _load().orc_f32_to_bf16_rne
    return np.array([f(float(v)) for v in a.reshape(-1)], np.uint16).reshape(a.shape)


def calibrate_scales(k_amax: float, v_amax: float, scale_dtype: str = "f32"):
    """(k, v) scales as fp32 values and as the bits of scale_dtype ("f32" ->
    uint32 fp32 bits, NaN as 0x7FC00000; "bf16" -> uint16 bf16 bits)."""
    out_v, out_b = [], []
    for a in (k_amax, v_amax):
        s = scale_from_amax(a)
        if scale_dtype == "bf16":
            b = np.uint16(f32_to_bf16(s))
            v = np.array([np.uint32(b) << np.uint32(16)], np.uint32).view(np.float32)[0]
        else:
            b = np.uint32(0x7FC00000) if np.isnan(s) else np.array([s], np.float32).view(np.uint32)[0]
            v = s
        out_v.append(np.float32(v))
        out_b.append(b)
    return tuple(out_v), tuple(out_b)


# ---------------------------------------------------------------- layout
def k_tile_offset(t: int, d: int, BS: int, D: int) -> int:
    return int(_load().orc_k_tile_offset(t, d, BS, D))


def v_tile_offset(t: int, d: int, BS: int, D: int) -> int:
    return int(_load().orc_v_tile_offset(t, d, BS, D))


def kv_bytes_per_block(BS: int, Hkv: int, D: int, elem_bytes: int) -> int:
    return int(_load().orc_kv_bytes_per_block(BS, Hkv, D, elem_bytes))


# ---------------------------------------------------------------- store
def _elem_bytes(pool) -> int:
    """Element bytes of an oracle pool: uint8 holds E4M3 codes, uint16 bf16 values."""
    assert pool.dtype in (np.uint8, np.uint16) and pool.flags.c_contiguous
    return pool.dtype.itemsize


def store(k_bits, v_bits, slots, k_pool, v_pool, *, Hkv: int, D: int, BS: int,
          k_scale: float, v_scale: float) -> None:
    """Store bf16 K/V rows [T][Hkv][D] into the pools in place.

    k_pool / v_pool: [NB][Hkv][BS*D] arrays, uint8 for an E4M3 pool (values
    quantized) or uint16 for a bf16 pool (the bf16 bits as given; its scale
    must be 1).  Slots that are negative or at or past NB*BS are skipped."""
    k = _c(k_bits, np.uint16).reshape(-1, Hkv * D)
    v = _c(v_bits, np.uint16).reshape(-1, Hkv * D)
    s = _c(slots, np.int64)
    assert k.shape[0] == v.shape[0] == s.shape[0]
    keb, veb = _elem_bytes(k_pool), _elem_bytes(v_pool)
    assert k_pool.size == v_pool.size and k_pool.size % (Hkv * BS * D) == 0
    NB = k_pool.size // (Hkv * BS * D)
    _load().orc_store_typed(_ptr(k), _ptr(v), Hkv * D, Hkv * D, _ptr(s), s.size, Hkv, D, BS, NB, keb, veb,
                            float(np.float32(k_scale)), float(np.float32(v_scale)),
                            _ptr(k_pool), _ptr(v_pool))


def gather_dequant(k_pool, v_pool, table, L: int, h: int, *, Hkv: int, D: int, BS: int,
                   k_scale: float, v_scale: float):
    """Dequantized fp32 K and V rows [L][D] of one sequence / kv-head (uint8 pools
    hold E4M3 codes, uint16 pools bf16 values)."""
    t = _c(table, np.int32)
    kd = np.empty((L, D), np.float32)
    vd = np.empty((L, D), np.float32)
    _load().orc_gather_typed(_ptr(k_pool), _ptr(v_pool), Hkv, D, BS, _elem_bytes(k_pool), _elem_bytes(v_pool),
                             _ptr(t), L, h, float(np.float32(k_scale)), float(np.float32(v_scale)),
                             _ptr(kd), _ptr(vd))
    return kd, vd


# ---------------------------------------------------------------- attention
def decode_attn(q_bits, k_pool, v_pool, block_tables, seq_lens, *, Hq: int, Hkv: int, D: int,
                BS: int, k_scale: float, v_scale: float, sm_scale: float, sel=None) -> np.ndarray:
    """fp64 paged decode attention. q_bits [B][Hq][D] bf16 bits -> out [B][Hq][D] fp64.

    k_pool / v_pool: uint8 (E4M3 codes) or uint16 (bf16 values) arrays.
    sel: optional int array [n][2] of (b, h) pairs; other outputs are NaN."""
    q = _c(q_bits, np.uint16)
    B = q.shape[0]
    bt = _c(block_tables, np.int32)
    sl = _c(seq_lens, np.int32)
    out = np.full((B, Hq, D), np.nan, np.float64)
    if sel is not None:
        s = _c(sel, np.int32).reshape(-1, 2)
        sp, n = _ptr(s), s.shape[0]
    else:
        s, sp, n = None, None, 0
    rc = _load().orc_decode_attn_typed(_ptr(q), Hq, _ptr(k_pool), _ptr(v_pool), Hkv, D, BS,
                                       _elem_bytes(k_pool), _elem_bytes(v_pool), _ptr(bt),
                                       bt.shape[1], _ptr(sl), B, float(np.float32(k_scale)),
                                       float(np.float32(v_scale)), float(sm_scale), sp, n, _ptr(out))
    if rc != 0:
        raise MemoryError("oracle scratch allocation failed")
    return out


def prefill_attn(q_bits, k_pool, v_pool, cu_q_lens, context_lens, block_tables, *, Hq: int,
                 Hkv: int, D: int, BS: int, k_scale: float, v_scale: float, sm_scale: float,
                 sel=None) -> np.ndarray:
    """fp64 causal chunked-prefill attention over the cache. q [total_q][Hq][D] -> fp64.

    sel: optional int array [n][2] of (global query index, head) pairs.  Pools
    as in decode_attn: uint8 holds E4M3 codes, uint16 bf16 values."""
    q = _c(q_bits, np.uint16)
    cu = _c(cu_q_lens, np.int32)
    cl = _c(context_lens, np.int32)
    bt = _c(block_tables, np.int32)
    B = cl.shape[0]
    out = np.full((q.shape[0], Hq, D), np.nan, np.float64)
    if sel is not None:
        s = _c(sel, np.int64).reshape(-1, 2)
        sp, n = _ptr(s), s.shape[0]
    else:
        s, sp, n = None, None, 0
    rc = _load().orc_prefill_attn_typed(_ptr(q), Hq, _ptr(k_pool), _ptr(v_pool), Hkv, D, BS,
                                        _elem_bytes(k_pool), _elem_bytes(v_pool), _ptr(cu), _ptr(cl), _ptr(bt),
                                        bt.shape[1], B, float(np.float32(k_scale)), float(np.float32(v_scale)),
                                        float(sm_scale), sp, n, _ptr(out))
    if rc != 0:
        raise MemoryError("oracle scratch allocation failed")
    return out


# ---------------------------------------------------------------- K-shift
def rope_table(rot_dim: int, delta: int, theta: float):
    c = np.empty(rot_dim // 2, np.float32)
    s = np.empty(rot_dim // 2, np.float32)
    _load().orc_rope_table(rot_dim, delta, float(np.float32(theta)), _ptr(c), _ptr(s))
    return c, s


def kshift(k_pool, slots, *, Hkv: int, D: int, BS: int, delta: int, theta: float, rot_dim: int,
           neox: bool) -> None:
    """Re-rotate cached K by a RoPE position delta, in place (scale-free).  Slots
    that are negative or at or past the pool's NB*BS slots are skipped.  A
    uint8 pool holds E4M3 codes, a uint16 pool bf16 values."""
    s = _c(slots, np.int64)
    eb = _elem_bytes(k_pool)
    assert k_pool.size % (Hkv * BS * D) == 0
    NB = k_pool.size // (Hkv * BS * D)
    rc = _load().orc_kshift_typed(_ptr(k_pool), eb, Hkv, D, BS, NB, _ptr(s), s.size, int(delta),
                                  float(np.float32(theta)), rot_dim, 1 if neox else 0)
    if rc != 0:
        raise MemoryError("oracle scratch allocation failed")


def kshift_per_slot(k_pool, slots, deltas, *, Hkv: int, D: int, BS: int, theta: float, rot_dim: int,
                    neox: bool) -> None:
    """kshift with its own position delta per slot (deltas[i] for slots[i]), in place."""
    s = _c(slots, np.int64)
    dl = _c(deltas, np.int32)
    assert s.shape == dl.shape
    eb = _elem_bytes(k_pool)
    assert k_pool.size % (Hkv * BS * D) == 0
    NB = k_pool.size // (Hkv * BS * D)
    rc = _load().orc_kshift_per_slot_typed(_ptr(k_pool), eb, Hkv, D, BS, NB, _ptr(s), _ptr(dl), s.size,
                                           float(np.float32(theta)), rot_dim, 1 if neox else 0)
    if rc != 0:
        raise MemoryError("oracle scratch allocation failed")
