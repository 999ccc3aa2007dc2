"""Python binding of the kvfp8 C ABI (include/kvfp8.h).

Argument marshalling only: every function here has the name of the C entry
point it calls, converts its arguments (torch tensors become device
pointers, torch streams become hipStream_t handles) and raises on a non-OK
status.  All computation happens in the HIP library libkvfp8.so, which is
built in-tree by ``python -m fp8_e4m3_scaled_amd.build``; importing this
package without it fails loudly.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvfp8.so")

OK, E_INVALID, E_SCALE, E_NOMEM, E_NOBLOCKS, E_UNSUPPORTED, E_HIP = range(7)
STATUS_NAMES = {0: "KVF8_OK", 1: "KVF8_E_INVALID", 2: "KVF8_E_SCALE", 3: "KVF8_E_NOMEM",
                4: "KVF8_E_NOBLOCKS", 5: "KVF8_E_UNSUPPORTED", 6: "KVF8_E_HIP"}
DTYPE_F32, DTYPE_BF16 = 0, 1
ROPE_NORM, ROPE_NEOX = 0, 1
ELEM_E4M3, ELEM_BF16 = 0, 1

# (restype, argtypes) of every exported function, in header order
P, I32, I64, U64, F32, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                             ctypes.c_float, ctypes.c_size_t)
SIGNATURES = {
    "kvf8_version": (ctypes.c_char_p, []),
    "kvf8_last_error": (ctypes.c_char_p, []),
    "kv_bytes_per_block": (SZ, [I32, I32, I32, I32]),
    "kv_cache_alloc": (I32, [I32, I64, I32, I32, I32, P, P, I32, P, P, ctypes.POINTER(P)]),
    "kv_cache_alloc_typed": (I32, [I32, I64, I32, I32, I32, I32, I32, P, P, I32, P, P, ctypes.POINTER(P)]),
    "kv_cache_elem_types": (I32, [P, P, P]),
    "kv_cache_free": (I32, [P]),
    "kv_cache_set_checked": (I32, [P, I32]),
    "kv_cache_set_scales": (I32, [P, I32, P, P, I32]),
    "kv_cache_get_scales": (I32, [P, I32, P, P]),
    "kv_cache_pools": (I32, [P, I32, P, P, P]),
    "kv_block_alloc": (I32, [P, I32, P]),
    "kv_block_free": (I32, [P, P, I32]),
    "kv_blocks_free": (I64, [P]),
    "kv_block_shuffle": (I32, [P, U64]),
    "kv_store_fp8": (I32, [P, I32, P, P, I64, I64, P, I64, P]),
    "paged_attn_decode_workspace": (SZ, [P, I32, I32, I32]),
    "paged_attn_decode": (I32, [P, I32, P, I32, P, I32, P, I32, I32, F32, P, I32, P, SZ, P]),
    "paged_attn_decode_noalloc": (I32, [P, I32, P, I32, P, I32, P, I32, I32, F32, P, I32, P]),
    "paged_attn_prefill_chunk": (I32, [P, I32, P, I32, P, P, P, I32, I32, I64, I32, I32, F32, P,
                                       I32, P]),
    "kv_shift_rope": (I32, [P, I32, P, I64, I32, F32, I32, I32, P]),
    "kv_rope_table": (I32, [P, I32, F32, I32, P]),
    "kv_shift_rope_per_slot": (I32, [P, I32, P, P, I64, P, I32, I32, I32, P]),
    "kv_calibrate_scales": (I32, [P, P, I64, I64, I64, I64, P, P, I32, P]),
}


class KvF8Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def _load_library():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m fp8_e4m3_scaled_amd.build`")
    # torch ships its own HIP runtime under the same soname as the system one.
    # Loading torch first makes the library bind to that copy, so the process
    # holds one HIP runtime; a second runtime would find the device already
    # claimed by the first and report that no device exists.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load_library()


def _check(status: int) -> None:
    if status != OK:
        raise KvF8Error(status, _lib.kvf8_last_error().decode())


def _ptr(x):
    """Device/host pointer of a torch tensor, a ctypes buffer, an int or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, ctypes.Array):
        return ctypes.addressof(x)
    return ctypes.cast(x, ctypes.c_void_p).value


def _stream(s):
    """hipStream_t of a torch stream (None -> torch's current stream)."""
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def kvf8_version() -> str:
    return _lib.kvf8_version().decode()


def kvf8_last_error() -> str:
    return _lib.kvf8_last_error().decode()


def kv_bytes_per_block(block_size: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    return int(_lib.kv_bytes_per_block(block_size, num_kv_heads, head_dim, elem_bytes))


def _scale_buffer(scales, dtype: int):
    if scales is None:
        return None
    vals = list(scales)
    if dtype == DTYPE_F32:
        return (ctypes.c_float * len(vals))(*[float(v) for v in vals])
    return (ctypes.c_uint16 * len(vals))(*[int(v) for v in vals])


def kv_cache_alloc(num_layers: int, num_blocks: int, block_size: int, num_kv_heads: int,
                   head_dim: int, k_scales=None, v_scales=None, scale_dtype: int = DTYPE_F32,
                   k_pool=None, v_pool=None) -> int:
    """Returns the cache handle (an opaque address).  Scales: host sequences of fp32
    values (DTYPE_F32) or bf16 bit patterns (DTYPE_BF16), one per layer."""
    out = ctypes.c_void_p()
    kb, vb = _scale_buffer(k_scales, scale_dtype), _scale_buffer(v_scales, scale_dtype)
    _check(_lib.kv_cache_alloc(num_layers, num_blocks, block_size, num_kv_heads, head_dim,
                               _ptr(kb), _ptr(vb), scale_dtype, _ptr(k_pool), _ptr(v_pool),
                               ctypes.byref(out)))
    return out.value


def kv_cache_alloc_typed(num_layers: int, num_blocks: int, block_size: int, num_kv_heads: int,
                         head_dim: int, k_elem: int, v_elem: int, k_scales=None, v_scales=None,
                         scale_dtype: int = DTYPE_F32, k_pool=None, v_pool=None) -> int:
    """kv_cache_alloc with an element type per pool (ELEM_E4M3 or ELEM_BF16)."""
    out = ctypes.c_void_p()
    kb, vb = _scale_buffer(k_scales, scale_dtype), _scale_buffer(v_scales, scale_dtype)
    _check(_lib.kv_cache_alloc_typed(num_layers, num_blocks, block_size, num_kv_heads, head_dim, k_elem,
                                     v_elem, _ptr(kb), _ptr(vb), scale_dtype, _ptr(k_pool), _ptr(v_pool),
                                     ctypes.byref(out)))
    return out.value


def kv_cache_elem_types(cache):
    """(k_elem, v_elem) of a cache."""
    k, v = ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.kv_cache_elem_types(cache, ctypes.byref(k), ctypes.byref(v)))
    return k.value, v.value


def kv_cache_free(cache) -> None:
    _check(_lib.kv_cache_free(cache))


def kv_cache_set_checked(cache, on: bool) -> None:
    _check(_lib.kv_cache_set_checked(cache, 1 if on else 0))


def kv_cache_set_scales(cache, layer: int, k_scale=None, v_scale=None,
                        scale_dtype: int = DTYPE_F32) -> None:
    kb = None if k_scale is None else _scale_buffer([k_scale], scale_dtype)
    vb = None if v_scale is None else _scale_buffer([v_scale], scale_dtype)
    _check(_lib.kv_cache_set_scales(cache, layer, _ptr(kb), _ptr(vb), scale_dtype))


def kv_cache_get_scales(cache, layer: int):
    k, v = ctypes.c_float(), ctypes.c_float()
    _check(_lib.kv_cache_get_scales(cache, layer, ctypes.byref(k), ctypes.byref(v)))
    return k.value, v.value


def kv_cache_pools(cache, layer: int):
    """(k_pool address, v_pool address, bytes of each)."""
    k, v, n = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_size_t()
    _check(_lib.kv_cache_pools(cache, layer, ctypes.byref(k), ctypes.byref(v), ctypes.byref(n)))
    return k.value, v.value, n.value


def kv_block_alloc(cache, n: int) -> list:
    ids = (ctypes.c_int32 * max(1, n))()
    _check(_lib.kv_block_alloc(cache, n, ids))
    return list(ids[:n])


def kv_block_free(cache, ids) -> None:
    ids = list(ids)
    buf = (ctypes.c_int32 * max(1, len(ids)))(*ids)
    _check(_lib.kv_block_free(cache, buf, len(ids)))


def kv_blocks_free(cache) -> int:
    return int(_lib.kv_blocks_free(cache))


def kv_block_shuffle(cache, seed: int) -> None:
    _check(_lib.kv_block_shuffle(cache, seed))


def kv_store_fp8(cache, layer: int, k_bf16, v_bf16, k_tok_stride: int, v_tok_stride: int,
                 slot_mapping, num_tokens: int, stream=None) -> None:
    _check(_lib.kv_store_fp8(cache, layer, _ptr(k_bf16), _ptr(v_bf16), k_tok_stride, v_tok_stride,
                             _ptr(slot_mapping), num_tokens, _stream(stream)))


def paged_attn_decode_workspace(cache, num_seqs: int, num_q_heads: int, max_seq_len: int) -> int:
    return int(_lib.paged_attn_decode_workspace(cache, num_seqs, num_q_heads, max_seq_len))


def paged_attn_decode(cache, layer: int, q_bf16, num_q_heads: int, block_tables,
                      max_blocks_per_seq: int, seq_lens, num_seqs: int, max_seq_len: int,
                      sm_scale: float, out, out_dtype: int, workspace=None,
                      workspace_bytes: int = 0, stream=None) -> None:
    _check(_lib.paged_attn_decode(cache, layer, _ptr(q_bf16), num_q_heads, _ptr(block_tables),
                                  max_blocks_per_seq, _ptr(seq_lens), num_seqs, max_seq_len,
                                  sm_scale, _ptr(out), out_dtype, _ptr(workspace), workspace_bytes,
                                  _stream(stream)))


def paged_attn_decode_noalloc(cache, layer: int, q_bf16, num_q_heads: int, block_tables,
                              max_blocks_per_seq: int, seq_lens, num_seqs: int, max_seq_len: int,
                              sm_scale: float, out, out_dtype: int, stream=None) -> None:
    _check(_lib.paged_attn_decode_noalloc(cache, layer, _ptr(q_bf16), num_q_heads, _ptr(block_tables),
                                          max_blocks_per_seq, _ptr(seq_lens), num_seqs, max_seq_len,
                                          sm_scale, _ptr(out), out_dtype, _stream(stream)))


def paged_attn_prefill_chunk(cache, layer: int, q_bf16, num_q_heads: int, cu_q_lens,
                             context_lens, block_tables, max_blocks_per_seq: int, num_seqs: int,
                             total_q: int, max_q_len: int, max_ctx_len: int, sm_scale: float, out,
                             out_dtype: int, stream=None) -> None:
    _check(_lib.paged_attn_prefill_chunk(cache, layer, _ptr(q_bf16), num_q_heads, _ptr(cu_q_lens),
                                         _ptr(context_lens), _ptr(block_tables), max_blocks_per_seq,
                                         num_seqs, total_q, max_q_len, max_ctx_len, sm_scale,
                                         _ptr(out), out_dtype, _stream(stream)))


def kv_shift_rope(cache, layer: int, slots, n_slots: int, delta: int, theta_base: float,
                  rot_dim: int, style: int, stream=None) -> None:
    _check(_lib.kv_shift_rope(cache, layer, _ptr(slots), n_slots, delta, theta_base, rot_dim, style,
                              _stream(stream)))


def kv_rope_table(deltas, theta_base: float, rot_dim: int):
    """Host cos/sin table [n_deltas][rot_dim/2][2] (numpy float32) for kv_shift_rope_per_slot."""
    import numpy as np
    d = np.ascontiguousarray(np.asarray(deltas, dtype=np.int32).reshape(-1))
    table = np.zeros((d.size, rot_dim // 2, 2), np.float32)
    _check(_lib.kv_rope_table(d.ctypes.data if d.size else None, d.size, theta_base, rot_dim,
                              table.ctypes.data if d.size else None))
    return table


def kv_shift_rope_per_slot(cache, layer: int, slots, table_rows, n_slots: int, table, n_rows: int,
                           rot_dim: int, style: int, stream=None) -> None:
    _check(_lib.kv_shift_rope_per_slot(cache, layer, _ptr(slots), _ptr(table_rows), n_slots, _ptr(table),
                                       n_rows, rot_dim, style, _stream(stream)))


def kv_calibrate_scales(k_bf16, v_bf16, k_tok_stride: int, v_tok_stride: int, num_tokens: int,
                        row_elems: int, amax, scales_out=None, scale_dtype: int = DTYPE_F32,
                        stream=None) -> None:
    _check(_lib.kv_calibrate_scales(_ptr(k_bf16), _ptr(v_bf16), k_tok_stride, v_tok_stride, num_tokens,
                                    row_elems, _ptr(amax), _ptr(scales_out), scale_dtype, _stream(stream)))

