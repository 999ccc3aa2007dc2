"""Measurement aids of the benchmark (not part of the kvfp8 library): a plain
streaming read, a plain read of a paged decode's K/V tiles, and the K-shift's
and the cache fill's traffic with no arithmetic, built into
probe/libkvf8probe.so from readprobe.hip (declared in readprobe.h)."""
from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvf8probe.so")
SRC = os.path.join(HERE, "readprobe.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-fPIC", "-shared", "-std=c++17", "--offload-arch=gfx950", "-I", HERE, "-Wall", "-Wextra",
         "-Werror", "-Wno-unused-parameter", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build() -> str:
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe build failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


class ProbeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"probe status {status}: {message}")
        self.status = status


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with probe.build()")
        import torch  # noqa: F401  (one HIP runtime per process: bind to torch's copy)
        lib = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        lib.kvf8_probe_last_error.restype = ctypes.c_char_p
        lib.kvf8_probe_last_error.argtypes = []
        lib.kvf8_probe_read.restype = I32
        lib.kvf8_probe_read.argtypes = [P, SZ, P, I32, P]
        lib.kvf8_probe_gather.restype = I32
        lib.kvf8_probe_gather.argtypes = [P, P, I64, I32, I32, I32, I32, I32, P, I32, P, I32, P, P]
        lib.kvf8_probe_gather_split.restype = I32
        lib.kvf8_probe_gather_split.argtypes = [P, P, I64, I32, I32, I32, I32, I32, P, I32, P, I32, I32, P, P]
        lib.kvf8_probe_rmw.restype = I32
        lib.kvf8_probe_rmw.argtypes = [P, I64, I32, I32, I32, I32, P, I64, P]
        lib.kvf8_probe_store_copy.restype = I32
        lib.kvf8_probe_store_copy.argtypes = [P, P, I64, I64, P, I64, P, P, I64, I32, I32, I32, P]
        _lib = lib
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    """hipStream_t of a torch stream (None -> torch's current stream)."""
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(st):
    if st != 0:
        raise ProbeError(st, _load().kvf8_probe_last_error().decode())


def read(buf, nbytes: int, out_words, n_out: int, stream=None) -> None:
    _check(_load().kvf8_probe_read(_ptr(buf), nbytes, _ptr(out_words), n_out, _stream(stream)))


def gather(k_pool, v_pool, num_blocks: int, kv_heads: int, block_size: int, head_dim: int, k_elem_bytes: int,
           v_elem_bytes: int, block_tables, max_blocks: int, seq_lens, num_seqs: int, out_words,
           stream=None) -> None:
    _check(_load().kvf8_probe_gather(_ptr(k_pool), _ptr(v_pool), num_blocks, kv_heads, block_size, head_dim,
                                     k_elem_bytes, v_elem_bytes, _ptr(block_tables), max_blocks, _ptr(seq_lens),
                                     num_seqs, _ptr(out_words), _stream(stream)))


def rmw(k_pool, num_blocks: int, kv_heads: int, block_size: int, head_dim: int, rot_dim: int, slots,
        n_slots: int, stream=None) -> None:
    _check(_load().kvf8_probe_rmw(_ptr(k_pool), num_blocks, kv_heads, block_size, head_dim, rot_dim,
                                  _ptr(slots), n_slots, _stream(stream)))


def store_copy(k, v, k_stride: int, v_stride: int, slots, num_tokens: int, k_pool, v_pool, num_blocks: int,
               kv_heads: int, block_size: int, head_dim: int, stream=None) -> None:
    _check(_load().kvf8_probe_store_copy(_ptr(k), _ptr(v), k_stride, v_stride, _ptr(slots), num_tokens,
                                         _ptr(k_pool), _ptr(v_pool), num_blocks, kv_heads, block_size, head_dim,
                                         _stream(stream)))


def gather_split(k_pool, v_pool, num_blocks: int, kv_heads: int, block_size: int, head_dim: int,
                 k_elem_bytes: int, v_elem_bytes: int, block_tables, max_blocks: int, seq_lens, num_seqs: int,
                 chunk_blocks: int, out_words, stream=None) -> None:
    _check(_load().kvf8_probe_gather_split(_ptr(k_pool), _ptr(v_pool), num_blocks, kv_heads, block_size, head_dim,
                                           k_elem_bytes, v_elem_bytes, _ptr(block_tables), max_blocks,
                                           _ptr(seq_lens), num_seqs, chunk_blocks, _ptr(out_words),
                                           _stream(stream)))
