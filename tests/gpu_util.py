"""Helpers for the GPU parity tests: device tensors as caller-owned memory and
a cache whose pools are torch tensors (so they can be copied out)."""
from __future__ import annotations

import numpy as np
import torch

import fp8_e4m3_scaled_amd as kv

DEV = "cuda:0"


def t_dev(a, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def bits_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> bf16 device tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


class GpuCache:
    """A one-layer (or n-layer) cache over torch-owned zeroed pools."""

    def __init__(self, NB, BS, Hkv, D, k_scale=1.0, v_scale=1.0, scale_dtype=kv.DTYPE_F32,
                 layers=1, fill=0):
        self.NB, self.BS, self.Hkv, self.D, self.layers = NB, BS, Hkv, D, layers
        shape = (layers, NB, Hkv, BS * D)
        self.k_pool = torch.full(shape, fill, dtype=torch.uint8, device=DEV)
        self.v_pool = torch.full(shape, fill, dtype=torch.uint8, device=DEV)
        ks = [k_scale] * layers if np.isscalar(k_scale) else list(k_scale)
        vs = [v_scale] * layers if np.isscalar(v_scale) else list(v_scale)
        self.handle = kv.kv_cache_alloc(layers, NB, BS, Hkv, D, ks, vs, scale_dtype,
                                        self.k_pool, self.v_pool)

    def pools(self, layer=0):
        torch.cuda.synchronize()
        return self.k_pool[layer].cpu().numpy(), self.v_pool[layer].cpu().numpy()

    def close(self):
        if self.handle:
            kv.kv_cache_free(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def log(msg: str) -> None:
    print(msg, flush=True)
