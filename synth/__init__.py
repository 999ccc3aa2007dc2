"""Seeded synthetic workloads for the FP8-E4M3 paged KV cache.

This module only draws inputs: bf16 K/V/Q values, lengths, block tables,
slot mappings and per-tensor scales.  It holds none of the cache's own
arithmetic (no quantization, no attention), so both the HIP library's
tests and the CPU oracle can be fed from it.

Values are fp32 N(0, 1) draws rounded to bf16 by torch.  Every (sequence,
4096-token chunk, tensor) has its own seed, so any token range can be
regenerated on its own, on CPU or on the GPU, without drawing the rest.

The five workloads (sizes as named):
  tiny      1 layer, 4 q / 2 kv heads, head_dim 64, block 16, lengths
            {17, 40, 73, 100}; k_scale 0.02, v_scale 0.015 (fp32)
  llama8b   32 q / 8 kv heads, head_dim 128, block 16, 64 sequences x 4096
            tokens, 4 outlier channels x20 in K and in V, per-tensor fp32
            scales amax/448, block table a random permutation of 16384 blocks
  varlen    same heads, 256 sequences with lengths uniform in [512, 32768],
            block tables drawn from a shuffled free list over a pool that is a
            fraction of 288 GB, bf16 scales bf16(amax/448); one new token each
  prefill   32 q / 8 kv heads, head_dim 128, block 16, 4 sequences with 16384
            cached tokens plus a 2048-token chunk; fp32 scales amax/448 of the
            cached (fill) tokens
  longctx   16 q / 2 kv heads, head_dim 256, block 32, 8 sequences x 131072
            tokens, scales 0.03 (fp32); RoPE shift delta -4096, theta 1e6
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

CHUNK = 4096          # tokens per independently seeded chunk
HBM_BYTES = 288e9     # MI355X HBM capacity used to size the varlen pool


@dataclasses.dataclass
class Spec:
    name: str
    Hq: int
    Hkv: int
    D: int
    BS: int
    lengths: list            # cached tokens per sequence before the step
    seed: int
    k_scale: float | None = None   # fixed scales; None -> amax/448
    v_scale: float | None = None
    scale_dtype: str = "f32"       # "f32" or "bf16"
    outliers: int = 0
    outlier_mult: float = 20.0
    new_tokens: int = 0            # tokens appended per sequence in the step (decode store / chunk)
    pool_blocks: int | None = None  # None -> exactly the blocks needed
    permute_all: bool = False      # block table = permutation of the whole pool
    delta: int = 0
    theta: float = 1e6


def _spec(name: str, scale_down: int = 1, pool_frac: float = 0.5) -> Spec:
    """Workload spec by name; scale_down divides sequence counts/lengths for quick runs."""
    sd = max(1, int(scale_down))
    if name == "tiny":
        return Spec("tiny", 4, 2, 64, 16, [17, 40, 73, 100], 1001, 0.02, 0.015)
    if name == "llama8b":
        B, L = max(1, 64 // sd), max(16, 4096 // sd)
        return Spec("llama8b", 32, 8, 128, 16, [L] * B, 1002, outliers=4, permute_all=True)
    if name == "varlen":
        B = max(2, 256 // sd)
        rng = np.random.default_rng(1003)
        lo, hi = max(16, 512 // sd), max(32, 32768 // sd)
        lengths = rng.integers(lo, hi + 1, size=B).tolist()
        kv_bytes_per_block = 2 * 16 * 8 * 128
        nb = int(pool_frac * HBM_BYTES // kv_bytes_per_block)
        need = sum(-(-(L + 1) // 16) for L in lengths)
        return Spec("varlen", 32, 8, 128, 16, lengths, 1003, scale_dtype="bf16", new_tokens=1,
                    pool_blocks=max(nb, need))
    if name == "prefill":
        B, ctx, chunk = 4, max(16, 16384 // sd), max(16, 2048 // sd)
        return Spec("prefill", 32, 8, 128, 16, [ctx] * B, 1004, new_tokens=chunk)
    if name == "longctx":
        B, L = max(1, 8 // sd), max(32, 131072 // sd)
        return Spec("longctx", 16, 2, 256, 32, [L] * B, 1005, 0.03, 0.03, delta=-4096, theta=1e6)
    raise KeyError(name)


NAMES = ["tiny", "llama8b", "varlen", "prefill", "longctx"]


def _seed(*parts) -> int:
    h = 0x9E3779B97F4A7C15
    for p in parts:
        h = (h ^ (int(p) & 0xFFFFFFFFFFFFFFFF)) * 0xBF58476D1CE4E5B9 & 0xFFFFFFFFFFFFFFFF
        h ^= h >> 31
    return h & 0x7FFFFFFFFFFFFFFF


def _randn(shape, seed: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bf16 bit patterns of a bf16 tensor as a host uint16 array."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32_to_bf16_bits(x: float) -> int:
    """Round an fp32 value to bf16 (round to nearest even, as torch does)."""
    return int(bf16_bits(torch.tensor([x], dtype=torch.float32).to(torch.bfloat16))[0])


class Workload:
    """One seeded workload: shapes, tables, per-token K/V draws and scales."""

    def __init__(self, name: str, device="cpu", scale_down: int = 1, pool_frac: float = 0.5,
                 spec: Spec | None = None):
        self.spec = spec if spec is not None else _spec(name, scale_down, pool_frac)
        s = self.spec
        self.device = torch.device(device)
        self.name, self.Hq, self.Hkv, self.D, self.BS = s.name, s.Hq, s.Hkv, s.D, s.BS
        self.B = len(s.lengths)
        self.lengths = np.asarray(s.lengths, np.int64)
        self.total_lengths = self.lengths + s.new_tokens
        rng = np.random.default_rng(_seed(s.seed, 77))
        if s.outliers:
            self.k_outliers = rng.choice(s.Hkv * s.D, s.outliers, replace=False)
            self.v_outliers = rng.choice(s.Hkv * s.D, s.outliers, replace=False)
        else:
            self.k_outliers = self.v_outliers = np.zeros(0, np.int64)
        self._build_tables(rng)
        self._scales = None

    # ------------------------------------------------------------ paging
    def _build_tables(self, rng):
        s = self.spec
        nblk = [-(-int(L) // s.BS) for L in self.total_lengths]
        need = sum(nblk)
        if s.permute_all:
            self.NB = need if s.pool_blocks is None else s.pool_blocks
            order = rng.permutation(self.NB)
        else:
            self.NB = max(need, s.pool_blocks or 0)
            if self.NB > 4 * need:
                order = rng.choice(self.NB, size=need, replace=False)
            else:
                order = rng.permutation(self.NB)[:need]
        self.max_blocks = max(nblk)
        self.block_tables = np.zeros((self.B, self.max_blocks), np.int32)
        pos = 0
        for b, n in enumerate(nblk):
            self.block_tables[b, :n] = order[pos:pos + n]
            pos += n

    def slots(self, b: int, start: int, count: int) -> np.ndarray:
        p = np.arange(start, start + count, dtype=np.int64)
        return self.block_tables[b, p // self.BS].astype(np.int64) * self.BS + p % self.BS

    # ------------------------------------------------------------ values
    def _chunk(self, kind: str, b: int, c: int, device) -> torch.Tensor:
        s = self.spec
        kid = {"k": 1, "v": 2}[kind]
        x = _randn((CHUNK, s.Hkv * s.D), _seed(s.seed, kid, b, c), device)
        idx = self.k_outliers if kind == "k" else self.v_outliers
        if len(idx):
            x[:, torch.as_tensor(idx, device=device)] *= s.outlier_mult
        return x.to(torch.bfloat16).view(CHUNK, s.Hkv, s.D)

    def kv(self, b: int, start: int, count: int, device=None):
        """bf16 K and V of sequence b at positions start..start+count-1, [count][Hkv][D]."""
        device = self.device if device is None else torch.device(device)
        ks, vs = [], []
        c0, c1 = start // CHUNK, (start + count - 1) // CHUNK if count else start // CHUNK - 1
        for c in range(c0, c1 + 1):
            lo = max(start, c * CHUNK) - c * CHUNK
            hi = min(start + count, (c + 1) * CHUNK) - c * CHUNK
            ks.append(self._chunk("k", b, c, device)[lo:hi])
            vs.append(self._chunk("v", b, c, device)[lo:hi])
        if not ks:
            z = torch.zeros((0, self.Hkv, self.D), dtype=torch.bfloat16, device=device)
            return z, z.clone()
        return torch.cat(ks), torch.cat(vs)

    def q_decode(self, device=None) -> torch.Tensor:
        device = self.device if device is None else torch.device(device)
        return _randn((self.B, self.Hq, self.D), _seed(self.spec.seed, 3), device).to(torch.bfloat16)

    def q_chunk(self, device=None) -> torch.Tensor:
        """Queries of the new-token chunk of every sequence, [sum new_tokens][Hq][D]."""
        device = self.device if device is None else torch.device(device)
        n = self.spec.new_tokens
        qs = [_randn((n, self.Hq, self.D), _seed(self.spec.seed, 4, b), device) for b in range(self.B)]
        return torch.cat(qs).to(torch.bfloat16)

    # ------------------------------------------------------------ scales
    def scales(self):
        """(k_scale, v_scale) as fp32 numbers, and the dtype name they are given in.

        Fixed scales are used as given.  Otherwise s = fl32(amax / 448) over the
        cached (fill) tokens of all sequences, rounded to bf16 for bf16 scales."""
        if self._scales is not None:
            return self._scales
        s = self.spec
        if s.k_scale is not None:
            ks, vs = np.float32(s.k_scale), np.float32(s.v_scale)
        else:
            ka = va = 0.0
            for b in range(self.B):
                L = int(self.lengths[b])
                for c in range(0, -(-L // CHUNK)):
                    n = min(CHUNK, L - c * CHUNK)
                    k = self._chunk("k", b, c, self.device)[:n]
                    v = self._chunk("v", b, c, self.device)[:n]
                    ka = max(ka, float(k.float().abs().max()))
                    va = max(va, float(v.float().abs().max()))
            ks = np.float32(ka) / np.float32(448.0)
            vs = np.float32(va) / np.float32(448.0)
        if s.scale_dtype == "bf16":
            kb, vb = f32_to_bf16_bits(float(ks)), f32_to_bf16_bits(float(vs))
            ks = np.array([kb << 16], np.uint32).view(np.float32)[0]
            vs = np.array([vb << 16], np.uint32).view(np.float32)[0]
        self._scales = (np.float32(ks), np.float32(vs), s.scale_dtype)
        return self._scales

    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.D)
