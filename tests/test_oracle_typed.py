"""Pins of the oracle's per-pool element types (E4M3 codes or bf16 values).

A bf16 pool holds the given bf16 values unchanged at the same element
positions as the E4M3 layout [P3, "What turning it on costs": the bf16 twin
of the fp8 cache; P1, tests/test-fp8.cpp: K and V cache types chosen
independently].  Pinned by:
* every stored element read back through the layout's offset functions equals
  the input bits, untouched elements stay zero, skipped slots write nothing;
* a mixed store (E4M3 K, bf16 V and the reverse) equals the single-type
  stores of each side;
* decode attention over every type combination equals torch's fp64
  scaled_dot_product_attention over values built without the oracle: bf16
  values straight from the inputs, E4M3 values through the independent NumPy
  codec.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import np_codec
from synth import Workload, bf16_bits

POOL = {1: np.uint8, 2: np.uint16}


def _pools(w, keb, veb):
    shape = (w.NB, w.Hkv, w.BS * w.D)
    return np.zeros(shape, POOL[keb]), np.zeros(shape, POOL[veb])


def _store_all(orc, w, kp, vp, ks, vs):
    for b in range(w.B):
        L = int(w.lengths[b])
        k, v = w.kv(b, 0, L)
        orc.store(bf16_bits(k), bf16_bits(v), w.slots(b, 0, L), kp, vp, Hkv=w.Hkv, D=w.D, BS=w.BS,
                  k_scale=ks, v_scale=vs)


def test_bf16_store_places_the_bits(orc):
    w = Workload("tiny")
    kp, vp = _pools(w, 2, 2)
    _store_all(orc, w, kp, vp, 1.0, 1.0)
    touched_k = np.zeros(kp.shape, bool)
    touched_v = np.zeros(vp.shape, bool)
    for b in range(w.B):
        L = int(w.lengths[b])
        k, v = w.kv(b, 0, L)
        kb, vb = bf16_bits(k), bf16_bits(v)
        for p in range(L):
            blk, t = int(w.block_tables[b, p // w.BS]), p % w.BS
            for h in range(w.Hkv):
                ko = [orc.k_tile_offset(t, d, w.BS, w.D) for d in range(w.D)]
                vo = [orc.v_tile_offset(t, d, w.BS, w.D) for d in range(w.D)]
                assert np.array_equal(kp[blk, h, ko], kb[p, h])
                assert np.array_equal(vp[blk, h, vo], vb[p, h])
                touched_k[blk, h, ko] = True
                touched_v[blk, h, vo] = True
    assert not kp[~touched_k].any() and not vp[~touched_v].any()
    # skipped slots write nothing
    kp2, vp2 = _pools(w, 2, 2)
    x = bf16_bits(torch.ones((3, w.Hkv, w.D), dtype=torch.bfloat16))
    orc.store(x, x, np.array([-1, w.NB * w.BS, -7]), kp2, vp2, Hkv=w.Hkv, D=w.D, BS=w.BS,
              k_scale=1.0, v_scale=1.0)
    assert not kp2.any() and not vp2.any()


@pytest.mark.parametrize("keb,veb", [(1, 2), (2, 1)])
def test_mixed_store_equals_single_type_stores(orc, keb, veb):
    w = Workload("tiny")
    ks, vs = 0.02, 0.015
    kp, vp = _pools(w, keb, veb)
    _store_all(orc, w, kp, vp, ks if keb == 1 else 1.0, vs if veb == 1 else 1.0)
    k8, v8 = _pools(w, 1, 1)
    _store_all(orc, w, k8, v8, ks, vs)
    k16, v16 = _pools(w, 2, 2)
    _store_all(orc, w, k16, v16, 1.0, 1.0)
    assert np.array_equal(kp, k8 if keb == 1 else k16)
    assert np.array_equal(vp, v8 if veb == 1 else v16)


def _values(x_bits, eb, scale):
    """fp32 values the cache holds for bf16 inputs: the inputs (bf16 pool) or the
    E4M3 round trip through the NumPy codec times the scale."""
    x = (x_bits.astype(np.uint32) << 16).view(np.float32)
    if eb == 2:
        return x
    inv = np.float32(1.0) / np.float32(scale)
    y = (x * inv).astype(np.float32)
    return (np_codec.decode(np_codec.encode(y)) * np.float32(scale)).astype(np.float32)


@pytest.mark.parametrize("keb,veb", [(1, 1), (1, 2), (2, 1), (2, 2)])
def test_typed_decode_matches_fp64_sdpa(orc, keb, veb):
    w = Workload("tiny")
    ks = 0.02 if keb == 1 else 1.0
    vs = 0.015 if veb == 1 else 1.0
    kp, vp = _pools(w, keb, veb)
    _store_all(orc, w, kp, vp, ks, vs)
    q = w.q_decode()
    qb = bf16_bits(q)
    lens = w.lengths.astype(np.int32)
    got = orc.decode_attn(qb, kp, vp, w.block_tables, lens, Hq=w.Hq, Hkv=w.Hkv, D=w.D, BS=w.BS,
                          k_scale=ks, v_scale=vs, sm_scale=w.sm_scale())
    g = w.Hq // w.Hkv
    for b in range(w.B):
        L = int(lens[b])
        k, v = w.kv(b, 0, L)
        K = torch.from_numpy(_values(bf16_bits(k), keb, ks)).double().permute(1, 0, 2)   # [Hkv][L][D]
        V = torch.from_numpy(_values(bf16_bits(v), veb, vs)).double().permute(1, 0, 2)
        K, V = K.repeat_interleave(g, dim=0), V.repeat_interleave(g, dim=0)
        Q = torch.from_numpy(orc.bf16_to_f32(qb[b:b + 1])).double().permute(1, 0, 2)      # [Hq][1][D]
        ref = F.scaled_dot_product_attention(Q, K, V, scale=w.sm_scale()).permute(1, 0, 2).numpy()[0]
        assert np.allclose(got[b], ref, rtol=1e-12, atol=1e-12), (keb, veb, b)
    if (keb, veb) != (1, 1):
        # the bf16 side really differs from an E4M3 cache of the same inputs
        k8, v8 = _pools(w, 1, 1)
        _store_all(orc, w, k8, v8, 0.02, 0.015)
        other = orc.decode_attn(qb, k8, v8, w.block_tables, lens, Hq=w.Hq, Hkv=w.Hkv, D=w.D, BS=w.BS,
                                k_scale=0.02, v_scale=0.015, sm_scale=w.sm_scale())
        assert not np.allclose(got, other, rtol=0, atol=1e-6)


@pytest.mark.parametrize("keb,veb", [(1, 1), (1, 2), (2, 1), (2, 2)])
def test_typed_prefill_matches_masked_fp64_sdpa(orc, keb, veb):
    """Chunked prefill over every element-type combination equals torch's fp64
    SDPA with the causal mask (query i at position ctx + i sees keys <= it),
    over values built without the oracle."""
    from synth import Spec
    ctx, chunk = 37, 19
    w = Workload("p", spec=Spec("p", 4, 2, 64, 16, [ctx, ctx + 7, 0], 4343, 0.05, 0.04, new_tokens=chunk))
    ks = 0.05 if keb == 1 else 1.0
    vs = 0.04 if veb == 1 else 1.0
    kp, vp = _pools(w, keb, veb)
    for b in range(w.B):
        L = int(w.total_lengths[b])
        k, v = w.kv(b, 0, L)
        orc.store(bf16_bits(k), bf16_bits(v), w.slots(b, 0, L), kp, vp, Hkv=w.Hkv, D=w.D, BS=w.BS,
                  k_scale=ks, v_scale=vs)
    qb = bf16_bits(w.q_chunk())
    cu = np.concatenate([[0], np.cumsum([chunk] * w.B)]).astype(np.int32)
    out = orc.prefill_attn(qb, kp, vp, cu, w.lengths.astype(np.int32), w.block_tables, Hq=w.Hq, Hkv=w.Hkv,
                           D=w.D, BS=w.BS, k_scale=ks, v_scale=vs, sm_scale=w.sm_scale())
    g = w.Hq // w.Hkv
    for b in range(w.B):
        c = int(w.lengths[b])
        L = c + chunk
        k, v = w.kv(b, 0, L)
        K = torch.from_numpy(_values(bf16_bits(k), keb, ks)).double().permute(1, 0, 2).repeat_interleave(g, 0)
        V = torch.from_numpy(_values(bf16_bits(v), veb, vs)).double().permute(1, 0, 2).repeat_interleave(g, 0)
        Q = torch.from_numpy(orc.bf16_to_f32(qb[cu[b]:cu[b + 1]])).double().permute(1, 0, 2)
        mask = torch.arange(L)[None, :] <= (c + torch.arange(chunk)[:, None])
        ref = F.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=w.sm_scale()).permute(1, 0, 2).numpy()
        np.testing.assert_allclose(out[cu[b]:cu[b + 1]], ref, rtol=1e-12, atol=1e-14)
