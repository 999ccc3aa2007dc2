"""Pins of the oracle's paged decode and chunked-prefill attention.

The oracle's attention is the plain definition softmax(q.K^T * sm_scale) V over
the dequantized cache [P1, tests/test-fp8.cpp check_fp8_attention: double
brute force, causal "past <= token"].  It is pinned against:
* torch's fp64 scaled_dot_product_attention on CPU over the same dequantized
  values, with grouped-query heads expanded by repeat_interleave (a library
  routine, not a retyping of the oracle's loops);
* special cases with closed forms: one key gives that key's V exactly;
  identical keys give the mean of V; zero length gives zeros;
* a causal prefill with no context equals is_causal SDPA; decode equals a
  one-row prefill chunk; the sampled mode equals the full mode.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from synth import Workload, bf16_bits


def _fill(orc, w, k_scale, v_scale, upto=None):
    kp = np.zeros((w.NB, w.Hkv, w.BS * w.D), np.uint8)
    vp = np.zeros_like(kp)
    for b in range(w.B):
        L = int(w.total_lengths[b] if upto is None else upto[b])
        k, v = w.kv(b, 0, L)
        orc.store(bf16_bits(k), bf16_bits(v), w.slots(b, 0, L), kp, vp, Hkv=w.Hkv, D=w.D,
                  BS=w.BS, k_scale=k_scale, v_scale=v_scale)
    return kp, vp


def _sdpa_ref(orc, w, kp, vp, q_bits_rows, b, L_keys, k_scale, v_scale, causal_offset=None):
    """fp64 SDPA over the dequantized keys of sequence b. q rows: [n][Hq][D] bf16 bits."""
    g = w.Hq // w.Hkv
    ks, vs = [], []
    for h in range(w.Hkv):
        kd, vd = orc.gather_dequant(kp, vp, w.block_tables[b], L_keys, h, Hkv=w.Hkv, D=w.D,
                                    BS=w.BS, k_scale=k_scale, v_scale=v_scale)
        ks.append(kd)
        vs.append(vd)
    K = torch.from_numpy(np.stack(ks)).double()           # [Hkv][L][D]
    V = torch.from_numpy(np.stack(vs)).double()
    K = K.repeat_interleave(g, dim=0)                      # [Hq][L][D]
    V = V.repeat_interleave(g, dim=0)
    Q = torch.from_numpy(orc.bf16_to_f32(q_bits_rows)).double().permute(1, 0, 2)   # [Hq][n][D]
    if causal_offset is None:
        mask = None
    else:
        n = Q.shape[1]
        pos = causal_offset + torch.arange(n)[:, None]
        mask = torch.arange(L_keys)[None, :] <= pos
    out = F.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=w.sm_scale())
    return out.permute(1, 0, 2).numpy()                    # [n][Hq][D]


def test_decode_matches_fp64_sdpa_tiny(orc):
    w = Workload("tiny")
    ks, vs, _ = w.scales()
    kp, vp = _fill(orc, w, ks, vs)
    q = bf16_bits(w.q_decode())
    out = orc.decode_attn(q, kp, vp, w.block_tables, w.lengths, Hq=w.Hq, Hkv=w.Hkv, D=w.D,
                          BS=w.BS, k_scale=ks, v_scale=vs, sm_scale=w.sm_scale())
    for b in range(w.B):
        ref = _sdpa_ref(orc, w, kp, vp, q[b:b + 1], b, int(w.lengths[b]), ks, vs)[0]
        np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-14)


def test_decode_gqa_mapping_is_grouped(orc):
    """Query head h reads kv-head h // (Hq/Hkv); the h % Hkv reading disagrees."""
    w = Workload("tiny")
    ks, vs, _ = w.scales()
    kp, vp = _fill(orc, w, ks, vs)
    q = bf16_bits(w.q_decode())
    out = orc.decode_attn(q, kp, vp, w.block_tables, w.lengths, Hq=w.Hq, Hkv=w.Hkv, D=w.D,
                          BS=w.BS, k_scale=ks, v_scale=vs, sm_scale=w.sm_scale())
    b, L = 3, int(w.lengths[3])
    kd1, vd1 = orc.gather_dequant(kp, vp, w.block_tables[b], L, 1, Hkv=w.Hkv, D=w.D, BS=w.BS,
                                  k_scale=ks, v_scale=vs)
    qh = torch.from_numpy(orc.bf16_to_f32(q[b, 1])).double()
    p = torch.softmax(torch.from_numpy(kd1).double() @ qh * w.sm_scale(), 0)
    wrong = (p[:, None] * torch.from_numpy(vd1).double()).sum(0).numpy()
    assert not np.allclose(out[b, 1], wrong)     # head 1 belongs to kv-head 0 when g = 2


def test_decode_special_cases(orc):
    Hq, Hkv, D, BS = 4, 2, 64, 16
    rng = np.random.default_rng(0)
    kp = rng.integers(0, 0x7E, size=(4, Hkv, BS * D), dtype=np.uint8)
    vp = rng.integers(0, 0x7E, size=(4, Hkv, BS * D), dtype=np.uint8)
    tables = np.array([[2, 0], [1, 3], [3, 1]], np.int32)
    q = rng.integers(0x3000, 0x4000, size=(3, Hq, D)).astype(np.uint16)
    out = orc.decode_attn(q, kp, vp, tables, np.array([1, 0, 20], np.int32), Hq=Hq, Hkv=Hkv, D=D,
                          BS=BS, k_scale=0.5, v_scale=0.25, sm_scale=0.125)
    # one key: the output is that key's dequantized V row exactly
    for h in range(Hq):
        _, vd = orc.gather_dequant(kp, vp, tables[0], 1, h // 2, Hkv=Hkv, D=D, BS=BS,
                                   k_scale=0.5, v_scale=0.25)
        assert np.array_equal(out[0, h], vd[0].astype(np.float64))
    # zero length: zeros
    assert np.all(out[1] == 0)
    # identical keys: the mean of V
    kp2 = kp.copy()
    for s in range(20):
        blk, t = tables[2, s // BS], s % BS
        for h in range(Hkv):
            for d in range(D):
                kp2[blk, h, orc.k_tile_offset(t, d, BS, D)] = kp[tables[2, 0], h, orc.k_tile_offset(0, d, BS, D)]
    out2 = orc.decode_attn(q, kp2, vp, tables, np.array([1, 0, 20], np.int32), Hq=Hq, Hkv=Hkv,
                           D=D, BS=BS, k_scale=0.5, v_scale=0.25, sm_scale=0.125)
    for h in range(Hq):
        _, vd = orc.gather_dequant(kp2, vp, tables[2], 20, h // 2, Hkv=Hkv, D=D, BS=BS,
                                   k_scale=0.5, v_scale=0.25)
        np.testing.assert_allclose(out2[2, h], vd.astype(np.float64).mean(0), rtol=0, atol=1e-13)


def test_decode_sampled_equals_full(orc):
    w = Workload("tiny")
    ks, vs, _ = w.scales()
    kp, vp = _fill(orc, w, ks, vs)
    q = bf16_bits(w.q_decode())
    kw = dict(Hq=w.Hq, Hkv=w.Hkv, D=w.D, BS=w.BS, k_scale=ks, v_scale=vs, sm_scale=w.sm_scale())
    full = orc.decode_attn(q, kp, vp, w.block_tables, w.lengths, **kw)
    sel = np.array([[0, 3], [2, 1], [3, 0]], np.int32)
    part = orc.decode_attn(q, kp, vp, w.block_tables, w.lengths, sel=sel, **kw)
    for b, h in sel:
        assert np.array_equal(part[b, h], full[b, h])
    assert np.isnan(part[1]).all()


def _prefill_workload(ctx, chunk):
    from synth import Spec
    spec = Spec("p", 4, 2, 64, 16, [ctx, ctx + 7, 0], 4242, 0.05, 0.04, new_tokens=chunk)
    return Workload("p", spec=spec)


@pytest.mark.parametrize("ctx,chunk", [(0, 21), (37, 19)])
def test_prefill_matches_masked_fp64_sdpa(orc, ctx, chunk):
    w = _prefill_workload(ctx, chunk)
    ks, vs, _ = w.scales()
    kp, vp = _fill(orc, w, ks, vs)
    q = bf16_bits(w.q_chunk())
    cu = np.concatenate([[0], np.cumsum([chunk] * w.B)]).astype(np.int32)
    out = orc.prefill_attn(q, kp, vp, cu, w.lengths.astype(np.int32), w.block_tables, Hq=w.Hq,
                           Hkv=w.Hkv, D=w.D, BS=w.BS, k_scale=ks, v_scale=vs, sm_scale=w.sm_scale())
    for b in range(w.B):
        c = int(w.lengths[b])
        rows = q[cu[b]:cu[b + 1]]
        if c == 0:
            # no context: textbook causal attention
            g = w.Hq // w.Hkv
            ks_, vs_ = [], []
            for h in range(w.Hkv):
                kd, vd = orc.gather_dequant(kp, vp, w.block_tables[b], chunk, h, Hkv=w.Hkv, D=w.D,
                                            BS=w.BS, k_scale=ks, v_scale=vs)
                ks_.append(kd)
                vs_.append(vd)
            K = torch.from_numpy(np.stack(ks_)).double().repeat_interleave(g, 0)
            V = torch.from_numpy(np.stack(vs_)).double().repeat_interleave(g, 0)
            Q = torch.from_numpy(orc.bf16_to_f32(rows)).double().permute(1, 0, 2)
            ref = F.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=w.sm_scale())
            ref = ref.permute(1, 0, 2).numpy()
        else:
            ref = _sdpa_ref(orc, w, kp, vp, rows, b, c + chunk, ks, vs, causal_offset=c)
        np.testing.assert_allclose(out[cu[b]:cu[b + 1]], ref, rtol=1e-12, atol=1e-14)


def test_decode_equals_one_row_prefill(orc):
    w = _prefill_workload(30, 1)
    ks, vs, _ = w.scales()
    kp, vp = _fill(orc, w, ks, vs)
    q = bf16_bits(w.q_chunk())                               # one query per sequence
    cu = np.arange(w.B + 1, dtype=np.int32)
    kw = dict(Hq=w.Hq, Hkv=w.Hkv, D=w.D, BS=w.BS, k_scale=ks, v_scale=vs, sm_scale=w.sm_scale())
    pre = orc.prefill_attn(q, kp, vp, cu, w.lengths.astype(np.int32), w.block_tables, **kw)
    dec = orc.decode_attn(q.reshape(w.B, w.Hq, w.D), kp, vp, w.block_tables,
                          w.total_lengths.astype(np.int32), **kw)
    assert np.array_equal(pre, dec)
