"""bench.py's CPU-oracle baselines on the host: bounded time and memory.

The prefill baseline samples query rows of the chunked-prefill workload and
asks the oracle for them; the oracle returns a full-size [rows][Hq][D] fp64
array per call (268 MB at this workload).  Keeping a view of each call's
output kept every array alive and exhausted host memory on a large host.
This runs the same code path on the full prefill workload with a short budget
and checks that the process's peak resident memory grows by a bounded amount
(one full-size output per worker thread, not one per sampled row).
"""
from __future__ import annotations

import importlib.util
import os
import resource

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("kvfp8_bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_prefill_cpu_baseline_memory_is_bounded():
    torch = pytest.importorskip("torch")
    import oracle
    from synth import Workload
    oracle.build()
    bench = _bench()
    w = Workload("prefill")
    n = w.spec.new_tokens
    ctx = w.lengths.astype(np.int32)
    q = w.q_chunk()
    out = torch.zeros((w.B * n, w.Hq, w.D), dtype=torch.bfloat16)   # stands in for the GPU output
    oh = bench.OracleHost(w, range(w.B), w.block_tables, w.total_lengths, *w.scales()[:2],
                          lambda b, lo, m: w.kv(b, lo, m))
    before = resource.getrusage(resource.RUSAGE_SELF).ru_maxrss * 1024
    res = bench._cpu_prefill(w, oh, q, out, ctx, n, 1.0)
    grown = resource.getrusage(resource.RUSAGE_SELF).ru_maxrss * 1024 - before
    threads = res["cores"]
    full_out = w.B * n * w.Hq * w.D * 8
    # the inputs and one full-size output per thread (the host pools were built before)
    assert grown < (threads + 4) * full_out, (grown, threads)
    assert res["kind"] == "oracle" and res["unit"] == "TFLOP/s" and res["value"] > 0
    assert res["single_thread"]["cores"] == 1 and res["single_thread"]["value"] > 0


def test_compact_oracle_pools_hold_the_full_pools_blocks():
    """OracleHost keeps only the sampled sequences' blocks, renumbered: every
    such block must hold exactly the bytes of the same block of a full-size
    oracle store through the workload's own tables (here a 1/16 variable-length
    workload over a pool four times larger than it needs)."""
    import oracle
    from synth import Workload, bf16_bits
    oracle.build()
    bench = _bench()
    w = Workload("varlen", scale_down=16, pool_frac=0.0)
    ks, vs, _ = w.scales()
    seqs = [1, 4, 7]
    oh = bench.OracleHost(w, seqs, w.block_tables, w.total_lengths, ks, vs, lambda b, lo, m: w.kv(b, lo, m))
    kp = np.zeros((w.NB, w.Hkv, w.BS * w.D), np.uint8)
    vp = np.zeros_like(kp)
    row = w.Hkv * w.D
    for b in seqs:
        L = int(w.total_lengths[b])
        k, v = w.kv(b, 0, L)
        oracle.store(bf16_bits(k).reshape(L, row), bf16_bits(v).reshape(L, row), w.slots(b, 0, L), kp, vp,
                     Hkv=w.Hkv, D=w.D, BS=w.BS, k_scale=ks, v_scale=vs)
    n = 0
    for b in seqs:
        nb = -(-int(w.total_lengths[b]) // w.BS)
        full = w.block_tables[b, :nb]
        compact = oh.tables[b, :nb]
        assert np.array_equal(compact, np.arange(n, n + nb))
        assert np.array_equal(oh.kp[compact], kp[full]) and np.array_equal(oh.vp[compact], vp[full])
        n += nb
    assert oh.kp.shape[0] == n


def test_per_operation_cpu_baselines_report_rates():
    """The decode, store and K-shift baselines on a 1/8 long-context workload:
    each reports a positive rate for one thread and for all host cores, and the
    decode's parity sample against its own oracle output is exact."""
    import oracle
    from synth import Workload, bf16_bits
    oracle.build()
    bench = _bench()
    w = Workload("longctx", scale_down=8)
    ks, vs, _ = w.scales()
    oh = bench.OracleHost(w, range(w.B), w.block_tables, w.total_lengths, ks, vs, lambda b, lo, m: w.kv(b, lo, m))
    q = w.q_decode()
    ref = oracle.decode_attn(bf16_bits(q), oh.kp, oh.vp, oh.tables, w.total_lengths.astype(np.int32), Hq=w.Hq,
                             Hkv=w.Hkv, D=w.D, BS=w.BS, k_scale=ks, v_scale=vs, sm_scale=w.sm_scale())
    cpu, parity = bench._cpu_decode(w, oh, q, {"fp32": ref.astype(np.float32)}, 1.0)
    assert parity["outside_tolerance_fp32_out"] == 0 and parity["max_abs_err_fp32_out"] < 1e-6
    st = bench._cpu_store(w, oh, 1.0)
    ksh = bench._cpu_kshift(w, oh, -4096, 1e6, w.D, 1.0)
    for r in (cpu, st, ksh):
        assert r["kind"] == "oracle" and r["value"] > 0 and r["single_thread"]["value"] > 0 and r["cores"] >= 1
