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
    before = resource.getrusage(resource.RUSAGE_SELF).ru_maxrss * 1024
    res = bench._cpu_prefill(w, q, out, ctx, n, 1.0)
    grown = resource.getrusage(resource.RUSAGE_SELF).ru_maxrss * 1024 - before
    threads = res["cores"]
    full_out = w.B * n * w.Hq * w.D * 8
    # the host pools (2 x 75 MB), the inputs and one full-size output per thread
    assert grown < (threads + 4) * full_out, (grown, threads)
    assert res["kind"] == "oracle" and res["unit"] == "TFLOP/s" and res["value"] > 0
    assert res["single_thread"]["cores"] == 1 and res["single_thread"]["value"] > 0
