"""Benchmark of the FP8-E4M3 paged KV cache on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama8b]

Default workload (the Llama-3-8B-shaped layer): 32 query / 8 kv heads, head
dim 128, block 16, 64 sequences x 4096 cached tokens, K/V ~ N(0,1) bf16 with
4 outlier channels x20, per-tensor fp32 scales amax/448, block table a random
permutation of the 16384 blocks.  One step = kv_store_fp8 of all 262,144
tokens (the cache fill) + paged_attn_decode of one query token per sequence.
Inputs are resident in HBM before timing starts.  Stores and decodes are
timed in separate back-to-back phases, and three copies of the pools are
rotated so that a decode never reads the copy the previous decode read (the
256 MB last-level cache cannot serve it).

Prints one JSON line.  `value` is the decode's achieved HBM bandwidth
(algorithmic bytes / decode time); decode tokens/s and kv_store tokens/s are
reported beside it.  `roofline` is for the decode kernel; `cpu_baseline` is
the CPU oracle timed on a bounded sample of the same workload (all host cores,
with the single-thread figure beside it); `stream_read_ceiling` is a plain
streaming read of 2 GiB buffers, the achievable-bandwidth ceiling.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama8b", choices=["llama8b", "prefill", "longctx", "varlen"])
    ap.add_argument("--pool-frac", type=float, default=0.5,
                    help="varlen: fraction of 288 GB used for the block pool")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="bound on the CPU-oracle sample time (0 disables it)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (counter calibration)")
    return ap.parse_args()


def _source_sha(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "fp8_e4m3_scaled_amd", "csrc", n), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic_from_profile(summary: str, kernel_sha: str):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(PROFILES, summary)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha") != kernel_sha:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration():
    """A plain device-to-device copy of 1 GiB, 10 times (for FETCH_SIZE / WRITE_SIZE scaling)."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "launches": 10}))


def _time_ms(fn, stream, events):
    import torch
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    fn()
    e.record(stream)
    events.append((s, e))


def run_llama8b(args):
    import torch
    import fp8_e4m3_scaled_amd as kv
    from synth import Workload, bf16_bits

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    w = Workload("llama8b", device=dev)
    ks, vs, _ = w.scales()
    T = int(w.total_lengths.sum())
    row = w.Hkv * w.D

    # inputs resident in HBM: all K/V rows of the fill, their slots, q, tables
    K = torch.empty((T, row), dtype=torch.bfloat16, device=dev)
    V = torch.empty((T, row), dtype=torch.bfloat16, device=dev)
    slots = np.empty(T, np.int64)
    pos = 0
    for b in range(w.B):
        L = int(w.total_lengths[b])
        k, v = w.kv(b, 0, L)
        K[pos:pos + L] = k.reshape(L, row)
        V[pos:pos + L] = v.reshape(L, row)
        slots[pos:pos + L] = w.slots(b, 0, L)
        pos += L
    slots_d = torch.from_numpy(slots).to(dev)
    q = w.q_decode(dev)
    tables = torch.from_numpy(w.block_tables.astype(np.int32)).to(dev)
    lens = torch.from_numpy(w.total_lengths.astype(np.int32)).to(dev)
    max_len = int(w.total_lengths.max())
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.bfloat16, device=dev)

    copies = 3
    pools, handles = [], []
    for _ in range(copies):
        kp = torch.zeros((w.NB, w.Hkv, w.BS * w.D), dtype=torch.uint8, device=dev)
        vp = torch.zeros_like(kp)
        h = kv.kv_cache_alloc(1, w.NB, w.BS, w.Hkv, w.D, [float(ks)], [float(vs)], kv.DTYPE_F32, kp, vp)
        kv.kv_store_fp8(h, 0, K, V, row, row, slots_d, T, stream)
        pools.append((kp, vp))
        handles.append(h)
    ws_bytes = kv.paged_attn_decode_workspace(handles[0], w.B, w.Hq, max_len)
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def store(i):
        kv.kv_store_fp8(handles[i % copies], 0, K, V, row, row, slots_d, T, stream)

    def decode(i):
        kv.paged_attn_decode(handles[(i + 1) % copies], 0, q, w.Hq, tables, w.max_blocks, lens, w.B,
                             max_len, w.sm_scale(), out, kv.DTYPE_BF16, ws, ws_bytes, stream)

    # Each operation is timed in its own phase: back-to-back store fills (each
    # one also pays the write-back of the previous fill's dirty lines), then
    # back-to-back decodes.  Timing them interleaved would charge the store's
    # deferred write-back to the decode that follows it.
    t0 = time.perf_counter()
    st_t = _timed(store, args.steps, args.warmup, stream)
    de_t = _timed(decode, args.steps, args.warmup, stream)
    wall = time.perf_counter() - t0
    # the same decode with fp32 outputs (untimed), for the parity sample
    out_f32 = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=dev)
    kv.paged_attn_decode(handles[0], 0, q, w.Hq, tables, w.max_blocks, lens, w.B, max_len, w.sm_scale(), out_f32,
                         kv.DTYPE_F32, ws, ws_bytes, stream)
    torch.cuda.synchronize()

    # algorithmic bytes (what the method must move)
    kv_bytes = int(w.total_lengths.sum()) * 2 * w.Hkv * w.D
    blocks = int(sum(-(-int(L) // w.BS) for L in w.total_lengths))
    decode_bytes = kv_bytes + w.B * w.Hq * w.D * (2 + 2) + 4 * blocks + 4 * w.B
    store_bytes = T * (6 * w.Hkv * w.D + 8)
    de_mean, st_mean = de_t.mean(), st_t.mean()
    decode_gbps = decode_bytes / (de_mean * 1e-3) / 1e9
    store_gbps = store_bytes / (st_mean * 1e-3) / 1e9

    kernel_sha = _source_sha("decode.hip", "fp8_device.hpp", "decode_args.hpp")
    traffic = _traffic_from_profile("decode_llama8b_pmc.txt", kernel_sha)

    result = {
        "metric": "fp8-KV paged decode attn achieved HBM GB/s + tokens/s; kv_store tokens/s",
        "value": round(decode_gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(st_mean + de_mean, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 cache; bf16/f16 MFMA, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": "llama8b", "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.D,
                   "block_size": w.BS, "num_seqs": w.B, "seq_len": max_len, "fill_tokens": T,
                   "out_dtype": "bf16", "decode_splits": ws_bytes > 0},
        "decode": {**_stats(de_t),
                   "algorithmic_bytes": decode_bytes, "GBps": round(decode_gbps, 1),
                   "frac_hbm_peak": round(decode_gbps / HBM_PEAK_GBPS, 4),
                   "tokens_per_s": round(w.B / (de_mean * 1e-3), 1),
                   "kv_tokens_scanned_per_s": round(int(w.total_lengths.sum()) / (de_mean * 1e-3), 1)},
        "kv_store": {**_stats(st_t), "tokens": T, "algorithmic_bytes": store_bytes,
                     "tokens_per_s": round(T / (st_mean * 1e-3), 1), "GBps": round(store_gbps, 1),
                     "frac_hbm_peak": round(store_gbps / HBM_PEAK_GBPS, 4)},
        "roofline": {"bound": "hbm", "achieved": round(decode_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(decode_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": "decode_kernel<128,16,1,1>",
                     "kernel_source_sha": kernel_sha},
        "wall_s_timed": round(wall, 3),
    }

    result["stream_read_ceiling"] = _stream_ceiling(stream)
    result["decode"]["frac_of_stream_ceiling"] = round(decode_gbps / result["stream_read_ceiling"]["GBps"], 4)
    result["paged_gather_ceiling"] = _gather_ceiling(args, kv, w, handles, tables, w.max_blocks, lens, w.B,
                                                     w.Hkv, kv_bytes, stream)
    result["decode"]["frac_of_gather_ceiling"] = round(
        decode_gbps / result["paged_gather_ceiling"]["GBps"], 4)
    # the fill's own traffic with no arithmetic (overwrites the pools: after every read of them)
    result["kv_store"]["pattern_ceiling"] = _store_ceiling(args, w, pools, K, V, row, slots_d, T, store_bytes,
                                                           stream)
    result["kv_store"]["frac_of_pattern_ceiling"] = round(
        store_gbps / result["kv_store"]["pattern_ceiling"]["list_order"]["GBps"], 4)
    result["calibrate"] = _calibrate(args, kv, K, V, T, row, ks, vs, stream)
    for h in handles:
        kv.kv_cache_free(h)
    handles = []
    del pools
    torch.cuda.empty_cache()
    result["element_types"] = _typed_exchange(args, kv, w, K, V, slots_d, T, q, tables, lens, max_len, out,
                                              ks, vs, de_mean, stream)
    if args.cpu_seconds > 0:
        offs = np.concatenate([[0], np.cumsum(w.total_lengths)]).astype(np.int64)
        oh = OracleHost(w, range(w.B), w.block_tables, w.total_lengths, ks, vs,
                        lambda b, lo, n: (K[offs[b] + lo:offs[b] + lo + n], V[offs[b] + lo:offs[b] + lo + n]))
        got = {"bf16": out.float().cpu().numpy(), "fp32": out_f32.cpu().numpy()}
        cpu_de, result["parity_sample"] = _cpu_decode(w, oh, q, got, args.cpu_seconds)
        result["cpu_baseline"] = cpu_de
        result["cpu_baseline_ops"] = {"decode": cpu_de, "store": _cpu_store(w, oh, args.cpu_seconds / 2)}
    return result


def _calibrate(args, kv, K, V, T, row, ks, vs, stream):
    """On-device scale calibration over the whole fill (K and V, 2 bytes per
    element read): event time per call, and whether the fp32 scales it
    produces equal the ones the input generator set for this workload."""
    import torch
    amax = torch.zeros(2, dtype=torch.float32, device=K.device)
    out = torch.zeros(2, dtype=torch.int32, device=K.device)

    def call(i):
        kv.kv_calibrate_scales(K, V, row, row, T, row, amax, out, kv.DTYPE_F32, stream)

    ms = _timed(call, args.steps, args.warmup, stream).mean()
    nbytes = 2 * T * row * 2 + 8 + 8
    got = out.cpu().numpy().view(np.float32)
    return {"ms_mean": round(ms, 5), "algorithmic_bytes": nbytes,
            "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "scales_equal_generator": bool(got[0] == np.float32(ks) and got[1] == np.float32(vs)),
            "kernel": "amax_kernel + scale_kernel"}


def _typed_exchange(args, kv, w, K, V, slots_d, T, q, tables, lens, max_len, out, ks, vs, fp8_ms, stream):
    """The same decode over caches whose pools hold bf16 values instead of E4M3
    codes (the bf16 twin, and the two mixed K/V combinations), on the same
    inputs and shape: the decode time of each and the exchange rate, the E4M3
    cache's decode throughput over the other's.  Algorithmic bytes count each
    pool at its own element size."""
    import torch
    E, B = kv.ELEM_E4M3, kv.ELEM_BF16
    row = w.Hkv * w.D
    n = w.NB * w.Hkv * w.BS * w.D
    kv_tokens = int(w.total_lengths.sum())
    blocks = int(sum(-(-int(L) // w.BS) for L in w.total_lengths))
    out = torch.empty_like(out)   # the E4M3 decode's output stays intact for the parity sample
    res = {}
    for name, ke, ve in (("bf16_twin", B, B), ("k_e4m3_v_bf16", E, B), ("k_bf16_v_e4m3", B, E)):
        keb, veb = (1 if ke == E else 2), (1 if ve == E else 2)
        hs, pools = [], []
        for _ in range(3):
            kp = torch.zeros(n * keb, dtype=torch.uint8, device=K.device)
            vp = torch.zeros(n * veb, dtype=torch.uint8, device=K.device)
            h = kv.kv_cache_alloc_typed(1, w.NB, w.BS, w.Hkv, w.D, ke, ve,
                                        [float(ks) if ke == E else 1.0], [float(vs) if ve == E else 1.0],
                                        kv.DTYPE_F32, kp, vp)
            kv.kv_store_fp8(h, 0, K, V, row, row, slots_d, T, stream)
            hs.append(h)
            pools.append((kp, vp))
        ws_bytes = kv.paged_attn_decode_workspace(hs[0], w.B, w.Hq, max_len)
        ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=K.device)
        torch.cuda.synchronize()

        def decode(i):
            kv.paged_attn_decode(hs[(i + 1) % 3], 0, q, w.Hq, tables, w.max_blocks, lens, w.B, max_len,
                                 w.sm_scale(), out, kv.DTYPE_BF16, ws, ws_bytes, stream)

        ms = _timed(decode, args.steps, args.warmup, stream).mean()
        nbytes = kv_tokens * w.Hkv * w.D * (keb + veb) + w.B * w.Hq * w.D * 4 + 4 * blocks + 4 * w.B
        res[name] = {"k_elem": "e4m3" if ke == E else "bf16", "v_elem": "e4m3" if ve == E else "bf16",
                     "ms_mean": round(ms, 5), "algorithmic_bytes": nbytes,
                     "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "tokens_per_s": round(w.B / (ms * 1e-3), 1),
                     "e4m3_speedup": round(ms / fp8_ms, 4)}
        for h in hs:
            kv.kv_cache_free(h)
        del pools, ws
        torch.cuda.empty_cache()
    return res


def _gather_ceiling(args, kv, w, handles, tables, max_blocks, lens, B, Hkv, kv_bytes, stream, chunk_blocks=None):
    """The gather probe over the decode's own pools and block tables: a plain
    read of exactly the K/V tiles the decode reads, the ceiling of its
    scattered-tile access pattern; one workgroup per (sequence, kv-head), or
    per chunk of chunk_blocks table entries of one.  GB/s counts the K/V
    bytes only."""
    import torch
    import probe
    chunks = 1 if chunk_blocks is None else -(-max_blocks // chunk_blocks)
    out = torch.empty(chunks * B * Hkv, dtype=torch.int32, device="cuda")
    pools = [kv.kv_cache_pools(h, 0) for h in handles]
    copies = len(handles)

    def call(i):
        kp, vp, _ = pools[(i + 1) % copies]
        if chunk_blocks is None:
            probe.gather(kp, vp, w.NB, w.Hkv, w.BS, w.D, 1, 1, tables, max_blocks, lens, B, out, stream)
        else:
            probe.gather_split(kp, vp, w.NB, w.Hkv, w.BS, w.D, 1, 1, tables, max_blocks, lens, B, chunk_blocks, out,
                               stream)

    ms = _timed(call, args.steps, args.warmup, stream).mean()
    gbps = kv_bytes / (ms * 1e-3) / 1e9
    what = ("one workgroup per (sequence, kv-head)" if chunk_blocks is None else
            f"one workgroup per {chunk_blocks} blocks of one (sequence, kv-head)")
    return {"GBps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4), "ms_mean": round(ms, 5),
            "bytes": kv_bytes, "kernel": f"gather_probe ({what})"}


def _kshift_ceiling(args, w, pools, slots, nsl, nbytes, stream):
    """The K-shift's own traffic with no arithmetic (the rmw probe: the same
    items and launch, each byte XORed with 1, in place) over the timed slot
    list, and over the same slots in address order.  The first is the ceiling
    of the K-shift through these block tables; the second shows what the
    shuffled block order costs.  GB/s counts the K-shift's algorithmic bytes."""
    import torch
    import probe
    ordered = torch.sort(slots).values
    copies = len(pools)
    out = {}
    for name, sl in (("list_order", slots), ("address_order", ordered)):
        def call(i, sl=sl):
            probe.rmw(pools[i % copies][0], w.NB, w.Hkv, w.BS, w.D, w.D, sl, nsl, stream)
        ms = _timed(call, args.steps, args.warmup, stream).mean()
        gbps = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"GBps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                     "ms_mean": round(ms, 5)}
    out["kernel"] = "rmw_probe (the K-shift's items and grid-stride launch, XOR instead of the rotation)"
    return out


def _store_ceiling(args, w, pools, K, V, row, slots, T, nbytes, stream):
    """The cache fill's own traffic with no arithmetic (the store_copy probe:
    the store's 16-token run path, each value's high byte written where the
    store writes its code) over the same inputs and rotating pools: with the
    timed slot list, the ceiling of the fill's access pattern; with token i
    going to slot i, what the shuffled block order costs.  GB/s counts the
    store's algorithmic bytes."""
    import torch
    import probe
    copies = len(pools)
    out = {}
    # the timed slot list, and token i to slot i (blocks handed out in address order)
    for name, sl in (("list_order", slots), ("address_order", torch.arange(T, dtype=torch.int64, device="cuda"))):
        def call(i, sl=sl):
            kp, vp = pools[i % copies]
            probe.store_copy(K, V, row, row, sl, T, kp, vp, w.NB, w.Hkv, w.BS, w.D, stream)

        ms = _timed(call, args.steps, args.warmup, stream).mean()
        gbps = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"GBps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4), "ms_mean": round(ms, 5)}
    out["kernel"] = "store_copy_probe (the store's run path, high bytes instead of codes)"
    return out


def _stream_ceiling(stream, nbytes=2 << 30, launches=20):
    """A plain streaming read (the read probe) of two alternating 2 GiB buffers:
    the achievable read bandwidth of this part, reported beside the 8 TB/s figure."""
    import torch
    import probe
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    n_out = 1024
    sink = torch.empty(n_out, dtype=torch.int32, device="cuda")
    ms = _timed(lambda i: probe.read(bufs[i % 2], nbytes, sink, n_out, stream), launches, 3, stream).mean()
    gbps = nbytes / (ms * 1e-3) / 1e9
    del bufs
    return {"GBps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4), "bytes": nbytes,
            "launches": launches, "kernel": "read_probe (XOR-reduce read, 1024 workgroups)"}


def _host_threads():
    """Host cores this process may use (at most 16: the share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _timed_oracle(items, fn, budget_s):
    """The oracle as it stands, timed twice on the same kind of work: one thread
    until half the budget is used, then all host cores (a thread pool: the C
    oracle releases the GIL) on the next items.  Returns the per-item results,
    the two (items, seconds) pairs and the thread count."""
    from concurrent.futures import ThreadPoolExecutor
    n = _host_threads()
    # leave at least as many items for every core as the single thread takes
    max_single = max(1, len(items) // (n + 1))
    results, single_t, i = [], 0.0, 0
    while i < min(len(items), max_single) and single_t < budget_s / 2:
        t0 = time.perf_counter()
        results.append(fn(items[i]))
        single_t += time.perf_counter() - t0
        i += 1
    single_n = i
    per_thread = max(1, single_n)
    batch = items[i:i + n * per_thread]
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=n) as ex:
        results += list(ex.map(fn, batch))
    multi_t = time.perf_counter() - t0
    return results, (single_n, single_t), (len(batch), multi_t), n


class OracleHost:
    """Host pools of the CPU oracle holding every token of the sequences `seqs`
    (stored by the oracle itself, untimed), in compact block ids: the blocks the
    sequences use, renumbered 0.. in table order, so that a pool of any size on
    the GPU (the variable-length workload's is 144 GB) needs only the sampled
    sequences' blocks on the host.  src(b, lo, n) gives the bf16 K/V rows."""

    def __init__(self, w, seqs, tables, lens, ks, vs, src):
        import oracle
        from concurrent.futures import ThreadPoolExecutor
        oracle._load()
        self.w, self.ks, self.vs, self.lens = w, np.float32(ks), np.float32(vs), np.asarray(lens, np.int64)
        self.seqs = list(seqs)
        self.tables = np.zeros_like(tables)
        nb = 0
        for b in self.seqs:
            n = -(-int(self.lens[b]) // w.BS)
            self.tables[b, :n] = np.arange(nb, nb + n, dtype=np.int32)
            nb += n
        self.kp = np.zeros((max(1, nb), w.Hkv, w.BS * w.D), np.uint8)
        self.vp = np.zeros_like(self.kp)
        self.src = src
        step = 16384

        def one(b):
            L = int(self.lens[b])
            for lo in range(0, L, step):
                n = min(step, L - lo)
                k, v = self.rows(b, lo, n)
                oracle.store(k, v, self.slots(b, lo, n), self.kp, self.vp, Hkv=w.Hkv, D=w.D, BS=w.BS,
                             k_scale=self.ks, v_scale=self.vs)
        with ThreadPoolExecutor(max_workers=_host_threads()) as ex:
            list(ex.map(one, self.seqs))

    def rows(self, b, lo, n):
        from synth import bf16_bits
        k, v = self.src(b, lo, n)
        row = self.w.Hkv * self.w.D
        return bf16_bits(k).reshape(n, row), bf16_bits(v).reshape(n, row)

    def slots(self, b, lo, n):
        p = np.arange(lo, lo + n, dtype=np.int64)
        return self.tables[b, p // self.w.BS].astype(np.int64) * self.w.BS + p % self.w.BS


def _cpu_decode(w, oh, q, got, budget_s):
    """The oracle's decode on a bounded sample: (sequence, kv-head) groups of the
    host pools' sequences in a seeded order, all query heads of each group, one
    thread and then all host cores.  Also compares the GPU decode outputs on
    those heads with the oracle: got maps "bf16" / "fp32" to [B][Hq][D] outputs;
    every element within |d| <= 2e-3 + 1e-2 |ref|, and the fp32 output's max |d|
    reported beside 2e-3."""
    import oracle
    from synth import bf16_bits
    q_bits = bf16_bits(q)
    G = w.Hq // w.Hkv
    lens = oh.lens.astype(np.int32)
    rng = np.random.default_rng(7)
    order = [(b, h) for b in oh.seqs for h in rng.permutation(w.Hkv).tolist()]

    def group(item):
        b, kvh = item
        sel = np.array([[b, kvh * G + j] for j in range(G)], np.int32)
        ref = oracle.decode_attn(q_bits, oh.kp, oh.vp, oh.tables, lens, Hq=w.Hq, Hkv=w.Hkv, D=w.D,
                                 BS=w.BS, k_scale=oh.ks, v_scale=oh.vs, sm_scale=w.sm_scale(), sel=sel)
        # a copy: the view would keep the oracle's whole [B][Hq][D] output alive
        return item, ref[b, kvh * G:(kvh + 1) * G].copy()

    def nbytes(item):
        L = int(lens[item[0]])
        return L * 2 * w.D + G * w.D * (2 + 2) + 4 * (-(-L // w.BS)) + 4

    results, (n1, t1), (n2, t2), threads = _timed_oracle(order, group, budget_s)
    parity = {"heads_checked": len(results) * G}
    for name, g in got.items():
        worst, bad = 0.0, 0
        for (b, kvh), ref in results:
            err = np.abs(g[b, kvh * G:(kvh + 1) * G] - ref)
            worst = max(worst, float(err.max()))
            bad += int((err > 2e-3 + 1e-2 * np.abs(ref)).sum())
        parity[f"max_abs_err_{name}_out"] = worst
        parity[f"outside_tolerance_{name}_out"] = bad
    b1 = sum(nbytes(it) for it, _ in results[:n1])
    b2 = sum(nbytes(it) for it, _ in results[n1:])
    cpu = {"value": round(b2 / t2 / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"{n2} (sequence, kv-head) groups x {G} query heads on {threads} threads, fp64 C "
                     f"oracle, {t2:.1f} s wall (seeded order over {len(order)} groups)",
           "single_thread": {"value": round(b1 / t1 / 1e9, 4), "cores": 1,
                             "sample": f"{n1} groups, {t1:.1f} s"},
           "tokens_per_s": round(n2 * G / w.Hq / t2, 4)}
    return cpu, parity


def _cpu_store(w, oh, budget_s, chunk=2048):
    """The oracle's store on a bounded sample: chunks of `chunk` tokens of the
    host pools' sequences (their rows drawn before the timed calls), one thread
    and then all host cores; chunks write disjoint slots.  Rewriting a token
    writes the bytes it already holds."""
    import oracle
    items = []
    for b in oh.seqs:
        for lo in range(0, int(oh.lens[b]), chunk):
            items.append((b, lo, min(chunk, int(oh.lens[b]) - lo)))
    rng = np.random.default_rng(8)
    items = [items[i] for i in rng.permutation(len(items))[:max(1, min(len(items), 16 * 32))]]
    rows = {}

    def prepare(it):
        if it not in rows:
            rows[it] = oh.rows(*it)
        return rows[it]

    def one(it):
        k, v = rows[it]
        b, lo, n = it
        oracle.store(k, v, oh.slots(b, lo, n), oh.kp, oh.vp, Hkv=w.Hkv, D=w.D, BS=w.BS, k_scale=oh.ks,
                     v_scale=oh.vs)
        return n

    # inputs of the first items (eight per host core), drawn outside the timed calls
    for it in items[:8 * (_host_threads() + 1)]:
        prepare(it)
    items = [it for it in items if it in rows]
    results, (n1, t1), (n2, t2), threads = _timed_oracle(items, one, budget_s)
    tok1, tok2 = sum(results[:n1]), sum(results[n1:])
    per_tok = 6 * w.Hkv * w.D + 8
    return {"value": round(tok2 / t2, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "GBps": round(tok2 * per_tok / t2 / 1e9, 4),
            "sample": f"{n2} chunks of up to {chunk} tokens on {threads} threads, C oracle, {t2:.2f} s wall",
            "single_thread": {"value": round(tok1 / t1, 1), "cores": 1, "GBps": round(tok1 * per_tok / t1 / 1e9, 4),
                              "sample": f"{n1} chunks, {t1:.2f} s"}}


def _cpu_kshift(w, oh, delta, theta, rot, budget_s, chunk=4096):
    """The oracle's K-shift (fp64 rotation, NEOX) on a bounded sample: chunks of
    `chunk` slots of the host pools' sequences, one thread and then all host
    cores (disjoint slots).  Runs in place on the host pools."""
    import oracle
    items = []
    for b in oh.seqs:
        for lo in range(0, int(oh.lens[b]), chunk):
            items.append((b, lo, min(chunk, int(oh.lens[b]) - lo)))
    rng = np.random.default_rng(9)
    items = [items[i] for i in rng.permutation(len(items))]

    def one(it):
        b, lo, n = it
        oracle.kshift(oh.kp, oh.slots(b, lo, n), Hkv=w.Hkv, D=w.D, BS=w.BS, delta=delta, theta=theta,
                      rot_dim=rot, neox=True)
        return n

    results, (n1, t1), (n2, t2), threads = _timed_oracle(items, one, budget_s)
    s1, s2 = sum(results[:n1]), sum(results[n1:])
    per_slot = 2 * w.Hkv * rot + 8
    return {"value": round(s2 * per_slot / t2 / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "slots_per_s": round(s2 / t2, 1),
            "sample": f"{n2} chunks of up to {chunk} slots on {threads} threads, C oracle, {t2:.2f} s wall",
            "single_thread": {"value": round(s1 * per_slot / t1 / 1e9, 4), "cores": 1,
                              "sample": f"{n1} chunks, {t1:.2f} s"}}


def _fill(w, kv, dev, stream, copies=1, upto=None, empty=False, elems=None):
    """Store tokens 0..upto[b]-1 of every sequence into `copies` caches (untimed setup).
    elems: (K, V) element types (default E4M3 both; a bf16 pool takes scale 1).
    Returns (pools, handles)."""
    import torch
    ks, vs, _ = w.scales()
    ke, ve = elems if elems is not None else (kv.ELEM_E4M3, kv.ELEM_E4M3)
    keb, veb = (1 if ke == kv.ELEM_E4M3 else 2), (1 if ve == kv.ELEM_E4M3 else 2)
    row = w.Hkv * w.D
    pools, handles = [], []
    for _ in range(copies):
        alloc = torch.empty if empty else torch.zeros
        kp = alloc((w.NB, w.Hkv, w.BS * w.D * keb), dtype=torch.uint8, device=dev)
        vp = alloc((w.NB, w.Hkv, w.BS * w.D * veb), dtype=torch.uint8, device=dev)
        handles.append(kv.kv_cache_alloc_typed(1, w.NB, w.BS, w.Hkv, w.D, ke, ve,
                                               [float(ks) if keb == 1 else 1.0], [float(vs) if veb == 1 else 1.0],
                                               kv.DTYPE_F32, kp, vp))
        pools.append((kp, vp))
    upto = w.lengths if upto is None else upto
    step = 65536
    for b in range(w.B):
        L = int(upto[b])
        for lo in range(0, L, step):
            n = min(step, L - lo)
            k, v = w.kv(b, lo, n, device=dev)
            sd = torch.from_numpy(w.slots(b, lo, n)).to(dev)
            for h in handles:
                kv.kv_store_fp8(h, 0, k.reshape(n, row), v.reshape(n, row), row, row, sd, n, stream)
    torch.cuda.synchronize()
    return pools, handles


class Timing:
    """Times of `steps` launches of one operation: per-launch HIP-event pairs
    (for the percentiles) and the mean over one timed region of the same
    number of back-to-back launches between a single event pair, which has no
    timing markers between the kernels.  mean() is the region mean."""

    def __init__(self, per_launch, region_ms):
        self.per_launch = per_launch
        self.region = float(region_ms)

    def mean(self):
        return self.region


def _timed(fn, steps, warmup, stream):
    """Times of fn(i) on `stream`: warm-up, a phase of per-launch event pairs,
    a second warm-up, then one event pair around `steps` back-to-back launches."""
    import torch
    for i in range(warmup):
        fn(i)
    ev = []
    for i in range(steps):
        _time_ms(lambda: fn(i), stream, ev)
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in ev])
    for i in range(warmup):
        fn(i)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(steps):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return Timing(per, a.elapsed_time(b) / steps)


def _stats(t):
    ms = t.per_launch
    return {"ms_mean": round(t.mean(), 5), "ms_mean_event_pairs": round(float(ms.mean()), 5),
            "ms_p10": round(float(np.percentile(ms, 10)), 5), "ms_p50": round(float(np.percentile(ms, 50)), 5),
            "ms_p90": round(float(np.percentile(ms, 90)), 5)}


def _decode_bytes(w, lens, out_bytes):
    blocks = int(sum(-(-int(L) // w.BS) for L in lens))
    return int(np.sum(lens)) * 2 * w.Hkv * w.D + w.B * w.Hq * w.D * (2 + out_bytes) + 4 * blocks + 4 * w.B


def _header(args, workload, value, unit, ms_per_step, config):
    return {"metric": "fp8-KV paged decode attn achieved HBM GB/s + tokens/s; kv_store tokens/s",
            "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "fp8_e4m3 cache; bf16/f16 MFMA, f32 accumulate",
            "data": "synthetic", "config": dict(workload=workload, **config)}


def run_prefill(args):
    """Chunked prefill: 4 sequences x (16384 cached + 2048 new) tokens, 32 q / 8 kv heads,
    head_dim 128, block 16.  Step = kv_store_fp8 of the 8192 chunk tokens + the causal
    prefill of their queries.  Roofline: the prefill kernel against the bf16/f16 MFMA peak."""
    import torch
    import fp8_e4m3_scaled_amd as kv
    from synth import Workload
    dev, stream = torch.device("cuda:0"), torch.cuda.current_stream()
    w = Workload("prefill", device=dev)
    pools, handles = _fill(w, kv, dev, stream)
    h = handles[0]
    n = w.spec.new_tokens
    row = w.Hkv * w.D
    ctx = w.lengths.astype(np.int32)
    K = torch.cat([w.kv(b, int(ctx[b]), n, device=dev)[0].reshape(n, row) for b in range(w.B)])
    V = torch.cat([w.kv(b, int(ctx[b]), n, device=dev)[1].reshape(n, row) for b in range(w.B)])
    sd = torch.from_numpy(np.concatenate([w.slots(b, int(ctx[b]), n) for b in range(w.B)])).to(dev)
    T = w.B * n
    q = w.q_chunk(dev)
    cu = torch.from_numpy((np.arange(w.B + 1) * n).astype(np.int32)).to(dev)
    ctx_d = torch.from_numpy(ctx).to(dev)
    tables = torch.from_numpy(w.block_tables.astype(np.int32)).to(dev)
    out = torch.empty((T, w.Hq, w.D), dtype=torch.bfloat16, device=dev)

    def store(i):
        kv.kv_store_fp8(h, 0, K, V, row, row, sd, T, stream)

    def prefill(i):
        kv.paged_attn_prefill_chunk(h, 0, q, w.Hq, cu, ctx_d, tables, w.max_blocks, w.B, T, n,
                                    int(ctx.max()), w.sm_scale(), out, kv.DTYPE_BF16, stream)

    st = _timed(store, args.steps, args.warmup, stream)
    pf = _timed(prefill, args.steps, args.warmup, stream)
    flops = sum(4 * w.D * w.Hq * (int(ctx[b]) * n + n * (n + 1) // 2) for b in range(w.B))
    tflops = flops / (pf.mean() * 1e-3) / 1e12
    store_bytes = T * (6 * w.Hkv * w.D + 8)
    res = _header(args, "prefill", round(tflops, 1), "TFLOP/s", float(st.mean() + pf.mean()),
                  {"q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.D, "block_size": w.BS,
                   "num_seqs": w.B, "context": int(ctx[0]), "chunk": n, "out_dtype": "bf16"})
    res["prefill"] = dict(_stats(pf), flops=flops, tflops=round(tflops, 2),
                          frac_mfma_peak=round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                          tokens_per_s=round(T / (pf.mean() * 1e-3), 1))
    res["kv_store"] = dict(_stats(st), tokens=T, algorithmic_bytes=store_bytes,
                           tokens_per_s=round(T / (st.mean() * 1e-3), 1),
                           GBps=round(store_bytes / (st.mean() * 1e-3) / 1e9, 1))
    psha = _source_sha("prefill.hip", "fp8_device.hpp", "internal.hpp")
    res["roofline"] = {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                       "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                       "traffic": _traffic_from_profile("prefill_pmc.txt", psha),
                       "kernel": "prefill_kernel<128,16,1,1>", "kernel_source_sha": psha}
    if args.cpu_seconds > 0:
        ks_, vs_, _ = w.scales()
        oh = OracleHost(w, range(w.B), w.block_tables, w.total_lengths, ks_, vs_,
                        lambda b, lo, m: w.kv(b, lo, m, device=dev))
        res["cpu_baseline"] = _cpu_prefill(w, oh, q, out, ctx, n, args.cpu_seconds)
        res["cpu_baseline_ops"] = {"prefill": res["cpu_baseline"], "store": _cpu_store(w, oh, args.cpu_seconds / 2)}
    kv.kv_cache_free(h)
    del pools
    # The same prefill over the bf16 twin and the mixed caches (context and
    # chunk stored untimed): time per call and the E4M3 cache's speedup.
    out2 = torch.empty_like(out)
    pf_ms = float(pf.mean())
    types = {}
    for name, ke, ve in (("bf16_twin", kv.ELEM_BF16, kv.ELEM_BF16), ("k_e4m3_v_bf16", kv.ELEM_E4M3, kv.ELEM_BF16),
                         ("k_bf16_v_e4m3", kv.ELEM_BF16, kv.ELEM_E4M3)):
        tp, th = _fill(w, kv, dev, stream, elems=(ke, ve))
        kv.kv_store_fp8(th[0], 0, K, V, row, row, sd, T, stream)

        def prefill_t(i, hh=th[0]):
            kv.paged_attn_prefill_chunk(hh, 0, q, w.Hq, cu, ctx_d, tables, w.max_blocks, w.B, T, n,
                                        int(ctx.max()), w.sm_scale(), out2, kv.DTYPE_BF16, stream)

        tt = _timed(prefill_t, args.steps, args.warmup, stream)
        types[name] = {"ms_mean": round(float(tt.mean()), 5),
                       "tflops": round(flops / (tt.mean() * 1e-3) / 1e12, 2),
                       "e4m3_speedup": round(float(tt.mean()) / pf_ms, 4)}
        kv.kv_cache_free(th[0])
        del tp
    res["element_types"] = types
    return res


def _cpu_prefill(w, oh, q, out, ctx, n, budget_s):
    """Oracle FLOP/s on sampled query rows, one thread and then all host cores
    (and the rows' parity with the GPU output); oh holds every sequence."""
    import oracle
    from synth import bf16_bits
    okp, ovp, ks, vs = oh.kp, oh.vp, oh.ks, oh.vs
    qb = bf16_bits(q)
    got = out.float().cpu().numpy()
    cu = (np.arange(w.B + 1) * n).astype(np.int32)
    rng = np.random.default_rng(11)
    rows = [(int(rng.integers(0, w.B * n)), int(rng.integers(0, w.Hq))) for _ in range(8192)]
    # The oracle takes a list of (row, head) pairs per call and returns a full-size
    # [rows][Hq][D] fp64 array (268 MB here): rows go 16 to a call and only the
    # selected outputs are copied out, so each call's array is released at once.
    per_call = 16
    calls = [rows[i:i + per_call] for i in range(0, len(rows), per_call)]

    def one(call):
        ref = oracle.prefill_attn(qb, okp, ovp, cu, ctx, oh.tables, Hq=w.Hq, Hkv=w.Hkv, D=w.D,
                                  BS=w.BS, k_scale=ks, v_scale=vs, sm_scale=w.sm_scale(),
                                  sel=np.array(call, np.int64))
        return [((r, hh), ref[r, hh].copy()) for r, hh in call]

    def flops(call):
        return sum(4 * w.D * (int(ctx[r // n]) + (r - (r // n) * n) + 1) for r, _ in call)

    results, (n1, t1), (n2, t2), threads = _timed_oracle(calls, one, budget_s)
    bad = 0
    for call_res in results:
        for (r, hh), ref in call_res:
            err = np.abs(got[r, hh] - ref)
            bad += int((err > 2e-3 + 1e-2 * np.abs(ref)).sum())
    f1 = sum(flops(c) for c in calls[:n1])
    f2 = sum(flops(c) for c in calls[n1:n1 + n2])
    return {"value": round(f2 / t2 / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n2 * per_call} random (query row, head) pairs, {per_call} per oracle call, on "
                      f"{threads} threads, fp64 C oracle (including the per-row dequantizing gather), "
                      f"{t2:.1f} s wall",
            "single_thread": {"value": round(f1 / t1 / 1e12, 6), "cores": 1,
                              "sample": f"{n1 * per_call} rows, {t1:.1f} s"},
            "parity_outside_tolerance": bad}


def run_longctx(args):
    """Long context + K-shift: 8 sequences x 131072 tokens, 16 q / 2 kv heads, head_dim 256,
    block 32, scales 0.03.  Step = decode, kv_shift_rope of every cached token by -4096
    (theta 1e6, NEOX), decode.  Roofline: the decode kernel against HBM."""
    import torch
    import fp8_e4m3_scaled_amd as kv
    from synth import Workload
    dev, stream = torch.device("cuda:0"), torch.cuda.current_stream()
    w = Workload("longctx", device=dev)
    copies = 3
    pools, handles = _fill(w, kv, dev, stream, copies=copies)
    lens = w.lengths.astype(np.int32)
    max_len = int(lens.max())
    q = w.q_decode(dev)
    tables = torch.from_numpy(w.block_tables.astype(np.int32)).to(dev)
    lens_d = torch.from_numpy(lens).to(dev)
    slots = torch.from_numpy(np.concatenate([w.slots(b, 0, int(lens[b])) for b in range(w.B)])).to(dev)
    nsl = int(slots.numel())
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.bfloat16, device=dev)
    ws_bytes = kv.paged_attn_decode_workspace(handles[0], w.B, w.Hq, max_len)
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=dev)

    def decode(i):
        kv.paged_attn_decode(handles[i % copies], 0, q, w.Hq, tables, w.max_blocks, lens_d, w.B, max_len,
                             w.sm_scale(), out, kv.DTYPE_BF16, ws, ws_bytes, stream)

    def shift(i):
        kv.kv_shift_rope(handles[i % copies], 0, slots, nsl, w.spec.delta, w.spec.theta, w.D,
                         kv.ROPE_NEOX, stream)

    # the same shift with a position delta per sequence (one table row each)
    seq_deltas = np.array([w.spec.delta - 512 * b for b in range(w.B)], np.int32)
    table = torch.from_numpy(kv.kv_rope_table(seq_deltas, w.spec.theta, w.D)).to(dev)
    rows = torch.from_numpy(np.repeat(np.arange(w.B, dtype=np.int32), lens.astype(np.int64))).to(dev)

    def shift_per_slot(i):
        kv.kv_shift_rope_per_slot(handles[i % copies], 0, slots, rows, nsl, table, w.B, w.D, kv.ROPE_NEOX,
                                  stream)

    # outputs for the parity sample, before the timed shifts turn the cached keys
    got = {}
    if args.cpu_seconds > 0:
        for name, dt, tdt in (("bf16", kv.DTYPE_BF16, torch.bfloat16), ("fp32", kv.DTYPE_F32, torch.float32)):
            o = torch.empty((w.B, w.Hq, w.D), dtype=tdt, device=dev)
            kv.paged_attn_decode(handles[0], 0, q, w.Hq, tables, w.max_blocks, lens_d, w.B, max_len,
                                 w.sm_scale(), o, dt, ws, ws_bytes, stream)
            torch.cuda.synchronize()
            got[name] = o.float().cpu().numpy()
    de = _timed(decode, args.steps, args.warmup, stream)
    sh = _timed(shift, args.steps, args.warmup, stream)
    sp = _timed(shift_per_slot, args.steps, args.warmup, stream)
    de_bytes = _decode_bytes(w, lens, 2)
    sh_bytes = nsl * (2 * w.Hkv * w.D + 8)
    de_gbps = de_bytes / (de.mean() * 1e-3) / 1e9
    sh_gbps = sh_bytes / (sh.mean() * 1e-3) / 1e9
    res = _header(args, "longctx", round(de_gbps, 1), "GB/s", float(2 * de.mean() + sh.mean()),
                  {"q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.D, "block_size": w.BS,
                   "num_seqs": w.B, "seq_len": max_len, "shift_delta": w.spec.delta,
                   "rope_theta": w.spec.theta, "out_dtype": "bf16", "decode_splits": ws_bytes > 0})
    res["decode"] = dict(_stats(de), algorithmic_bytes=de_bytes, GBps=round(de_gbps, 1),
                         frac_hbm_peak=round(de_gbps / HBM_PEAK_GBPS, 4),
                         tokens_per_s=round(w.B / (de.mean() * 1e-3), 1))
    res["kv_shift"] = dict(_stats(sh), algorithmic_bytes=sh_bytes, GBps=round(sh_gbps, 1),
                           frac_hbm_peak=round(sh_gbps / HBM_PEAK_GBPS, 4),
                           tokens_per_s=round(nsl / (sh.mean() * 1e-3), 1))
    sp_bytes = sh_bytes + nsl * 4
    sp_gbps = sp_bytes / (sp.mean() * 1e-3) / 1e9
    res["kv_shift_per_slot"] = dict(_stats(sp), algorithmic_bytes=sp_bytes, GBps=round(sp_gbps, 1),
                                    frac_hbm_peak=round(sp_gbps / HBM_PEAK_GBPS, 4), distinct_deltas=w.B,
                                    tokens_per_s=round(nsl / (sp.mean() * 1e-3), 1))
    res["kv_shift_pattern_ceiling"] = _kshift_ceiling(args, w, pools, slots, nsl, sh_bytes, stream)
    # the decode's tiles read with no compute, split into the decode's own chunks
    kv_bytes = int(np.sum(lens)) * 2 * w.Hkv * w.D
    res["paged_gather_ceiling"] = _gather_ceiling(args, kv, w, handles, tables, w.max_blocks, lens_d, w.B, w.Hkv,
                                                  kv_bytes, stream, chunk_blocks=4096 // w.BS)
    res["decode"]["frac_of_gather_ceiling"] = round(de_gbps / res["paged_gather_ceiling"]["GBps"], 4)
    dsha = _source_sha("decode.hip", "fp8_device.hpp", "decode_args.hpp")
    res["roofline"] = {"bound": "hbm", "achieved": round(de_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                       "frac": round(de_gbps / HBM_PEAK_GBPS, 4),
                       "traffic": _traffic_from_profile("decode_longctx_pmc.txt", dsha),
                       "kernel": "decode_kernel<256,32,1,1> + decode_reduce<256>", "kernel_source_sha": dsha}
    for h in handles:
        kv.kv_cache_free(h)
    del pools
    torch.cuda.empty_cache()
    if args.cpu_seconds > 0:
        ks, vs, _ = w.scales()
        oh = OracleHost(w, range(w.B), w.block_tables, lens, ks, vs, lambda b, lo, n: w.kv(b, lo, n, device=dev))
        cpu_de, res["parity_sample"] = _cpu_decode(w, oh, q, got, args.cpu_seconds)
        res["cpu_baseline"] = cpu_de
        res["cpu_baseline_ops"] = {"decode": cpu_de, "store": _cpu_store(w, oh, args.cpu_seconds / 2),
                                   "kv_shift": _cpu_kshift(w, oh, w.spec.delta, w.spec.theta, w.D,
                                                           args.cpu_seconds / 2)}
    return res


def run_varlen(args):
    """Variable-length decode: 256 sequences with lengths uniform in [512, 32768], 32 q / 8 kv
    heads, head_dim 128, block 16, bf16 scales, block tables drawn from a shuffled free list
    over a pool that is --pool-frac of 288 GB.  Step = kv_store_fp8 of one new token per
    sequence (at position L) + decode over L+1 tokens.  Roofline: the decode kernel."""
    import torch
    import fp8_e4m3_scaled_amd as kv
    from synth import Workload
    dev, stream = torch.device("cuda:0"), torch.cuda.current_stream()
    from synth import f32_to_bf16_bits
    w = Workload("varlen", device=dev, pool_frac=args.pool_frac)
    # The pool (its contents are never read outside the stored tokens), the
    # scales as bf16 bit patterns (KVF8_DTYPE_BF16), and block tables drawn by
    # the library's allocator from a shuffled free list over the whole pool.
    ks, vs, _ = w.scales()
    kp = torch.empty((w.NB, w.Hkv, w.BS * w.D), dtype=torch.uint8, device=dev)
    vp = torch.empty_like(kp)
    h = kv.kv_cache_alloc(1, w.NB, w.BS, w.Hkv, w.D, [f32_to_bf16_bits(float(ks))], [f32_to_bf16_bits(float(vs))],
                          kv.DTYPE_BF16, kp, vp)
    w.block_tables = _library_tables(kv, h, w, 1003)
    row = w.Hkv * w.D
    for b in range(w.B):
        Lb = int(w.lengths[b])
        for lo in range(0, Lb, 65536):
            n = min(65536, Lb - lo)
            k, v = w.kv(b, lo, n, device=dev)
            kv.kv_store_fp8(h, 0, k.reshape(n, row), v.reshape(n, row), row, row,
                            torch.from_numpy(w.slots(b, lo, n)).to(dev), n, stream)
    torch.cuda.synchronize()
    L = w.lengths
    K = torch.cat([w.kv(b, int(L[b]), 1, device=dev)[0].reshape(1, row) for b in range(w.B)])
    V = torch.cat([w.kv(b, int(L[b]), 1, device=dev)[1].reshape(1, row) for b in range(w.B)])
    sd = torch.from_numpy(np.concatenate([w.slots(b, int(L[b]), 1) for b in range(w.B)])).to(dev)
    lens = w.total_lengths.astype(np.int32)
    max_len = int(lens.max())
    q = w.q_decode(dev)
    tables = torch.from_numpy(w.block_tables.astype(np.int32)).to(dev)
    lens_d = torch.from_numpy(lens).to(dev)
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.bfloat16, device=dev)
    ws_bytes = kv.paged_attn_decode_workspace(h, w.B, w.Hq, max_len)
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=dev)

    def store(i):
        kv.kv_store_fp8(h, 0, K, V, row, row, sd, w.B, stream)

    def decode(i):
        kv.paged_attn_decode(h, 0, q, w.Hq, tables, w.max_blocks, lens_d, w.B, max_len, w.sm_scale(),
                             out, kv.DTYPE_BF16, ws, ws_bytes, stream)

    st = _timed(store, args.steps, args.warmup, stream)
    de = _timed(decode, args.steps, args.warmup, stream)
    out_f32 = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=dev)
    kv.paged_attn_decode(h, 0, q, w.Hq, tables, w.max_blocks, lens_d, w.B, max_len, w.sm_scale(), out_f32,
                         kv.DTYPE_F32, ws, ws_bytes, stream)
    torch.cuda.synchronize()
    de_bytes = _decode_bytes(w, lens, 2)
    de_gbps = de_bytes / (de.mean() * 1e-3) / 1e9
    res = _header(args, "varlen", round(de_gbps, 1), "GB/s", float(st.mean() + de.mean()),
                  {"q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.D, "block_size": w.BS,
                   "num_seqs": w.B, "max_seq_len": max_len, "mean_seq_len": float(lens.mean()),
                   "pool_blocks": int(w.NB), "pool_frac_of_288GB": args.pool_frac, "scale_dtype": "bf16",
                   "tables": "kv_block_shuffle + kv_block_alloc", "out_dtype": "bf16"})
    res["decode"] = dict(_stats(de), algorithmic_bytes=de_bytes, GBps=round(de_gbps, 1),
                         frac_hbm_peak=round(de_gbps / HBM_PEAK_GBPS, 4),
                         tokens_per_s=round(w.B / (de.mean() * 1e-3), 1))
    res["kv_store"] = dict(_stats(st), tokens=w.B, tokens_per_s=round(w.B / (st.mean() * 1e-3), 1))
    dsha = _source_sha("decode.hip", "fp8_device.hpp", "decode_args.hpp")
    res["roofline"] = {"bound": "hbm", "achieved": round(de_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                       "frac": round(de_gbps / HBM_PEAK_GBPS, 4),
                       "traffic": _traffic_from_profile("decode_varlen_pmc.txt", dsha),
                       "kernel": "decode_kernel<128,16,1,1> + decode_reduce<128>", "kernel_source_sha": dsha}
    # Beside the linear-stream ceiling: a plain read of the same tiles with one
    # workgroup per (sequence, kv-head) and no split, which the decode's split
    # plan beats on this length mix (long sequences would serialize).
    kv_bytes = int(lens.astype(np.int64).sum()) * 2 * w.Hkv * w.D
    res["stream_read_ceiling"] = _stream_ceiling(stream)
    res["decode"]["frac_of_stream_ceiling"] = round(de_gbps / res["stream_read_ceiling"]["GBps"], 4)
    res["paged_gather_unsplit"] = _gather_ceiling(args, kv, w, [h], tables, w.max_blocks, lens_d, w.B, w.Hkv,
                                                  kv_bytes, stream)
    res["decode"]["speedup_over_unsplit_gather"] = round(de_gbps / res["paged_gather_unsplit"]["GBps"], 4)
    # and split into the decode's own 4096-token chunks
    res["paged_gather_ceiling"] = _gather_ceiling(args, kv, w, [h], tables, w.max_blocks, lens_d, w.B, w.Hkv,
                                                  kv_bytes, stream, chunk_blocks=4096 // w.BS)
    res["decode"]["frac_of_gather_ceiling"] = round(de_gbps / res["paged_gather_ceiling"]["GBps"], 4)
    kv.kv_cache_free(h)
    del kp, vp
    torch.cuda.empty_cache()
    if args.cpu_seconds > 0:
        # the oracle holds the blocks of a seeded sample of the sequences (ids remapped)
        seqs = sorted(np.random.default_rng(12).choice(w.B, 24, replace=False).tolist())
        oh = OracleHost(w, seqs, w.block_tables, w.total_lengths, ks, vs, lambda b, lo, n: w.kv(b, lo, n, device=dev))
        got = {"bf16": out.float().cpu().numpy(), "fp32": out_f32.cpu().numpy()}
        cpu_de, res["parity_sample"] = _cpu_decode(w, oh, q, got, args.cpu_seconds)
        res["parity_sample"]["sequences"] = f"{len(seqs)} seeded sequences of {w.B}, ids as drawn from the {w.NB}-block pool"
        res["cpu_baseline"] = cpu_de
        res["cpu_baseline_ops"] = {"decode": cpu_de, "store": _cpu_store(w, oh, args.cpu_seconds / 2)}
    return res


def _library_tables(kv, handle, w, seed):
    """Block tables from the library's allocator: the free list shuffled with
    kv_block_shuffle(seed), then kv_block_alloc of each sequence's blocks."""
    kv.kv_block_shuffle(handle, seed)
    tables = np.zeros((w.B, w.max_blocks), np.int32)
    for b in range(w.B):
        n = -(-int(w.total_lengths[b]) // w.BS)
        tables[b, :n] = kv.kv_block_alloc(handle, n)
    return tables


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              f"(the path shards by kv-head or sequence with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    run = {"llama8b": run_llama8b, "prefill": run_prefill, "longctx": run_longctx,
           "varlen": run_varlen}[args.workload]
    print(json.dumps(run(args)), flush=True)


if __name__ == "__main__":
    main()
