"""GPU checks of the measurement aids: the streaming read's per-workgroup XOR
words must XOR to the XOR of every 32-bit word of the buffer (so every byte
was read), for several sizes and worker counts, including a buffer smaller
than one grid pass and one that is not a multiple of the unrolled stride; the
paged-gather read covers exactly a decode's tiles; the K-shift traffic probe
touches exactly the K-shift's bytes, and the fill traffic probe writes exactly
where the store writes, for whole aligned 16-token runs only."""
import numpy as np
import pytest
import torch

import fp8_e4m3_scaled_amd as kv
import probe
from tests.gpu_util import DEV, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,n_out", [(16, 1), (4096, 7), (1 << 20, 64), ((64 << 20) + 48, 2048),
                                          ((256 << 20) + 16 * 999, 1024)])
def test_read_probe_xor(nbytes, n_out):
    log(f"read probe bytes={nbytes} n_out={n_out}")
    rng = np.random.default_rng(nbytes % 9973 + n_out)
    host = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(DEV)
    out = torch.full((n_out,), -1, dtype=torch.int32, device=DEV)
    probe.read(buf, nbytes, out, n_out)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(host))


@pytest.mark.parametrize("BS,Hkv,D,v_elem", [(16, 2, 64, kv.ELEM_E4M3), (32, 3, 256, kv.ELEM_E4M3),
                                              (16, 8, 128, kv.ELEM_BF16)])
def test_gather_probe_xor(BS, Hkv, D, v_elem):
    """The paged-gather measurement read covers exactly the decode's tiles: per
    (sequence, kv-head), the XOR of every word of the K and V tiles of the
    sequence's blocks, including an empty sequence and a partial last block."""
    rng = np.random.default_rng(BS + Hkv + D + v_elem)
    lens = np.array([0, 1, 17, 100, 3 * BS], np.int32)
    NB = 40
    max_blocks = 8
    tables = rng.permutation(NB)[:lens.size * max_blocks].reshape(lens.size, max_blocks).astype(np.int32)
    veb = 2 if v_elem == kv.ELEM_BF16 else 1
    tile_k, tile_v = BS * D, BS * D * veb
    kp = rng.integers(0, 1 << 32, size=NB * Hkv * tile_k // 4, dtype=np.uint32)
    vp = rng.integers(0, 1 << 32, size=NB * Hkv * tile_v // 4, dtype=np.uint32)
    k_dev = torch.from_numpy(kp.view(np.int32)).to(DEV)
    v_dev = torch.from_numpy(vp.view(np.int32)).to(DEV)
    out = torch.full((lens.size * Hkv,), -1, dtype=torch.int32, device=DEV)
    probe.gather(k_dev, v_dev, NB, Hkv, BS, D, 1, veb, torch.from_numpy(tables).to(DEV), max_blocks,
                 torch.from_numpy(lens).to(DEV), lens.size, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    kt = kp.reshape(NB, Hkv, tile_k // 4)
    vt = vp.reshape(NB, Hkv, tile_v // 4)
    for b, L in enumerate(lens):
        blocks = tables[b, :-(-int(L) // BS)] if L > 0 else tables[b, :0]
        for hh in range(Hkv):
            want = np.uint32(0)
            if blocks.size:
                want = np.bitwise_xor.reduce(np.concatenate([kt[blocks, hh].ravel(), vt[blocks, hh].ravel()]))
            assert int(got[b * Hkv + hh]) == int(want), (b, hh)


@pytest.mark.parametrize("chunk", [1, 3, 8])
def test_gather_split_probe_xor(chunk):
    """The split read covers, per (chunk, sequence, kv-head), exactly that
    chunk of the sequence's table entries: the XOR of their K and V tiles
    (0 for chunks past the sequence's blocks)."""
    rng = np.random.default_rng(7 + chunk)
    BS, Hkv, D = 32, 2, 256
    lens = np.array([0, 1, 33, 200, 8 * BS], np.int32)
    NB, max_blocks = 48, 8
    tables = rng.permutation(NB)[:lens.size * max_blocks].reshape(lens.size, max_blocks).astype(np.int32)
    tile = BS * D
    kp = rng.integers(0, 1 << 32, size=NB * Hkv * tile // 4, dtype=np.uint32)
    vp = rng.integers(0, 1 << 32, size=NB * Hkv * tile // 4, dtype=np.uint32)
    chunks = -(-max_blocks // chunk)
    log(f"gather split probe chunk={chunk}")
    out = torch.full((chunks * lens.size * Hkv,), -1, dtype=torch.int32, device=DEV)
    probe.gather_split(torch.from_numpy(kp.view(np.int32)).to(DEV), torch.from_numpy(vp.view(np.int32)).to(DEV), NB,
                       Hkv, BS, D, 1, 1, torch.from_numpy(tables).to(DEV), max_blocks, torch.from_numpy(lens).to(DEV),
                       lens.size, chunk, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    kt, vt = kp.reshape(NB, Hkv, tile // 4), vp.reshape(NB, Hkv, tile // 4)
    for c in range(chunks):
        for b, L in enumerate(lens):
            nblk = min(-(-int(L) // BS), max_blocks)
            blocks = tables[b, c * chunk:min(nblk, (c + 1) * chunk)] if nblk > c * chunk else tables[b, :0]
            for hh in range(Hkv):
                want = np.uint32(0)
                if blocks.size:
                    want = np.bitwise_xor.reduce(np.concatenate([kt[blocks, hh].ravel(), vt[blocks, hh].ravel()]))
                assert int(got[(c * lens.size + b) * Hkv + hh]) == int(want), (c, b, hh)


@pytest.mark.parametrize("BS,Hkv,D,rot", [(16, 2, 64, 64), (32, 2, 256, 256), (16, 3, 128, 64), (16, 1, 64, 32)])
def test_rmw_probe_touches_the_kshift_bytes(BS, Hkv, D, rot):
    """One pass flips bit 0 of exactly the rotated bytes (dims [0, rot)) of the
    listed in-pool slots in every kv-head and nothing else; a second pass
    restores the pool."""
    rng = np.random.default_rng(BS + Hkv + D + rot)
    NB = 9
    pool = rng.integers(0, 256, size=(NB, Hkv, BS * D), dtype=np.uint8)
    slots = rng.choice(NB * BS, size=NB * BS // 2, replace=False).astype(np.int64)
    slots = np.concatenate([slots, [-1, NB * BS, NB * BS + 5]])
    rng.shuffle(slots)
    log(f"rmw probe BS={BS} Hkv={Hkv} D={D} rot={rot}")
    dev = torch.from_numpy(pool).to(DEV)
    sd = torch.from_numpy(slots).to(DEV)
    probe.rmw(dev, NB, Hkv, BS, D, rot, sd, slots.size)
    torch.cuda.synchronize()
    once = dev.cpu().numpy()
    want = pool.copy()
    q = D // 4
    for s in slots:
        if s < 0 or s >= NB * BS:
            continue
        b, t = divmod(int(s), BS)
        for d in range(rot):
            want[b, :, (d // q) * BS * q + t * q + d % q] ^= 1
    assert np.array_equal(once, want)
    probe.rmw(dev, NB, Hkv, BS, D, rot, sd, slots.size)
    torch.cuda.synchronize()
    assert np.array_equal(dev.cpu().numpy(), pool)


@pytest.mark.parametrize("BS,Hkv,D", [(16, 2, 64), (32, 3, 128), (16, 1, 256)])
def test_store_copy_probe_writes_the_store_positions(BS, Hkv, D):
    """Groups of 16 tokens bound for an aligned run of 16 slots get each bf16
    value's high byte at the byte the store's layout gives that (token, dim);
    a group whose run is broken, one whose run is not aligned, one past the
    pool and a short last group leave the pools untouched."""
    rng = np.random.default_rng(BS + Hkv + D)
    NB = 8
    row = Hkv * D
    stride = row + 8
    runs = [np.arange(16 * i, 16 * i + 16) for i in (3, 0, 5)]                   # whole aligned runs
    broken = np.arange(16 * 6, 16 * 6 + 16)[::-1]                               # reversed
    shifted = np.arange(16 * 1 + 8, 16 * 1 + 24)                                # not aligned
    past = np.arange(NB * BS, NB * BS + 16)                                     # outside the pool
    short = np.arange(16 * 7, 16 * 7 + 5)                                       # last, partial
    slots = np.concatenate(runs + [broken, shifted, past, short]).astype(np.int64)
    n = slots.size
    kb = rng.integers(0, 1 << 16, size=(n, stride), dtype=np.uint16)
    vb = rng.integers(0, 1 << 16, size=(n, stride), dtype=np.uint16)
    log(f"store copy probe BS={BS} Hkv={Hkv} D={D}")
    kp = torch.zeros((NB, Hkv, BS * D), dtype=torch.uint8, device=DEV)
    vp = torch.zeros_like(kp)
    probe.store_copy(torch.from_numpy(kb.view(np.int16)).to(DEV), torch.from_numpy(vb.view(np.int16)).to(DEV),
                     stride, stride, torch.from_numpy(slots).to(DEV), n, kp, vp, NB, Hkv, BS, D)
    torch.cuda.synchronize()
    want_k = np.zeros((NB, Hkv, BS * D), np.uint8)
    want_v = np.zeros_like(want_k)
    q = D // 4
    d = np.arange(D)
    for i in range(3 * 16):
        b, t = divmod(int(slots[i]), BS)
        for h in range(Hkv):
            want_k[b, h, ((d // q) * BS + t) * q + d % q] = (kb[i, h * D + d] >> 8).astype(np.uint8)
            want_v[b, h, ((t // 4) * D + d) * 4 + t % 4] = (vb[i, h * D + d] >> 8).astype(np.uint8)
    assert np.array_equal(kp.cpu().numpy(), want_k)
    assert np.array_equal(vp.cpu().numpy(), want_v)
