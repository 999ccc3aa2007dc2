"""Host-side checks of the benchmark's measurement probes (probe/, a library
of its own, outside the kvfp8 library): every bad argument is refused before
anything is launched; empty work is a no-op.  No GPU is touched."""
import pytest

import probe

E_INVALID = 1


def test_read_probe_host_checks():
    """The streaming read refuses misaligned or ragged buffers and bad worker
    counts before launching anything; zero bytes is a no-op."""
    probe.read(None, 0, None, 1, 0)
    for buf, nbytes, n_out in [((1 << 30) + 4, 64, 8), (1 << 30, 60, 8), (1 << 30, 64, 0),
                               (1 << 30, 64, (1 << 20) + 1)]:
        with pytest.raises(probe.ProbeError) as ei:
            probe.read(buf, nbytes, 1 << 30, n_out, 0)
        assert ei.value.status == E_INVALID
    with pytest.raises(probe.ProbeError) as ei:
        probe.read(1 << 30, 64, None, 8, 0)
    assert ei.value.status == E_INVALID


def test_gather_probe_host_checks():
    """The paged-gather read refuses bad shapes, element sizes and NULL
    pointers; no sequences is a no-op."""
    K, V, T, L, O = 1 << 33, 1 << 34, 1 << 35, 1 << 36, 1 << 37
    good = dict(k=K, v=V, nb=8, h=2, bs=16, d=64, keb=1, veb=1, t=T, mb=4, l=L, n=2, o=O)
    probe.gather(None, None, 8, 2, 16, 64, 1, 1, None, 4, None, 0, None, 0)
    bad = [dict(nb=0), dict(h=0), dict(bs=8), dict(d=96), dict(keb=3), dict(veb=0), dict(mb=-1), dict(n=-1),
           dict(k=None), dict(v=None), dict(t=None), dict(l=None), dict(o=None)]
    for change in bad:
        a = {**good, **change}
        with pytest.raises(probe.ProbeError) as ei:
            probe.gather(a["k"], a["v"], a["nb"], a["h"], a["bs"], a["d"], a["keb"], a["veb"], a["t"], a["mb"],
                         a["l"], a["n"], a["o"], 0)
        assert ei.value.status == E_INVALID, change
    for change in bad + [dict(cb=0), dict(cb=-3)]:
        a = {**good, "cb": 2, **change}
        with pytest.raises(probe.ProbeError) as ei:
            probe.gather_split(a["k"], a["v"], a["nb"], a["h"], a["bs"], a["d"], a["keb"], a["veb"], a["t"],
                               a["mb"], a["l"], a["n"], a["cb"], a["o"], 0)
        assert ei.value.status == E_INVALID, change


def test_rmw_probe_host_checks():
    """The K-shift traffic probe refuses bad shapes, rotary widths off the run
    path, negative counts and NULL pointers; no slots is a no-op."""
    K, S = 1 << 33, 1 << 34
    good = dict(k=K, nb=8, h=2, bs=16, d=64, rot=64, s=S, n=5)
    probe.rmw(None, 8, 2, 16, 64, 64, None, 0, 0)
    bad = [dict(nb=0), dict(h=0), dict(bs=8), dict(d=96), dict(rot=16), dict(rot=48), dict(rot=128), dict(n=-1),
           dict(k=None), dict(s=None)]
    for change in bad:
        a = {**good, **change}
        with pytest.raises(probe.ProbeError) as ei:
            probe.rmw(a["k"], a["nb"], a["h"], a["bs"], a["d"], a["rot"], a["s"], a["n"], 0)
        assert ei.value.status == E_INVALID, change


def test_store_copy_probe_host_checks():
    """The fill traffic probe refuses bad shapes, short or ragged strides,
    misaligned buffers and NULL pointers; no tokens is a no-op."""
    K, V, S, KP, VP = 1 << 33, 1 << 34, 1 << 35, 1 << 36, 1 << 37
    good = dict(k=K, v=V, ks=256, vs=256, s=S, n=32, kp=KP, vp=VP, nb=8, h=2, bs=16, d=128)
    probe.store_copy(None, None, 256, 256, None, 0, None, None, 8, 2, 16, 128, 0)
    bad = [dict(nb=0), dict(h=0), dict(bs=8), dict(d=96), dict(n=-1), dict(ks=128), dict(vs=260),
           dict(k=None), dict(v=None), dict(s=None), dict(kp=None), dict(vp=None), dict(k=K + 8), dict(vp=VP + 4)]
    for change in bad:
        a = {**good, **change}
        with pytest.raises(probe.ProbeError) as ei:
            probe.store_copy(a["k"], a["v"], a["ks"], a["vs"], a["s"], a["n"], a["kp"], a["vp"], a["nb"], a["h"],
                             a["bs"], a["d"], 0)
        assert ei.value.status == E_INVALID, change
