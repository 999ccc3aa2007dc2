"""GPU check of the streaming-read measurement aid: the XOR of the per-workgroup
words must equal the XOR of every 32-bit word of the buffer (so every byte was
read), for several sizes and worker counts, including a buffer smaller than one
grid pass and one that is not a multiple of the unrolled stride."""
import numpy as np
import pytest
import torch

import fp8_e4m3_scaled_amd as kv
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
    kv.kvf8_read_probe(buf, nbytes, out, n_out)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(host))
