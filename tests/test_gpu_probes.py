"""The two measurement probes the benchmarks time for their ceilings: the read stream must
read every 16-byte unit exactly once (its checksums add up to the host's sum over the
units, wrapping at 2^32, whatever the grid), and the matrix-rate probe must run to the end
and give the same finite accumulators on every call."""
import numpy as np
import pytest
import torch

import invariant_numerics_amd as inv
from gpu_util import requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]


@pytest.mark.parametrize("nbytes,grid", [(16, 1), (4096 * 16, 7), ((1 << 22) + 48, 300), ((1 << 24) + 16 * 1013, 4096)])
def test_read_stream_reads_every_unit_once(nbytes, grid):
    say(f"[case] read stream {nbytes} bytes grid {grid}")
    rng = np.random.default_rng(nbytes % 9973 + grid)
    words = rng.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    sink = inv.inv_read_stream_probe(src, grid=grid)
    got = int(sink.cpu().numpy().view(np.uint32).astype(np.uint64).sum()) % (1 << 32)
    u = words.reshape(-1, 4)
    want = int((u[:, 0] ^ u[:, 1] ^ u[:, 2] ^ u[:, 3]).astype(np.uint64).sum()) % (1 << 32)
    assert got == want


@pytest.mark.parametrize("shape", [0, 1])
def test_mfma_rate_probe_runs_and_repeats(shape):
    say(f"[case] mfma rate probe shape {shape}")
    a = inv.inv_mfma_rate_probe(shape, 50, 8).cpu().numpy()
    b = inv.inv_mfma_rate_probe(shape, 50, 8).cpu().numpy()
    assert a.shape == (512 * 256,)
    assert np.isfinite(a).all() and (a != 0).all()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
