"""The benchmark's measurement kernels (libmoe_probes.so) do the work they are timed on.

Streaming read: the XOR of the words it writes equals the XOR of every 32-bit word of the
buffer, for every variant (loads per lane, cache policy) and grid shape the benchmark times,
including looping grids and sizes that leave a ragged last round.  MFMA throughput: every
wave's sums equal their exact value (known operands, integer results below 2^24), so no
instruction was dropped, for both kinds and every grid the benchmark times."""
from __future__ import annotations

import ctypes as C
import os
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


@pytest.mark.parametrize("nbytes", [16, 4096 + 16 * 3, 58556416, 1 << 26])
def test_stream_read_covers_every_byte(nbytes):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench
    L = bench.probes()
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    want = np.bitwise_xor.reduce(host)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.empty(4 * (1 << 19), dtype=torch.int32, device="cuda")
    for v in range(L.moe_probe_stream_read_variants()):
        for max_groups in (1 << 19, 256 * 8, 256 * 2, 3):
            groups = int(L.moe_probe_stream_read_groups(nbytes, v, max_groups))
            sink.zero_()
            rc = L.moe_probe_stream_read(C.c_void_p(buf.data_ptr()), nbytes, v, groups, C.c_void_p(sink.data_ptr()),
                                         C.c_void_p(torch.cuda.current_stream().cuda_stream))
            assert rc == 0
            torch.cuda.synchronize()
            got = np.bitwise_xor.reduce(sink[:4 * groups].cpu().numpy().view(np.uint32))
            assert got == want, (nbytes, v, groups)


@pytest.mark.parametrize("kind", [0, 1], ids=["f16_16x16x32", "fp4_16x16x128"])
@pytest.mark.parametrize("groups,iters", [(1, 1), (3, 37), (256 * 4, 64), (256 * 16, 8192)])
def test_mfma_probe_sums_are_exact(kind, groups, iters):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench
    L = bench.probes()
    want = L.moe_probe_mfma_expected_sink(kind, iters)
    sink = torch.full((groups * 4,), -1.0, dtype=torch.float32, device="cuda")
    rc = L.moe_probe_mfma_peak(kind, groups, iters, C.c_void_p(sink.data_ptr()),
                               C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    got = sink.cpu().numpy()
    assert np.all(got == np.float32(want)), (kind, groups, iters, want, np.unique(got)[:4])


def test_mfma_probe_refuses_bad_launches():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench
    L = bench.probes()
    sink = torch.empty(4, dtype=torch.float32, device="cuda")
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    for kind, groups, iters in ((2, 1, 1), (0, 0, 1), (0, 1, 0), (0, 1, 8193)):
        assert L.moe_probe_mfma_peak(kind, groups, iters, C.c_void_p(sink.data_ptr()), stream) != 0
    assert L.moe_probe_mfma_peak(0, 1, 1, None, stream) != 0
