"""What HBM delivers to the quantisers' access pattern, measured cold.

The quantisers are judged against the published 8 TB/s.  This test measures
the read rate plain kernels reach on the quant-only tensor (B1 N32760 H40
D128 bf16, 335 MB): with the statistics pass's pattern (one head's 256-byte
row slices, 10 KB apart) and as one contiguous stream, each launch preceded by
a 1 GiB read so the tensor is not in the last-level cache.  It prints the
rates; the bounds asserted are only sanity bounds (the figures are the
result)."""
import statistics
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu


def _log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import hbm_probe
    return hbm_probe.load()


def test_cold_read_rates(probe):
    N, H, D = 32760, 40, 128
    dev = torch.device("cuda")
    x = torch.ones((N, H, D), dtype=torch.bfloat16, device=dev)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    out = torch.empty(1 << 22, dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    nbytes = x.numel() * 2

    def cold(launch):
        ts = []
        for i in range(12):
            assert probe.probe_read_flat(flush.data_ptr(), flush.numel() * 4, 2048, out.data_ptr(), s) == 0
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            assert launch() == 0
            e1.record()
            torch.cuda.synchronize()
            if i >= 2:
                ts.append(e0.elapsed_time(e1) * 1e3)
        return statistics.median(ts)

    rates = {}
    for nchunk in (26, 52):
        assert nchunk * H * 256 <= out.numel()
        us = cold(lambda: probe.probe_read_rows(x.data_ptr(), N, H, nchunk, out.data_ptr(), s))
        rates[f"head row slices, {nchunk * H} workgroups"] = (us, nbytes / us / 1e6)
    for wgs in (1024, 2048):
        us = cold(lambda: probe.probe_read_flat(x.data_ptr(), nbytes, wgs, out.data_ptr(), s))
        rates[f"contiguous, {wgs} workgroups"] = (us, nbytes / us / 1e6)
    for k, (us, tbs) in rates.items():
        _log(f"  cold read of {nbytes / 1e6:.1f} MB, {k}: {us:.1f} us, {tbs:.2f} TB/s")
    for us, tbs in rates.values():
        assert 1.0 < tbs < 8.0
