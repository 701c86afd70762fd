"""Issue rates of the instructions that bound the attention kernel's key step,
measured on the GPU (tests/issue_probe.hip): cycles per wave64 instruction per
SIMD, with one and with two waves per SIMD (the attention runs two).

The per-tile cycle budget of the attention (per 64-key tile and wave: 8 INT8
32x32x32 and 4 FP8 32x32x64 MFMAs; 32 int-to-float conversions, 32 FMAs, 33
exp2, 32 adds and 16 FP8 packs on the vector ALU) takes its instruction costs
from this probe; the assertions pin the relations it relies on: the two MFMA
shapes cost their nominal 32 and 64 cycles, and exp2 and the FP8 pack cost
well over an FMA."""
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
    from tests import issue_probe
    return issue_probe, issue_probe.load()


def _cycles(lib, op, per_iter, waves, iters, cus):
    seed = torch.linspace(-1.0, 1.0, 64, dtype=torch.float32, device="cuda")
    nwaves = cus * 4 * waves
    cyc = torch.zeros(nwaves, dtype=torch.int64, device="cuda")
    sink = torch.empty(nwaves * 64, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    for _ in range(2):  # the first run warms the clock and the code
        st = lib.probe_issue(op, cus, waves, iters, seed.data_ptr(), cyc.data_ptr(), sink.data_ptr())
        assert st == 0, st
    # the waves sharing a SIMD need not progress evenly (one can finish first
    # and its partner run on alone), so a SIMD's time is its slowest wave's:
    # per workgroup (one per CU) the slowest wave, then the median over CUs
    slowest = cyc.view(cus, 4 * waves).max(dim=1).values.cpu().tolist()
    return statistics.median(slowest) / (iters * per_iter) / waves


def test_issue_rates(probe):
    mod, lib = probe
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rates = {}
    for waves in (1, 2):
        for op, (name, per_iter) in mod.OPS.items():
            iters = 1024 if op >= 4 else 4096
            _log(f"[issue] {name} waves/SIMD {waves}")
            rates[(op, waves)] = _cycles(lib, op, per_iter, waves, iters, cus)
    _log("cycles per wave64 instruction per SIMD (1 / 2 waves per SIMD):")
    for op, (name, _) in mod.OPS.items():
        _log(f"  {name:36s} {rates[(op, 1)]:6.2f} {rates[(op, 2)]:6.2f}")
    for w in (1, 2):
        assert 24 <= rates[(4, w)] <= 48       # INT8 32x32x32: 32 cycles
        assert 48 <= rates[(5, w)] <= 96       # FP8 32x32x64: 64 cycles
        assert 1.6 <= rates[(5, w)] / rates[(4, w)] <= 2.4
    # at the attention's two waves per SIMD, exp2 and the FP8 pack each cost
    # well over an FMA, and the conversion at least about as much as an FMA
    assert rates[(2, 2)] >= 1.5 * rates[(0, 2)]
    assert rates[(3, 2)] >= 1.5 * rates[(0, 2)]
    assert rates[(1, 2)] >= 0.8 * rates[(0, 2)]


def test_matrix_and_vector_waves_overlap(probe):
    """One SIMD's two waves, one running only FP8 MFMAs and one only a vector
    instruction (each sized to take about as long alone as the other): how
    much of the shorter one the pair hides.  In the attention each wave mixes
    both units; its counters show 0.57-0.63 of the MFMA-busy cycles overlapped."""
    mod, lib = probe
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    iters_m = 1024
    t_m = _cycles(lib, 5, 4, 1, iters_m, cus) * iters_m * 4       # one wave per SIMD, alone
    seed = torch.linspace(-1.0, 1.0, 64, dtype=torch.float32, device="cuda")
    cyc = torch.zeros(cus * 8, dtype=torch.int64, device="cuda")
    sink = torch.empty(cus * 8 * 64, dtype=torch.float32, device="cuda")
    hidden = {}
    for vop in (0, 1, 2, 3):
        name = mod.OPS[vop][0]
        per = _cycles(lib, vop, 8, 1, 4096, cus)
        iters_v = max(1, int(t_m / (8 * per)))
        t_v = per * iters_v * 8
        for _ in range(2):
            st = lib.probe_pair(vop, cus, iters_m, iters_v, seed.data_ptr(), cyc.data_ptr(), sink.data_ptr())
            assert st == 0, st
        both = statistics.median(cyc.view(cus, 8).max(dim=1).values.cpu().tolist())
        hidden[name] = (t_m + t_v - both) / min(t_m, t_v)
        _log(f"MFMA-only wave alone {t_m:.0f} cycles, {name}-only wave alone {t_v:.0f}, the pair {both:.0f}: "
             f"{100 * hidden[name]:.0f}% of the shorter one hidden")
        # side by side, not one after the other
        assert both <= 0.8 * (t_m + t_v)
