"""Host-side pieces of bench.py: the GPU clock / power sampler's sysfs parsing
and the oracle-baseline sample sizing (no GPU needed)."""
import math
import os

import bench


def _fake_card(tmp_path, sclk, mclk, power_uw):
    dev = tmp_path / "device"
    (dev / "hwmon" / "hwmon0").mkdir(parents=True)
    (dev / "pp_dpm_sclk").write_text(sclk)
    (dev / "pp_dpm_mclk").write_text(mclk)
    (dev / "hwmon" / "hwmon0" / "power1_input").write_text(f"{power_uw}\n")
    return str(dev)


def test_sampler_reads_starred_levels_and_power(tmp_path):
    # the formats the amdgpu driver prints: an "S:" line for the current
    # shader clock when it sits between levels, else a starred level
    dev = _fake_card(tmp_path, "S: 2104Mhz *\n0: 500Mhz\n1: 2400Mhz\n", "0: 2000Mhz *\n", 250000000)
    smp = bench.GpuStateSampler()
    smp.dev = dev
    assert smp._read() == (2104.0, 2000.0, 250.0)
    dev2 = _fake_card(tmp_path / "b", "0: 500Mhz\n1: 2400Mhz *\n", "0: 1900Mhz *\n", 1)
    smp.dev = dev2
    assert smp._read() == (2400.0, 1900.0, 1e-6)


def test_sampler_summary(tmp_path):
    smp = bench.GpuStateSampler()
    smp.dev = "/x"
    smp.samples = [(2100.0, 2000.0, 900.0), (2400.0, 2000.0, 1000.0), (2300.0, 2000.0, 950.0)]
    s = smp.summary()
    assert s["samples"] == 3
    assert s["sclk_mhz"] == {"min": 2100.0, "median": 2300.0, "max": 2400.0}
    assert s["socket_power_w"]["median"] == 950.0
    smp.samples = []
    assert bench.GpuStateSampler.summary(smp)["samples"] == 0


def test_oracle_sample_stride_targets_a_bounded_sample():
    # FLUX joint: every 2nd of 144 blocks; Long T2V: 15 of 1024 blocks
    for (B, N, H), want in (((2, 4608, 24), 2), ((1, 32760, 40), 72)):
        nb = math.ceil(N / 32)
        stride = max(1, math.ceil(nb * 32.0 * N * B * H / bench.ORACLE_SAMPLE_PAIRS))
        assert stride == want
        rows = 32 * len(range(0, nb, stride))
        assert rows * N * B * H <= 1.1 * bench.ORACLE_SAMPLE_PAIRS


def test_host_info_fields():
    h = bench.host_info()
    assert set(h) == {"cpu_model", "logical_cpus", "usable_cpus"}
    assert h["usable_cpus"] >= 1 and h["logical_cpus"] >= h["usable_cpus"]


def test_sp_shards_cover_the_sequence():
    """The ranks' token ranges of `--sp P`: contiguous, disjoint, starting on
    multiples of 64, covering [0, N); ranks past the end hold nothing."""
    for N, P in ((32760, 8), (4608, 2), (3128, 3), (100, 2), (64, 4)):
        got = []
        for r in range(P):
            a, b = bench.sp_shard(N, P, r)
            if a >= N:
                continue
            assert a % 64 == 0 and a < b <= N
            got.append((a, b))
        assert got[0][0] == 0 and got[-1][1] == N
        assert all(x[1] == y[0] for x, y in zip(got, got[1:]))
    assert bench.sp_shard(32760, 8, 7) == (28672, 32760)


def test_attention_schedule_names():
    # the default is the interleaved schedule; 1 and 2 force a schedule
    assert [bench.attn_sch(w) for w in (4, 8)] == [1, 1]
    assert [bench.attn_sch(w, 1) for w in (4, 8)] == [0, 0]
    assert [bench.attn_sch(w, 2) for w in (4, 8)] == [1, 1]


def test_abba_variant_parsing():
    assert bench.parse_variant("default") == {}
    assert bench.parse_variant("producer=fused;streams=1") == {"producer": "fused", "streams": 1}
    assert bench.parse_variant("q-block=1;k_block=16") == {"q_block": 1, "k_block": 16}
    assert bench.parse_variant("qgroups=4") == {"qgroups": 4}
    import pytest
    for bad in ("waves=3", "producer=both", "streams=3", "k_block=32", "q_block", "qgroups=0", "qgroups=41"):
        with pytest.raises(SystemExit):
            bench.parse_variant(bad)
