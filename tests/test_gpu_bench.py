"""bench.py end to end on the tiny workload (B1 H2 N256 D64), eager and with
--graph: one JSON line with the contract's keys, and per-call times that are
positive, finite and within the step time.  Under --graph the attention's
times come from event-record nodes added to the captured graph through the
HIP graph API, so this also checks that those nodes record on every replay.
Runs bench.py in a child process (one GPU process at a time)."""
import json
import math
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("graph", [False, True], ids=["eager", "graph"])
def test_bench_tiny(graph):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--steps", "5",
           "--warmup", "3", "--no-cpu-baseline", "--gpu-state-seconds", "0"] + (["--graph"] if graph else [])
    print("[bench]", " ".join(cmd[1:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    line = r.stdout.strip().splitlines()[-1]
    d = json.loads(line)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in d
    assert d["config"]["graph"] is graph
    assert d["steps"] == 5 and d["n_gpus"] == 1
    assert math.isfinite(d["value"]) and d["value"] > 0
    att = d["kernels_ms"]["attn_fwd"]
    assert 0 < att["min"] <= att["median"] <= att["p90"]
    assert att["avg"] <= 5 * d["ms_per_step"]
    assert 0 < d["roofline"]["frac"] < 1
    print(f"  step {d['ms_per_step']} ms, attention {att['avg']} ms, kernels {sorted(d['kernels_ms'])}",
          flush=True)


def _run_bench(args):
    cmd = [sys.executable, os.path.join(ROOT, "bench.py")] + args
    print("[bench]", " ".join(cmd[1:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    return json.loads(r.stdout.strip().splitlines()[-1])


def test_bench_parts():
    """The metric's other parts in the same JSON line: an attention part and a
    quant-only part, each with its own roofline and pre-warm record."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    d = _run_bench(["--workload", "tiny", "--parts", "tiny,quant_long", "--steps", "3", "--warmup", "1",
                    "--prewarm-ms", "20", "--no-cpu-baseline", "--gpu-state-seconds", "0"])
    assert d["prewarm"]["steps"] >= 4
    assert set(d["parts"]) == {"tiny", "quant_long"}
    pa, pq = d["parts"]["tiny"], d["parts"]["quant_long"]
    assert pa["unit"] == "TFLOPS" and 0 < pa["roofline"]["frac"] < 1 and pa["roofline"]["bound"] == "mfma"
    assert pq["unit"] == "GB/s" and pq["roofline"]["bound"] == "hbm" and pq["config"]["streams"] == 1
    assert 0 < pq["roofline"]["frac"] < 1 and 0 < pq["roofline_quant_v"]["frac"] < 1
    print(f"  parts: tiny {pa['ms_per_step']} ms, quant_long {pq['quant_qk_gbs']} / {pq['quant_v_gbs']} GB/s",
          flush=True)


def test_bench_abba():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    d = _run_bench(["--workload", "tiny", "--abba", "streams=1,streams=2", "--abba-groups", "3", "--steps", "3",
                    "--warmup", "1", "--prewarm-ms", "20"])
    assert d["mode"] == "abba" and d["A"]["streams"] == 1 and d["B"]["streams"] == 2
    assert len(d["per_group"]) == 3
    assert all(g["A_step_ms"] > 0 and g["B_step_ms"] > 0 for g in d["per_group"])
    assert d["median_ratio_step"] > 0
    print(f"  ABBA streams 1 vs 2 on tiny: step ratio {d['median_ratio_step']}", flush=True)
