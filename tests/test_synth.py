"""The seeded generator: deterministic, thread-count independent, and shaped
like the stated workloads."""
import hashlib
import os
import subprocess
import sys

import numpy as np

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _digest(cfg_idx):
    h = hashlib.sha256()
    for which in ("q", "k", "v"):
        h.update(synth.fill_f32(synth.config(cfg_idx), which).tobytes())
    return h.hexdigest()


def test_deterministic_and_thread_independent():
    a = _digest(0)
    assert a == _digest(0)
    code = "import synth; import tests.test_synth as t; print(t._digest(0))"
    env = dict(os.environ, OMP_NUM_THREADS="1", PYTHONPATH=ROOT)
    out = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True,
                         text=True, check=True).stdout.strip()
    assert out == a


def test_streams_differ():
    c = synth.config(0)
    q, k = synth.fill_f32(c, "q"), synth.fill_f32(c, "k")
    assert not np.array_equal(q, k)
    assert not np.array_equal(synth.fill_f32(synth.config(1), "v")[0, :256, 0, :64].ravel(),
                              synth.fill_f32(c, "v")[0, :256, 0, :].ravel())


def test_moments_and_offsets():
    c = synth.config(1)
    q = synth.fill_f32(c, "q").astype(np.float64)
    out = synth.outlier_channels(c)
    assert out.size == 31 and np.unique(out).size == 31
    flat = q.reshape(-1, c.H * c.D)
    normal = np.setdiff1d(np.arange(c.H * c.D), out)
    assert abs(flat[:, normal].std() - 1.0) < 0.01
    assert abs(flat[:, out].std() - 8.0) < 0.2
    v = synth.fill_f32(c, "v").astype(np.float64).reshape(-1, c.H * c.D)
    # per-channel means ~ N(0,1) offsets, within-channel std 1
    assert abs(v.mean(0).std() - 1.0) < 0.1 and abs(v.std(0).mean() - 1.0) < 0.01
    k = synth.fill_f32(c, "k").astype(np.float64).reshape(-1, c.H * c.D)
    assert abs(k.mean(0).std() - np.sqrt(3.0)) < 0.15


def test_query_subset():
    rows = synth.query_subset(3128)
    assert rows[0] == 0 and rows[-1] == 3127 and np.all(np.diff(rows) > 0)
    assert 3128 // 9 < rows.size < 3128 // 7
