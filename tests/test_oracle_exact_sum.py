"""Reading R3: the channel sums behind the K and V means are the correctly
rounded fp64 value of the exact sum, so the mean bits do not depend on any
summation order, also for channels where plain fp64 accumulation would lose
bits (a tiny value among O(1) values, heavy cancellation).

Pins: the oracle's exact summation against Python's math.fsum (a library
routine computing the same correctly rounded sum), and the K / V means of
constructed channels against closed forms."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def test_fsum_matches_math_fsum_random():
    rng = np.random.default_rng(11)
    for _ in range(400):
        n = int(rng.integers(1, 300))
        x = rng.standard_normal(n) * np.exp2(rng.integers(-60, 60, n))
        if rng.random() < 0.5:  # heavy cancellation
            x = np.concatenate([x, -x[: n // 2] * (1 + 2.0 ** -40)])
        rng.shuffle(x)
        assert oracle.fsum(x) == math.fsum(x)


def test_fsum_matches_math_fsum_bf16_channels():
    rng = np.random.default_rng(12)
    for _ in range(100):
        n = int(rng.integers(2, 5000))
        x = torch.from_numpy(rng.standard_normal(n) * 3).to(torch.bfloat16)
        # one to three tiny (some subnormal) values among O(1) ones
        for j in rng.integers(0, n, int(rng.integers(1, 4))):
            x[j] = float(2.0 ** -float(rng.integers(60, 133)))
        xd = x.double().numpy()
        assert oracle.fsum(xd) == math.fsum(xd)


def test_fsum_ties_and_specials():
    cases = [
        [],
        [0.0],
        [1.0, 2.0 ** -53],                  # tie, rounds to even (1.0)
        [1.0, 2.0 ** -53, 2.0 ** -106],     # beyond the tie: rounds up
        [1.0, 2.0 ** -53, -(2.0 ** -106)],  # short of the tie: rounds down
        [1.0 + 2.0 ** -52, 2.0 ** -53],     # tie, rounds to even (up)
        [1e300, 1e300, -1e300, -1e300, 1.0],
        [2.0 ** -1074, 2.0 ** -1074, -(2.0 ** -1073)],
    ]
    for c in cases:
        x = np.array(c, dtype=np.float64)
        assert oracle.fsum(x) == math.fsum(x), c


def _tiny_channel(N, tiny=2.0 ** -100):
    """Token 0: tiny, tokens 1..N-2: +1, -1, +1, ..., token N-1: 0 (N even):
    the exact sum is `tiny`, while an fp64 running sum that meets +1 after
    `tiny` loses it."""
    assert N % 2 == 0
    col = np.zeros(N)
    col[0] = tiny
    col[1:N - 1] = np.where(np.arange(N - 2) % 2 == 0, 1.0, -1.0)
    return col


def _bf16_bits(x32):
    return torch.tensor([x32], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).item() & 0xFFFF


@pytest.mark.parametrize("tiny", [2.0 ** -100, 2.0 ** -133])
def test_k_and_v_mean_of_a_tiny_value_among_ones(tiny):
    cfg = synth.custom(1, 4608, 2, 64, tag=402)
    q, k, v = synth.make_qkv(cfg)
    col = torch.from_numpy(_tiny_channel(cfg.N, tiny)).to(torch.bfloat16)
    assert float(col[0]) == tiny
    k[0, :, 1, 5] = col
    v[0, :, 1, 9] = col
    qk, vq = oracle.quant_qk(q, k), oracle.quant_v(v)
    # the plain ascending fp64 sum loses the tiny value; the channels are flagged
    assert sum(col.double().numpy().tolist()) == 0.0
    assert qk["inexact"] == 1 and vq["inexact"] == 1 and vq["bad"] == 0
    mean32 = np.float32(math.fsum(col.double().numpy()) / cfg.N)
    assert mean32 == np.float32(tiny / cfg.N)
    assert vq["v_mean"][0, 1, 9] == mean32
    assert qk["k_mean"][0, 1, 5] == _bf16_bits(float(mean32))
    if tiny == 2.0 ** -100:
        assert mean32 != 0 and qk["k_mean"][0, 1, 5] != 0


def test_exact_channels_unchanged():
    """Where plain fp64 accumulation is provably exact (every workload here),
    the rounded exact sum is that sum: means equal the ascending fp64 sum."""
    cfg = synth.custom(2, 300, 3, 64, tag=403)
    q, k, v = synth.make_qkv(cfg)
    qk, vq = oracle.quant_qk(q, k), oracle.quant_v(v)
    assert qk["inexact"] == 0 and vq["inexact"] == 0
    kd = k.double().numpy()
    vd = v.double().numpy()
    for (b, h, d) in [(0, 0, 0), (1, 2, 63), (0, 1, 17)]:
        s = 0.0
        for n in range(cfg.N):
            s += kd[b, n, h, d]
        assert qk["k_mean"][b, h, d] == _bf16_bits(float(np.float32(s / cfg.N)))
        s = 0.0
        for n in range(cfg.N):
            s += vd[b, n, h, d]
        assert vq["v_mean"][b, h, d] == np.float32(s / cfg.N)
