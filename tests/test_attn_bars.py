"""CPU checks of the attention bars in tests/attn_bars.py: they pass the
oracle against itself plus bf16 output rounding, and fail on mistakes planted
in a copy of the oracle's output (one wrong head, one bad tail row, a scaled
attention term, NaN)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.attn_bars import attention_report, bf16_half_ulp, check_attention


@pytest.fixture(scope="module")
def case():
    cfg = synth.custom(2, 200, 3, 64, tag=401)
    q, k, v = synth.make_qkv(cfg)
    qk, vq = oracle.quant_qk(q, k), oracle.quant_v(v)
    tiled = oracle.attn_tiled(qk, vq)
    return tiled, vq["v_mean"]


def _bf16(x):
    return torch.from_numpy(x).float().to(torch.bfloat16).double().numpy()


def test_half_ulp():
    x = np.array([1.0, 1.5, -3.0, 2.0 ** -130, 0.0])
    h = bf16_half_ulp(x)
    assert h[0] == 2.0 ** -8 * (1 + 2.0 ** -7) and h[1] == h[0] and h[2] == 2.0 ** -7 * (1 + 2.0 ** -7)
    # rounding any value to bf16 moves it by at most the allowance
    rng = np.random.default_rng(0)
    y = rng.standard_normal(100000) * np.exp2(rng.integers(-20, 20, 100000))
    assert np.all(np.abs(_bf16(y) - y) <= bf16_half_ulp(y))


def test_rounded_oracle_passes(case):
    tiled, vm = case
    r = check_attention(_bf16(tiled), tiled, vm)
    assert r["term"] == 0.0 and r["maxabs_head_max"] == 0.0


def test_planted_wrong_head_fails(case):
    tiled, vm = case
    bad = _bf16(tiled)
    bad[1, 2] = _bf16(tiled[1, 1])  # head 2 of batch 1 holds head 1's output
    r = attention_report(bad, tiled, vm)
    assert r["rel_head_max"] > 5e-3
    with pytest.raises(AssertionError):
        check_attention(bad, tiled, vm)


def test_planted_tail_row_fails(case):
    tiled, vm = case
    bad = _bf16(tiled)
    bad[0, 0, -1] = _bf16(vm[0, 0])  # last query row of one head loses its attention term
    r = attention_report(bad, tiled, vm)
    assert r["maxabs_head_max"] > 1.0 / 16
    with pytest.raises(AssertionError):
        check_attention(bad, tiled, vm)


def test_planted_scaled_term_fails(case):
    tiled, vm = case
    vmb = vm[:, :, None, :]
    bad = _bf16(vmb + (tiled - vmb) * 1.02)  # attention term 2% too large everywhere
    r = attention_report(bad, tiled, vm)
    assert r["term"] > 5e-3
    with pytest.raises(AssertionError):
        check_attention(bad, tiled, vm)


def test_planted_nan_fails(case):
    tiled, vm = case
    bad = _bf16(tiled)
    bad[0, 1, 5, 3] = np.nan
    with pytest.raises(AssertionError):
        check_attention(bad, tiled, vm)
