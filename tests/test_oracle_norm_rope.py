"""Pins of the oracle's QK RMSNorm + RoPE producer (orc_norm_rope) against
closed forms, exact invariances and an independent fp64 reference.

The producer is the fused QK RMSNorm + RoPE of the "FLUX 3 Action" SGLang page
(§1 and the latency notes), storing BF16 NHD (report card B); the arithmetic
reading (each bf16 rounding of the eager composition kept) is stated in the
oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import synth


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _identity_table(N, D):
    t = np.zeros((N, D // 2, 2), np.float32)
    t[..., 0] = 1.0
    return t


def _ones(D):
    return torch.ones(D, dtype=torch.bfloat16)


@pytest.fixture(scope="module")
def x():
    cfg = synth.custom(2, 70, 3, 64, tag=401)
    q, _, _ = synth.make_qkv(cfg)
    return q


def test_unit_weight_identity_rotation_is_rms_normalisation(x):
    """w = 1 and (c, s) = (1, 0): y = bf16(x r), within one bf16 ulp of the fp64
    x / sqrt(mean x^2 + eps) computed by numpy, and of unit RMS."""
    B, N, H, D = x.shape
    eps = 1e-6
    y, bad = oracle.norm_rope(x, _ones(D), _identity_table(N, D), eps)
    assert bad == 0
    xd = x.double().numpy()
    ref = xd / np.sqrt((xd * xd).mean(-1, keepdims=True) + eps)
    yd = y.double().numpy()
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    assert np.all(np.abs(yd - ref) <= ulp)
    rms2 = (yd * yd).mean(-1)
    assert np.all(np.abs(rms2 - 1.0) < 2 ** -7)


def test_scale_by_powers_of_two_is_exact_without_eps(x):
    """With eps = 0, scaling x by 2 or 1/2 (exact in bf16) scales r by exactly
    the inverse, so y is bit-identical."""
    B, N, H, D = x.shape
    w, t = synth.norm_weight(synth.custom(1, 1, 1, D, tag=401), "q"), synth.rope_table(N, D)
    y, _ = oracle.norm_rope(x, w, t, 0.0)
    for f in (2.0, 0.5, 64.0):
        y2, _ = oracle.norm_rope((x.float() * f).to(torch.bfloat16), w, t, 0.0)
        assert torch.equal(y2.view(torch.int16), y.view(torch.int16))


def test_quarter_turn_swaps_each_pair(x):
    """(c, s) = (0, 1) maps (u_2i, u_2i+1) to (-u_2i+1, u_2i) exactly; (c, s) =
    (-1, 0) negates; the identity table returns u itself."""
    B, N, H, D = x.shape
    w = synth.norm_weight(synth.custom(1, 1, 1, D, tag=402), "k")
    u, _ = oracle.norm_rope(x, w, _identity_table(N, D))
    quarter = np.zeros((N, D // 2, 2), np.float32)
    quarter[..., 1] = 1.0
    yq, _ = oracle.norm_rope(x, w, quarter)
    uf, yf = u.float(), yq.float()
    assert torch.equal(yf[..., 0::2], -uf[..., 1::2])
    assert torch.equal(yf[..., 1::2], uf[..., 0::2])
    half = np.zeros((N, D // 2, 2), np.float32)
    half[..., 0] = -1.0
    yh, _ = oracle.norm_rope(x, w, half)
    assert torch.equal(yh.float(), -uf)


def test_table_indexed_by_token_and_pair(x):
    """Only the rotated (token, pair) changes: pair i covers channels 2i, 2i+1
    and row n of the table belongs to token n (every batch entry and head)."""
    B, N, H, D = x.shape
    w = _ones(D)
    t = _identity_table(N, D)
    u, _ = oracle.norm_rope(x, w, t)
    t2 = t.copy()
    t2[5, 3] = (0.0, 1.0)
    y, _ = oracle.norm_rope(x, w, t2)
    diff = (y.view(torch.int16) != u.view(torch.int16))
    assert not diff[:, :5].any() and not diff[:, 6:].any()
    assert not diff[:, 5, :, :6].any() and not diff[:, 5, :, 8:].any()
    assert torch.equal(y[:, 5, :, 6].float(), -u[:, 5, :, 7].float())
    assert torch.equal(y[:, 5, :, 7].float(), u[:, 5, :, 6].float())


def test_weight_multiplies_the_rounded_normalisation(x):
    """w = 2 doubles y exactly; w = 0.5 on channel 7 alone halves only that
    channel (identity rotation), exactly."""
    B, N, H, D = x.shape
    t = _identity_table(N, D)
    u, _ = oracle.norm_rope(x, _ones(D), t)
    y2, _ = oracle.norm_rope(x, 2 * _ones(D), t)
    assert torch.equal(y2.float(), 2 * u.float())
    w = _ones(D)
    w[7] = 0.5
    yh, _ = oracle.norm_rope(x, w, t)
    assert torch.equal(yh[..., 7].float(), 0.5 * u[..., 7].float())
    keep = [d for d in range(D) if d != 7]
    assert torch.equal(yh[..., keep].view(torch.int16), u[..., keep].view(torch.int16))


def test_rotation_preserves_pair_norms(x):
    """A rotation keeps |(y_2i, y_2i+1)| = |(u_2i, u_2i+1)| up to bf16 rounding."""
    B, N, H, D = x.shape
    w = synth.norm_weight(synth.custom(1, 1, 1, D, tag=403), "q")
    u, _ = oracle.norm_rope(x, w, _identity_table(N, D))
    y, _ = oracle.norm_rope(x, w, synth.rope_table(N, D))
    nu = (u.double()[..., 0::2] ** 2 + u.double()[..., 1::2] ** 2).sqrt()
    ny = (y.double()[..., 0::2] ** 2 + y.double()[..., 1::2] ** 2).sqrt()
    assert torch.all((ny - nu).abs() <= 2 ** -7 * nu + 1e-30)
    # and the angles are the table's: y = R(theta) u within bf16 rounding
    t = torch.from_numpy(synth.rope_table(N, D)).double()
    c, s = t[None, :, None, :, 0], t[None, :, None, :, 1]
    u0, u1 = u.double()[..., 0::2], u.double()[..., 1::2]
    assert torch.all((y.double()[..., 0::2] - (u0 * c - u1 * s)).abs() <= 2 ** -8 * nu + 1e-30)
    assert torch.all((y.double()[..., 1::2] - (u0 * s + u1 * c)).abs() <= 2 ** -8 * nu + 1e-30)


def test_eps_sits_inside_the_root():
    """Small rows with a large eps: r ~ 1 / sqrt(eps); checked against fp64."""
    B, N, H, D = 1, 4, 1, 64
    rng = np.random.default_rng(3)
    xs = _bf16(rng.standard_normal((B, N, H, D)) * 1e-3)
    eps = 1e-2
    y, _ = oracle.norm_rope(xs, _ones(D), _identity_table(N, D), eps)
    xd = xs.double().numpy()
    ref = xd / np.sqrt((xd * xd).mean(-1, keepdims=True) + eps)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    assert np.all(np.abs(y.double().numpy() - ref) <= ulp)
    assert np.abs(y.double().numpy()).max() < 0.05


def test_zero_row_and_exactness_flag():
    """An all-zero row with eps > 0 stays zero.  A row holding 2^-40 next to
    O(1) values is flagged as a sum that may be inexact; plain rows are not."""
    B, N, H, D = 1, 3, 1, 64
    rng = np.random.default_rng(4)
    xv = rng.standard_normal((B, N, H, D)).astype(np.float32)
    xv[0, 0] = 0.0
    xv[0, 2, 0, 5] = 2.0 ** -40
    y, bad = oracle.norm_rope(_bf16(xv), _ones(D), _identity_table(N, D), 1e-6)
    assert torch.all(y[0, 0] == 0)
    assert bad == 1


def test_matches_torch_eager_composition(x):
    """The eager composition written with torch CPU tensor ops: normalise in
    fp32 and store bf16, multiply by the bf16 weight in bf16, rotate in fp32
    and store bf16.  r comes from numpy in fp64, rounded once to fp32.  Equal
    bit for bit: the oracle keeps exactly these roundings."""
    B, N, H, D = x.shape
    eps = 1e-6
    w = synth.norm_weight(synth.custom(1, 1, 1, D, tag=404), "k")
    t = synth.rope_table(N, D)
    y, _ = oracle.norm_rope(x, w, t, eps)
    xd = x.double().numpy()
    r = torch.from_numpy((1.0 / np.sqrt((xd * xd).sum(-1, keepdims=True) / D + eps)).astype(np.float32))
    n = (x.float() * r).to(torch.bfloat16)
    u = (n * w).float()
    tt = torch.from_numpy(t)
    c, s = tt[None, :, None, :, 0], tt[None, :, None, :, 1]
    u0, u1 = u[..., 0::2], u[..., 1::2]
    want = torch.empty_like(u)
    want[..., 0::2] = u0 * c - u1 * s
    want[..., 1::2] = u0 * s + u1 * c
    assert torch.equal(y.view(torch.int16), want.to(torch.bfloat16).view(torch.int16))
