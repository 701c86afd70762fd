"""Pins for the oracle's quantisation steps (K smoothing + INT8, Q INT8,
V smoothing + FP8 with transpose / pad / permutation).

Passages: FLUX.3 Action RTX 5090 report, §02 stage 03 (INT8 QK, FP8 PV, K and V
smoothing), stage 04 (fused == unfused, bit exact), card A (K centre + BF16 round
+ INT8; Q quant and INT8 rules unchanged), card C (V transpose, padding and
permutation; V mean / scale / quant).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)


def _f(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


SHAPES = [
    synth.config(0),
    synth.custom(2, 200, 3, 64, tag=101),   # ragged: 200 = 3*64 + 8, 200 = 6*32 + 8
    synth.custom(1, 77, 2, 128, tag=102),   # D = 128, one partial block each
    synth.custom(1, 1, 2, 64, tag=103),     # N = 1
]


@pytest.fixture(scope="module", params=SHAPES, ids=lambda c: c.name)
def qkv(request):
    cfg = request.param
    return cfg, synth.make_qkv(cfg)


def test_fused_equals_composed(qkv):
    """Stage 04 / card A: centring fused into the quantiser is bit-identical to
    materialising the BF16 mean and BF16 centred K first."""
    cfg, (q, k, v) = qkv
    fused = oracle.quant_qk(q, k)
    mean, bad = oracle.k_mean(k)
    assert bad == 0 and fused["inexact"] == 0
    kc = oracle.k_center(k, mean)
    kc_codes, kc_scales = oracle.quant_i8_blocks(kc, 64)
    q_codes, q_scales = oracle.quant_i8_blocks(q.view(torch.int16).numpy().view(np.uint16), 32)
    np.testing.assert_array_equal(fused["k_mean"], mean)
    np.testing.assert_array_equal(fused["k_i8"], kc_codes)
    np.testing.assert_array_equal(fused["k_scale"], kc_scales)
    np.testing.assert_array_equal(fused["q_i8"], q_codes)
    np.testing.assert_array_equal(fused["q_scale"], q_scales)


def test_k_mean_matches_numpy(qkv):
    """Library pin: fp64 mean (numpy) -> fp32 -> bf16 (torch cast)."""
    cfg, (q, k, v) = qkv
    got, _ = oracle.k_mean(k)
    m = k.float().numpy().astype(np.float64).mean(axis=1)          # [B, H, D]
    want = _bf16(m.astype(np.float32)).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, want)


def test_k_center_is_bf16_of_difference(qkv):
    cfg, (q, k, v) = qkv
    mean, _ = oracle.k_mean(k)
    kc = oracle.k_center(k, mean)
    diff = k.float().numpy() - _f(mean)[:, None, :, :]               # fp32 numpy subtraction
    want = _bf16(diff).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(kc, want)


def _check_int8_blocks(x_f32_bhnd, codes, scales, blk):
    """Closed-form properties of a symmetric absmax INT8 quantiser."""
    B, H, N, D = x_f32_bhnd.shape
    assert np.abs(codes.astype(np.int32)).max() <= 127
    for t in range(scales.shape[-1]):
        xs = x_f32_bhnd[:, :, t * blk:(t + 1) * blk, :]
        cs = codes[:, :, t * blk:(t + 1) * blk, :].astype(np.float64)
        a = np.abs(xs).reshape(B, H, -1).max(-1)
        s = scales[:, :, t].astype(np.float64)
        np.testing.assert_allclose(s, a / 127.0, rtol=2**-23)
        # the absmax element maps to +-127
        flat_x = np.abs(xs).reshape(B, H, -1)
        flat_c = np.abs(cs).reshape(B, H, -1)
        idx = flat_x.argmax(-1)
        am = np.take_along_axis(flat_c, idx[..., None], -1)[..., 0]
        assert np.all(am[a > 0] == 127)
        # reconstruction within half a step, signs agree
        err = np.abs(cs * s[:, :, None, None] - xs)
        assert np.all(err <= s[:, :, None, None] * (0.5 + 1e-5) + 1e-30)
        assert np.all(np.sign(cs) * np.sign(xs) >= 0)
        assert np.all(cs[a == 0] == 0)


def test_int8_closed_forms(qkv):
    cfg, (q, k, v) = qkv
    out = oracle.quant_qk(q, k)
    qf = q.float().numpy().transpose(0, 2, 1, 3)
    _check_int8_blocks(qf, out["q_i8"], out["q_scale"], 32)
    mean, _ = oracle.k_mean(k)
    kc = _f(oracle.k_center(k, mean)).transpose(0, 2, 1, 3)
    _check_int8_blocks(kc, out["k_i8"], out["k_scale"], 64)


def test_per_token_q_closed_forms(qkv):
    """One Q scale per token (the finer granularity of §02 stage 03): each
    row is its own absmax block; K is untouched by the Q granularity."""
    cfg, (q, k, v) = qkv
    out1 = oracle.quant_qk(q, k, q_block=1)
    out32 = oracle.quant_qk(q, k)
    assert out1["q_scale"].shape == (cfg.B, cfg.H, cfg.N)
    qf = q.float().numpy().transpose(0, 2, 1, 3)
    _check_int8_blocks(qf, out1["q_i8"], out1["q_scale"], 1)
    for key in ("k_i8", "k_scale", "k_mean"):
        np.testing.assert_array_equal(out1[key], out32[key])
    # a token's scale never exceeds its 32-token block's
    blk = out32["q_scale"][:, :, np.arange(cfg.N) // 32]
    assert np.all(out1["q_scale"] <= blk)


def test_per_token_equals_block_when_rows_share_absmax():
    """If every row of a 32-token block has the same absmax, per-token and
    per-block quantisation are the same numbers, and so is the attention."""
    B, N, H, D = 1, 100, 2, 64
    rng = np.random.default_rng(9)
    qv = rng.uniform(-1.0, 1.0, (B, N, H, D)).astype(np.float32)
    qv[..., 5] = np.where(np.arange(N) % 2 == 0, 2.0, -2.0)[None, :, None]   # |x| = 2 is each row's max
    q, k, v = _bf16(qv), _bf16(rng.standard_normal((B, N, H, D))), _bf16(rng.standard_normal((B, N, H, D)))
    out1, out32 = oracle.quant_qk(q, k, q_block=1), oracle.quant_qk(q, k)
    np.testing.assert_array_equal(out1["q_i8"], out32["q_i8"])
    np.testing.assert_array_equal(out1["q_scale"], out32["q_scale"][:, :, np.arange(N) // 32])
    vq = oracle.quant_v(v)
    np.testing.assert_array_equal(oracle.attn_tiled(out1, vq), oracle.attn_tiled(out32, vq))


def test_k16_closed_forms(qkv):
    """16-token K blocks: closed-form quantiser properties per 16-token block of
    the centred K; Q and the K mean do not depend on the K granularity; the
    largest of the four 16-token scales inside a 64-token block is that
    block's scale exactly (a/127 is monotone in a)."""
    cfg, (q, k, v) = qkv
    out16 = oracle.quant_qk(q, k, k_block=16)
    out64 = oracle.quant_qk(q, k)
    assert out16["k_scale"].shape == (cfg.B, cfg.H, math.ceil(cfg.N / 16))
    mean, _ = oracle.k_mean(k)
    kc = _f(oracle.k_center(k, mean)).transpose(0, 2, 1, 3)
    _check_int8_blocks(kc, out16["k_i8"], out16["k_scale"], 16)
    for key in ("q_i8", "q_scale", "k_mean"):
        np.testing.assert_array_equal(out16[key], out64[key])
    n16 = out16["k_scale"].shape[-1]
    for t in range(out64["k_scale"].shape[-1]):
        sub = out16["k_scale"][:, :, 4 * t:min(4 * t + 4, n16)]
        np.testing.assert_array_equal(sub.max(-1), out64["k_scale"][:, :, t])


def test_k16_equals_k64_when_subblocks_share_absmax():
    """K built from +-x token pairs has a channel mean of exactly 0, so the
    centred K is K itself; with |x| = 2 planted in every token, each 16-token
    block has the 64-token block's absmax, and both granularities give the
    same codes, the same (repeated) scales and the same attention."""
    B, N, H, D = 1, 100, 2, 64
    rng = np.random.default_rng(11)
    half = rng.uniform(-1.0, 1.0, (B, N // 2, H, D)).astype(np.float32)
    half[..., 5] = 2.0
    kv = np.empty((B, N, H, D), np.float32)
    kv[:, 0::2], kv[:, 1::2] = half, -half
    k = _bf16(kv)
    q, v = _bf16(rng.standard_normal((B, N, H, D))), _bf16(rng.standard_normal((B, N, H, D)))
    out16, out64 = oracle.quant_qk(q, k, k_block=16), oracle.quant_qk(q, k)
    assert np.all(out64["k_mean"] == 0)
    np.testing.assert_array_equal(out16["k_i8"], out64["k_i8"])
    np.testing.assert_array_equal(out16["k_scale"], out64["k_scale"][:, :, np.arange(7) // 4])
    vq = oracle.quant_v(v)
    np.testing.assert_array_equal(oracle.attn_tiled(out16, vq), oracle.attn_tiled(out64, vq))


def test_constant_k_channels_give_zero_codes():
    B, N, H, D = 1, 130, 2, 64
    rng = np.random.default_rng(5)
    base = rng.standard_normal((1, 1, H, D)).astype(np.float32)
    k = _bf16(np.broadcast_to(base, (B, N, H, D)))
    q = _bf16(rng.standard_normal((B, N, H, D)))
    out = oracle.quant_qk(q, k)
    assert np.all(out["k_i8"] == 0) and np.all(out["k_scale"] == 0)
    np.testing.assert_array_equal(out["k_mean"], k[0, 0].view(torch.int16).numpy().view(np.uint16)[None])


def test_zero_q_block_and_block_isolation():
    B, N, H, D = 1, 96, 1, 64
    rng = np.random.default_rng(6)
    qv = rng.standard_normal((B, N, H, D)).astype(np.float32)
    qv[:, 32:64] = 0.0
    out = oracle.quant_qk(_bf16(qv), _bf16(qv))
    assert out["q_scale"][0, 0, 1] == 0 and np.all(out["q_i8"][0, 0, 32:64] == 0)
    qv2 = qv.copy()
    qv2[0, 70, 0, 5] = 1000.0
    out2 = oracle.quant_qk(_bf16(qv2), _bf16(qv))
    np.testing.assert_array_equal(out2["q_scale"][0, 0, :2], out["q_scale"][0, 0, :2])
    assert out2["q_scale"][0, 0, 2] != out["q_scale"][0, 0, 2]
    np.testing.assert_array_equal(out2["q_i8"][0, 0, :64], out["q_i8"][0, 0, :64])


def test_token_permutation_within_block_permutes_codes():
    """The K mean and block absmax do not depend on token order inside a block."""
    cfg = synth.custom(1, 192, 2, 64, tag=104)
    q, k, v = synth.make_qkv(cfg)
    perm = np.arange(192)
    rng = np.random.default_rng(7)
    for t in range(3):
        perm[t * 64:(t + 1) * 64] = t * 64 + rng.permutation(64)
    a = oracle.quant_qk(q, k)
    b = oracle.quant_qk(q[:, perm].contiguous(), k[:, perm].contiguous())
    np.testing.assert_array_equal(b["k_mean"], a["k_mean"])
    np.testing.assert_array_equal(b["k_scale"], a["k_scale"])
    np.testing.assert_array_equal(b["k_i8"], a["k_i8"][:, :, perm])


def test_strided_inputs_equal_contiguous():
    """A row-strided view (V or K read out of a wider projection output) gives the
    same bits as the contiguous tensor."""
    cfg = synth.custom(2, 100, 3, 64, tag=105)
    q, k, v = synth.make_qkv(cfg)
    wide = torch.zeros(2, 100, 3 * 64 + 96, dtype=torch.bfloat16)
    wide[:, :, 32:32 + 192] = v.reshape(2, 100, 192)
    v_view = wide[:, :, 32:32 + 192].view(2, 100, 3, 64)
    assert not v_view.is_contiguous()
    a, b = oracle.quant_v(v), oracle.quant_v(v_view)
    for key in ("v_fp8", "v_scale", "v_mean"):
        np.testing.assert_array_equal(a[key], b[key])
    wide[:, :, 32:32 + 192] = k.reshape(2, 100, 192)
    k_view = wide[:, :, 32:32 + 192].view(2, 100, 3, 64)
    a, b = oracle.quant_qk(q, k), oracle.quant_qk(q, k_view)
    for key in ("k_i8", "k_scale", "k_mean"):
        np.testing.assert_array_equal(a[key], b[key])


# ---- V ---------------------------------------------------------------------

def _unpermute(v_fp8, N):
    Np = v_fp8.shape[-1]
    slots = np.array([oracle.v_slot(t) for t in range(64)])
    cols = (np.arange(N) // 64) * 64 + slots[np.arange(N) % 64]
    return v_fp8[..., cols], cols


def test_v_mean_scale_and_codes(qkv):
    cfg, (q, k, v) = qkv
    out = oracle.quant_v(v)
    assert out["bad"] == 0
    B, N, H, D = v.shape
    vf = v.float().numpy()                                               # [B,N,H,D]
    mu = vf.astype(np.float64).mean(axis=1).astype(np.float32)           # numpy fp64 mean -> fp32
    np.testing.assert_array_equal(out["v_mean"], mu)
    centred = (vf - mu[:, None]).astype(np.float32)                      # fp32 subtraction
    a = np.abs(centred).max(axis=1)                                      # brute-force absmax
    zero = a == 0
    scale = np.where(zero, np.float32(0), a / np.float32(448)).astype(np.float32)
    np.testing.assert_array_equal(out["v_scale"], scale)
    codes, cols = _unpermute(out["v_fp8"], N)                            # [B,H,D,N]
    codes = codes.transpose(0, 3, 1, 2)                                  # [B,N,H,D]
    dec = oracle.e4m3_decode(codes)
    # absmax element of each channel maps to +-448 (0x7E / 0xFE)
    idx = np.abs(centred).argmax(axis=1)
    am = np.take_along_axis(codes, idx[:, None], 1)[:, 0]
    assert np.all((am[~zero] & 0x7F) == 0x7E)
    # reconstruction: relative error <= 2^-4 (3 mantissa bits), absolute <= 2^-10 * 448 scale-steps
    s64 = out["v_scale"].astype(np.float64)[:, None]
    err = np.abs(dec * s64 - centred)
    tol = np.maximum(np.abs(centred) * 2.0**-4, 2.0**-10 * s64) * (1 + 1e-6) + 1e-30
    assert np.all(err <= tol)
    # library cross-check of the encoding: torch's float8_e4m3fn cast of fp32 (V - mu) * inv
    inv = np.where(zero, np.float32(0), np.float32(448) / np.where(zero, 1, a)).astype(np.float32)
    y = (centred * inv[:, None]).astype(np.float32)
    want = torch.from_numpy(np.clip(y, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    want = np.where(zero[:, None], np.uint8(0), want)
    np.testing.assert_array_equal(codes, want)


def test_v_padding_is_zero(qkv):
    cfg, (q, k, v) = qkv
    out = oracle.quant_v(v)
    N = v.shape[1]
    _, cols = _unpermute(out["v_fp8"], N)
    pad = np.setdiff1d(np.arange(out["v_fp8"].shape[-1]), cols)
    assert out["v_fp8"].shape[-1] == math.ceil(N / 64) * 64
    assert np.all(out["v_fp8"][..., pad] == 0)


def test_v_layout_transposed_and_permuted():
    """Token order is recoverable through the slot map: with values increasing in
    the token index, un-permuted codes increase monotonically."""
    B, N, H, D = 1, 150, 1, 64
    base = np.linspace(-3, 5, N, dtype=np.float32)[None, :, None, None]
    vals = np.broadcast_to(base, (B, N, H, D)) + np.linspace(0, 0.5, D, dtype=np.float32)
    out = oracle.quant_v(_bf16(vals))
    codes, _ = _unpermute(out["v_fp8"], N)
    dec = oracle.e4m3_decode(codes)[0, 0]                                # [D, N]
    assert np.all(np.diff(dec, axis=1) >= 0)
    assert np.any(np.diff(dec[:, :64], axis=1) > 0)


def test_v_single_token_is_all_zero():
    q, k, v = synth.make_qkv(synth.custom(1, 1, 2, 64, tag=106))
    out = oracle.quant_v(v)
    assert np.all(out["v_fp8"] == 0) and np.all(out["v_scale"] == 0)
    np.testing.assert_array_equal(out["v_mean"], v.float().numpy()[:, 0])


@pytest.mark.parametrize("idx", [1, 2])
def test_sums_exact_on_workloads(idx):
    """Reading R3: the per-channel fp64 sums of the synthetic workloads are exact,
    so any reduction order on the GPU gives the same mean bits."""
    q, k, v = synth.make_qkv(idx)
    assert oracle.k_mean(k)[1] == 0
    assert oracle.quant_v(v)["bad"] == 0
