"""Pins for the oracle's attention: the online softmax loop, the exact fp64
reference, and the quantised tiled path.

Passages: FLUX.3 Action RTX 5090 report, §02 stage 03 (INT8 QK, FP8 PV, FP32
accumulation, K smooth and V smooth kept); MiniMax H3 on DGX Spark, §01
(Sage2++ = QK INT8 / PV FP8).  The invariances are the ones smoothing relies on:
softmax rows do not change when a per-channel constant is added to K, and
rows sum to one, so a per-channel shift of V passes straight to the output.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def _softmax_pv(s, vals):
    w = np.exp(s - s.max())
    return (w / w.sum()) @ vals


@pytest.mark.parametrize("n,bc", [(1, 64), (5, 2), (70, 64), (200, 16), (256, 64), (256, 256), (300, 1)])
def test_online_softmax_equals_plain_softmax(n, bc):
    """With the FP8 step switched off, tiling and rescaling must not change the
    result (flash attention identity), including a ragged last tile."""
    rng = np.random.default_rng(n * 1000 + bc)
    s = rng.standard_normal(n) * 6.0
    s[rng.integers(0, n)] += 25.0          # a late dominant score forces rescaling
    vals = rng.standard_normal((n, 7))
    got = oracle.online_softmax_pv(s, vals, bc, quant_p=False)
    np.testing.assert_allclose(got, _softmax_pv(s, vals), rtol=1e-12, atol=1e-13)


def _e4m3_torch(x):
    return torch.from_numpy(np.asarray(x, np.float64)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_fp8_p_hand_expanded_two_tiles():
    """R13/R14 written out for N = 5, tiles {0,1}, {2,3}, {4}: each tile's FP8
    weights E4M3(448 p) use the running max including that tile; older tiles are
    rescaled by exp(m_old - m_new); the row sum uses unquantised p."""
    rng = np.random.default_rng(11)
    s = rng.standard_normal(5) * 3.0
    vals = rng.standard_normal((5, 3))
    m1 = s[:2].max()
    m2 = max(m1, s[2:4].max())
    m3 = max(m2, s[4])
    q = lambda p: _e4m3_torch(448.0 * p) / 448.0
    acc = (np.exp(m1 - m3) * (q(np.exp(s[:2] - m1)) @ vals[:2])
           + np.exp(m2 - m3) * (q(np.exp(s[2:4] - m2)) @ vals[2:4])
           + q(np.exp(s[4:] - m3)) @ vals[4:])
    l = np.exp(s - m3).sum()
    got = oracle.online_softmax_pv(s, vals, 2, quant_p=True)
    np.testing.assert_allclose(got, acc / l, rtol=1e-13)


def test_fp8_p_single_tile_is_final_max_rounding():
    rng = np.random.default_rng(12)
    s = rng.standard_normal(40) * 2.0
    vals = rng.standard_normal((40, 4))
    p = np.exp(s - s.max())
    want = (_e4m3_torch(448.0 * p) / 448.0) @ vals / p.sum()
    np.testing.assert_allclose(oracle.online_softmax_pv(s, vals, 40, True), want, rtol=1e-13)


CASES = [synth.config(0), synth.custom(1, 150, 2, 64, tag=201), synth.custom(2, 70, 2, 128, tag=202)]


@pytest.fixture(scope="module", params=CASES, ids=lambda c: c.name)
def case(request):
    cfg = request.param
    q, k, v = synth.make_qkv(cfg)
    return cfg, q, k, v


def test_exact_matches_torch_sdpa_fp64(case):
    cfg, q, k, v = case
    got = oracle.attn_exact(q, k, v)
    qt, kt, vt = (x.double().permute(0, 2, 1, 3) for x in (q, k, v))
    want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)


def test_exact_k_shift_invariance_and_v_shift_equivariance(case):
    """Values on a 1/16 grid in [-4, 4] shifted by integers in [-3, 3] stay exact
    in bf16, so the shifted inputs are exactly K + 1 c^T and V + 1 c^T."""
    cfg, q, k, v = case
    B, N, H, D = q.shape
    rng = np.random.default_rng(13)
    grid = lambda x: (torch.round(x.float().clamp(-4, 4) * 16) / 16).to(torch.bfloat16)
    q, k, v = grid(q), grid(k), grid(v)
    ck = torch.from_numpy(rng.integers(-3, 4, (1, 1, H, D)).astype(np.float32))
    cv = torch.from_numpy(rng.integers(-3, 4, (1, 1, H, D)).astype(np.float32))
    k2 = (k.float() + ck).to(torch.bfloat16)
    v2 = (v.float() + cv).to(torch.bfloat16)
    assert torch.equal(k2.float(), k.float() + ck) and torch.equal(v2.float(), v.float() + cv)
    base = oracle.attn_exact(q, k, v)
    np.testing.assert_allclose(oracle.attn_exact(q, k2, v), base, rtol=1e-10, atol=1e-12)
    shift = cv.numpy().transpose(0, 2, 1, 3)           # [1,H,1,D]
    np.testing.assert_allclose(oracle.attn_exact(q, k, v2), base + shift, rtol=1e-10, atol=1e-12)


def test_exact_rows_sum_to_one(case):
    cfg, q, k, v = case
    ones = torch.ones_like(v)
    np.testing.assert_allclose(oracle.attn_exact(q, k, ones), 1.0, rtol=0, atol=1e-14)


@pytest.mark.parametrize("q_block,k_block", [(32, 64), (1, 64), (32, 16), (1, 16)])
def test_tiled_wiring_matches_numpy(case, q_block, k_block):
    """Step 7 indexing: scores from INT8 codes with the per-32 (or per-token) Q
    and per-64 (or per-16) K scales, V codes read back through the slot map,
    V scale and mean applied."""
    cfg, q, k, v = case
    qk, vq = oracle.quant_qk(q, k, q_block=q_block, k_block=k_block), oracle.quant_v(v)
    B, N, H, D = q.shape
    rows = np.array(sorted({0, 1, 31, 32, N // 2, N - 1}), np.int32)
    got = oracle.attn_tiled(qk, vq, rows=rows)
    sm = 1.0 / math.sqrt(D)
    slots = np.array([oracle.v_slot(t) for t in range(64)])
    cols = (np.arange(N) // 64) * 64 + slots[np.arange(N) % 64]
    for b in range(B):
        for h in range(H):
            kd = qk["k_i8"][b, h].astype(np.int64)
            vals = oracle.e4m3_decode(vq["v_fp8"][b, h][:, cols]).T          # [N, D]
            for r, i in enumerate(rows):
                dots = kd @ qk["q_i8"][b, h, i].astype(np.int64)
                s = dots * (float(qk["q_scale"][b, h, i // q_block]) * sm) * qk["k_scale"][b, h, np.arange(N) // k_block].astype(np.float64)
                o = oracle.online_softmax_pv(s, vals, 64, True)
                want = o * vq["v_scale"][b, h] + vq["v_mean"][b, h]
                np.testing.assert_allclose(got[b, h, r], want, rtol=1e-12, atol=1e-12)


def test_tiled_zero_q_closed_form(case):
    """Q = 0: every score is 0, p = 1 exactly, E4M3(448) = 448, so
    O = v_mean + v_scale * mean_j decode(v_j)."""
    cfg, q, k, v = case
    B, N, H, D = q.shape
    qk, vq = oracle.quant_qk(torch.zeros_like(q), k), oracle.quant_v(v)
    got = oracle.attn_tiled(qk, vq)
    slots = np.array([oracle.v_slot(t) for t in range(64)])
    cols = (np.arange(N) // 64) * 64 + slots[np.arange(N) % 64]
    dec = oracle.e4m3_decode(vq["v_fp8"][..., cols])                          # [B,H,D,N]
    want = vq["v_mean"][:, :, None, :] + vq["v_scale"][:, :, None, :] * dec.mean(-1)[:, :, None, :]
    np.testing.assert_allclose(got, np.broadcast_to(want, got.shape), rtol=1e-13, atol=1e-13)


def test_tiled_constant_v_returns_v(case):
    """V constant over tokens: V - mean = 0, so the output is the mean exactly."""
    cfg, q, k, v = case
    vc = v[:, :1].expand_as(v).contiguous()
    qk, vq = oracle.quant_qk(q, k), oracle.quant_v(vc)
    got = oracle.attn_tiled(qk, vq)
    want = vc.float().numpy()[:, 0][:, :, None, :]
    np.testing.assert_array_equal(got, np.broadcast_to(want, got.shape))


def test_tiled_single_token():
    q, k, v = synth.make_qkv(synth.custom(1, 1, 2, 64, tag=203))
    got = oracle.attn_tiled(oracle.quant_qk(q, k), oracle.quant_v(v))
    np.testing.assert_array_equal(got[:, :, 0], v.float().numpy()[:, 0])


def test_tiled_unquantised_limit_is_close_to_exact():
    """With K smoothing the tiled path approximates softmax(QK^T)V; on a D=64
    case with mild values its error is dominated by the FP8 P and V steps."""
    cfg = synth.custom(1, 256, 2, 64, tag=204)
    q, k, v = synth.make_qkv(cfg)
    o = oracle.attn_tiled(oracle.quant_qk(q, k), oracle.quant_v(v))
    e = oracle.attn_exact(q, k, v)
    assert oracle.rel_l2(o, e) < 0.06


def test_tiny_error_budget():
    """The method's own error on the tiny workload (smoothing + INT8 + FP8).
    The quantised path is ~3.6e-2 from exact fp64 attention, above a 3e-2 bar:
    this is a property of E4M3's 3 mantissa bits on both PV operands."""
    q, k, v = synth.make_qkv(0)
    qk, vq = oracle.quant_qk(q, k), oracle.quant_v(v)
    o = oracle.attn_tiled(qk, vq)
    e = oracle.attn_exact(q, k, v)
    err = oracle.rel_l2(o, e)
    assert 0.02 < err < 0.05, err
    final_max = oracle.attn_tiled(qk, vq, bc=256)
    assert 0.01 < oracle.rel_l2(final_max, o) < 0.03
