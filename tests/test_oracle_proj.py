"""Pins of the oracle's row-wise FP8 projection: the row quantiser
(orc_quant_rows_e4m3) and the scaled FP8 GEMM (orc_gemm_fp8_rowwise) of the
FLUX.3 Action report §02 stage 02 ("mixed-precision projections": row-wise FP8)
and the SGLang page's latency notes (E4M3 weights, one scale per output row,
per-token activation scales)."""
import numpy as np
import pytest
import torch

import oracle
import synth


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


@pytest.fixture(scope="module")
def xw():
    return synth.proj_inputs(37, 256, 29, tag=601)


def test_row_quant_closed_forms(xw):
    """Per row: scale = fp32(a / 448); the absmax element codes to +-448;
    every code decodes to within half an E4M3 step of x * (448 / a); signs
    agree; codes never exceed 448 in magnitude."""
    x, _, _ = xw
    codes, scales = oracle.quant_rows_e4m3(x)
    xf = x.float().numpy()
    a = np.abs(xf).max(1)
    np.testing.assert_array_equal(scales, (a / np.float32(448.0)).astype(np.float32))
    dec = oracle.e4m3_decode(codes)
    inv = (np.float32(448.0) / a).astype(np.float32)
    y = (xf * inv[:, None]).astype(np.float32).astype(np.float64)
    assert np.all(np.abs(dec) <= 448)
    am = np.abs(xf).argmax(1)
    assert np.all(np.abs(dec[np.arange(len(am)), am]) == 448)
    tol = np.maximum(2.0 ** -4 * np.abs(y), 2.0 ** -10)
    assert np.all(np.abs(dec - y) <= tol + 1e-12)
    assert np.all(np.sign(dec) * np.sign(y) >= 0)


def test_row_quant_scaling_and_zero_rows(xw):
    """x -> 2x (exact in bf16) doubles every scale exactly and keeps the codes;
    an all-zero row has scale 0 and codes 0; a strided row view reads the same."""
    x, _, _ = xw
    c1, s1 = oracle.quant_rows_e4m3(x)
    c2, s2 = oracle.quant_rows_e4m3((x.float() * 2).to(torch.bfloat16))
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(s2, 2 * s1)
    xz = x.clone()
    xz[3] = 0
    cz, sz = oracle.quant_rows_e4m3(xz)
    assert sz[3] == 0 and np.all(cz[3] == 0)
    wide = torch.zeros(x.shape[0], x.shape[1] + 40, dtype=torch.bfloat16)
    wide[:, 24:24 + x.shape[1]] = x
    cv, sv = oracle.quant_rows_e4m3(wide[:, 24:24 + x.shape[1]])
    np.testing.assert_array_equal(cv, c1)
    np.testing.assert_array_equal(sv, s1)


def test_row_quant_matches_the_v_rule():
    """A V channel whose token mean is exactly 0 (tokens in +-pairs) is the
    same row quantisation: identical codes and scale (the V slot order undone)."""
    rng = np.random.default_rng(7)
    N, D = 64, 64
    half = rng.standard_normal((N // 2, D)).astype(np.float32)
    v = np.empty((N, D), np.float32)
    v[0::2], v[1::2] = half, -half
    vb = _bf16(v)
    ref_v = oracle.quant_v(vb.reshape(1, N, 1, D))
    assert np.all(ref_v["v_mean"] == 0)
    slots = np.array([oracle.v_slot(t) for t in range(64)])
    vcodes = ref_v["v_fp8"][0, 0][:, slots]                        # [D, N] in token order
    rc, rs = oracle.quant_rows_e4m3(vb.t().contiguous())            # channels as rows
    np.testing.assert_array_equal(rc, vcodes)
    np.testing.assert_array_equal(rs, ref_v["v_scale"][0, 0])


def test_gemm_matches_numpy_matmul(xw):
    """The scaled GEMM against numpy's fp64 matmul of the decoded codes, with
    the row scales on the rows, the weight scales on the columns, plus bias."""
    x, w, b = xw
    ca, sa = oracle.quant_rows_e4m3(x)
    cb, sb = oracle.quant_rows_e4m3(w)
    out, absum, blk = oracle.gemm_fp8_rowwise(ca, sa, cb, sb, bias=b)
    A, Bm = oracle.e4m3_decode(ca), oracle.e4m3_decode(cb)
    want = (A @ Bm.T) * sa.astype(np.float64)[:, None] * sb.astype(np.float64)[None, :] + b.double().numpy()[None, :]
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-12)
    wabs = (np.abs(A) @ np.abs(Bm).T) * sa[:, None] * sb[None, :] + np.abs(b.double().numpy())[None, :]
    np.testing.assert_allclose(absum, wabs, rtol=1e-12, atol=1e-12)
    # blk: sum over 64-blocks of |earlier partial sum| + the block's largest |product|
    P = A[:, None, :] * Bm[None, :, :]                               # [M, N, K]
    K = A.shape[1]
    pre = np.concatenate([np.zeros(P.shape[:2] + (1,)), np.cumsum(P, -1)[..., 63:K - 1:64]], -1)
    bmax = np.abs(P).reshape(P.shape[0], P.shape[1], -1, 64).max(-1)
    wblk = (np.abs(pre) + bmax).sum(-1) * sa[:, None] * sb[None, :]
    np.testing.assert_allclose(blk, wblk, rtol=1e-9, atol=1e-12)
    rows, cols = np.array([0, 5, 36], np.int32), np.array([28, 3], np.int32)
    sub, _, _ = oracle.gemm_fp8_rowwise(ca, sa, cb, sb, bias=b, rows=rows, cols=cols)
    np.testing.assert_array_equal(sub, out[np.ix_(rows, cols)])


def test_gemm_identity_weight_returns_the_dequantised_rows(xw):
    """W codes = 1.0 on the diagonal (0x38), scale 1, no bias: each output row is
    the dequantised activation row, exactly."""
    x, _, _ = xw
    ca, sa = oracle.quant_rows_e4m3(x)
    K = x.shape[1]
    cb = np.zeros((K, K), np.uint8)
    np.fill_diagonal(cb, 0x38)
    assert oracle.e4m3_decode(np.array([0x38], np.uint8))[0] == 1.0
    out, _, _ = oracle.gemm_fp8_rowwise(ca, sa, cb, np.ones(K, np.float32))
    np.testing.assert_array_equal(out, oracle.e4m3_decode(ca) * sa.astype(np.float64)[:, None])
