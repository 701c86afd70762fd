"""GPU parity at the size limits the C ABI accepts: B*H*Np*D just below 2^31
elements (the largest offsets any kernel forms), and more (b, h) pairs than
65535 (the grid dimension that carries them in the quantisers).

The whole path runs on the GPU; the oracle checks sampled heads, including the
last one, bit for bit for the quantised outputs and within 5e-3 relative L2
for attention.  Every head is quantised and attended independently of the
others, so the oracle runs on those heads alone.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.attn_bars import check_attention

pytestmark = pytest.mark.gpu

TOL_ORACLE = 5e-3


def _log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def sage():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_attention_video_smooth_amd as s
    s.lib()
    return s


def _check_heads(sage, cfg, heads, rows):
    B, N, H, D = cfg.B, cfg.N, cfg.H, cfg.D
    Np = sage.sage_padded_tokens(N)
    _log(f"  elements B*H*Np*D = {B * H * Np * D} (2^31 = {1 << 31}), B*H = {B * H}")
    q, k, v = synth.make_qkv(cfg, device="cuda")
    qk = sage.quant_qk(q, k)
    vq = sage.quant_v(v)
    out = sage.attn_fwd(*qk[:4], *vq, N=N)
    torch.cuda.synchronize()
    hs = torch.tensor(heads, device="cuda")
    qh, kh, vh = (t.index_select(2, hs).cpu() for t in (q, k, v))
    del q, k, v
    ref_qk, ref_v = oracle.quant_qk(qh, kh), oracle.quant_v(vh)
    assert ref_qk["inexact"] == 0 and ref_v["bad"] == 0
    g = {name: t.index_select(1, hs).cpu() for name, t in
         (("q_i8", qk[0]), ("q_scale", qk[1]), ("k_i8", qk[2]), ("k_scale", qk[3]), ("k_mean", qk[4]),
          ("v_fp8", vq[0]), ("v_scale", vq[1]), ("v_mean", vq[2]))}
    nq, nk = -(-N // 32), -(-N // 64)
    np.testing.assert_array_equal(g["q_i8"][:, :, :N].numpy(), ref_qk["q_i8"])
    np.testing.assert_array_equal(g["k_i8"][:, :, :N].numpy(), ref_qk["k_i8"])
    np.testing.assert_array_equal(g["q_scale"][:, :, :nq].numpy().view(np.uint32), ref_qk["q_scale"].view(np.uint32))
    np.testing.assert_array_equal(g["k_scale"][:, :, :nk].numpy().view(np.uint32), ref_qk["k_scale"].view(np.uint32))
    np.testing.assert_array_equal(g["k_mean"].view(torch.int16).numpy().view(np.uint16), ref_qk["k_mean"])
    np.testing.assert_array_equal(g["v_fp8"].numpy(), ref_v["v_fp8"])
    np.testing.assert_array_equal(g["v_scale"].numpy().view(np.uint32), ref_v["v_scale"].view(np.uint32))
    np.testing.assert_array_equal(g["v_mean"].numpy().view(np.uint32), ref_v["v_mean"].view(np.uint32))
    rows = np.asarray(rows, np.int32)
    got = out.index_select(2, hs).float().cpu()[:, rows].permute(0, 2, 1, 3).double().numpy()
    _log(f"  heads {heads}, rows {rows.tolist()}: quantised outputs bit-exact")
    check_attention(got, oracle.attn_tiled(ref_qk, ref_v, rows=rows), ref_v["v_mean"], log=_log)


def test_largest_element_count(sage):
    """B1 H16383 N1023 D128: B*H*Np*D = 2147352576, the last head's codes end
    just below 2^31 elements."""
    cfg = synth.custom(1, 1023, 16383, 128, tag=901)
    _log(f"[limits] B{cfg.B} N{cfg.N} H{cfg.H} D{cfg.D}")
    _check_heads(sage, cfg, [0, 8191, 16382], [0, 31, 32, 511, 1022])


def test_more_heads_than_65535(sage):
    """B2 H40000 N50 D64: 80000 (b, h) pairs, ragged single key tile."""
    cfg = synth.custom(2, 50, 40000, 64, tag=902)
    _log(f"[limits] B{cfg.B} N{cfg.N} H{cfg.H} D{cfg.D}")
    _check_heads(sage, cfg, [0, 1, 39999], [0, 31, 32, 49])
