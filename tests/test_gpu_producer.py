"""GPU parity of the QK RMSNorm + RoPE producer (sage_norm_rope) and of the
producer fused into the quantiser (sage_norm_rope_quant_qk), through the C ABI.

Bar: bit-exact bf16 outputs of the producer against the oracle; the fused
quantiser's INT8 codes, scales and K mean bit-exact against the oracle's
quantiser applied to the oracle producer's outputs, and bit-identical to the
composed GPU path (sage_norm_rope, then sage_quant_qk_ex); attention on the
fused operands within 5e-3 relative L2 of the oracle.
"""
import math
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


def _consts(cfg):
    wq, wk = synth.norm_weight(cfg, "q"), synth.norm_weight(cfg, "k")
    rope = torch.from_numpy(synth.rope_table(cfg.N, cfg.D))
    return wq, wk, rope


def _check_qk(qk, ref, N):
    q_i8, q_scale, k_i8, k_scale, k_mean = [t.cpu() for t in qk]
    nq, nk = math.ceil(N / ref["q_block"]), math.ceil(N / ref["k_block"])
    np.testing.assert_array_equal(q_i8[:, :, :N].numpy(), ref["q_i8"])
    np.testing.assert_array_equal(k_i8[:, :, :N].numpy(), ref["k_i8"])
    assert torch.all(q_i8[:, :, N:] == 0) and torch.all(k_i8[:, :, N:] == 0)
    np.testing.assert_array_equal(q_scale[:, :, :nq].numpy().view(np.uint32), ref["q_scale"].view(np.uint32))
    np.testing.assert_array_equal(k_scale[:, :, :nk].numpy().view(np.uint32), ref["k_scale"].view(np.uint32))
    assert torch.all(q_scale[:, :, nq:] == 0) and torch.all(k_scale[:, :, nk:] == 0)
    np.testing.assert_array_equal(k_mean.view(torch.int16).numpy().view(np.uint16), ref["k_mean"])


SHAPES = [
    synth.config(0),
    synth.custom(1, 1, 2, 64, tag=501),
    synth.custom(2, 63, 3, 64, tag=502),
    synth.custom(1, 65, 2, 128, tag=503),
    synth.custom(3, 200, 2, 128, tag=504),
    synth.custom(1, 777, 4, 128, tag=505),
]


@pytest.mark.parametrize("cfg", SHAPES, ids=lambda c: f"{c.name}-B{c.B}N{c.N}H{c.H}D{c.D}")
def test_norm_rope_bits(sage, cfg):
    _log(f"[producer] norm_rope {cfg.name} B{cfg.B} N{cfg.N} H{cfg.H} D{cfg.D}")
    q, k, _ = synth.make_qkv(cfg)
    wq, wk, rope = _consts(cfg)
    for x, w in ((q, wq), (k, wk)):
        ref, bad = oracle.norm_rope(x, w, rope.numpy())
        got = sage.norm_rope(x.cuda(), w.cuda(), rope.cuda())
        torch.cuda.synchronize()
        _log(f"  rows with a possibly inexact fp64 sum of squares: {bad}")
        assert torch.equal(got.cpu().view(torch.int16), ref.view(torch.int16))


def test_norm_rope_strided_views(sage):
    """Input read as a column slice of a wider projection output, output
    written into a wider buffer; eps 0 and 1e-2."""
    cfg = synth.custom(2, 130, 3, 128, tag=506)
    _log("[producer] strided views")
    q, _, _ = synth.make_qkv(cfg)
    wq, _, rope = _consts(cfg)
    B, N, H, D = q.shape
    wide = torch.zeros(B, N, H * D + 384, dtype=torch.bfloat16)
    wide[:, :, 256:256 + H * D] = q.reshape(B, N, H * D)
    xv = wide.cuda()[:, :, 256:256 + H * D].view(B, N, H, D)
    obuf = torch.zeros(B, N, H * D + 128, dtype=torch.bfloat16, device="cuda")
    ov = obuf[:, :, 128:].view(B, N, H, D)
    for eps in (0.0, 1e-2):
        sage.norm_rope(xv, wq.cuda(), rope.cuda(), eps=eps, out=ov)
        torch.cuda.synchronize()
        ref, _ = oracle.norm_rope(q, wq, rope.numpy(), eps)
        assert torch.equal(ov.cpu().view(torch.int16), ref.view(torch.int16))
    assert torch.all(obuf[:, :, :128] == 0)


@pytest.mark.parametrize("qb,kb", [(32, 64), (1, 16)], ids=str)
@pytest.mark.parametrize("cfg", SHAPES, ids=lambda c: f"{c.name}-B{c.B}N{c.N}H{c.H}D{c.D}")
def test_fused_producer_quant(sage, cfg, qb, kb):
    """sage_norm_rope_quant_qk == oracle quant_qk(norm_rope(q), norm_rope(k))
    bit for bit, and == the composed GPU path."""
    _log(f"[producer] fused quant q_block {qb} k_block {kb} {cfg.name} B{cfg.B} N{cfg.N} H{cfg.H} D{cfg.D}")
    q, k, _ = synth.make_qkv(cfg)
    wq, wk, rope = _consts(cfg)
    yq, _ = oracle.norm_rope(q, wq, rope.numpy())
    yk, _ = oracle.norm_rope(k, wk, rope.numpy())
    ref = oracle.quant_qk(yq, yk, q_block=qb, k_block=kb)
    qd, kd, wqd, wkd, rd = q.cuda(), k.cuda(), wq.cuda(), wk.cuda(), rope.cuda()
    fused = sage.norm_rope_quant_qk(qd, kd, wqd, wkd, rd, q_block=qb, k_block=kb)
    composed = sage.quant_qk(sage.norm_rope(qd, wqd, rd), sage.norm_rope(kd, wkd, rd),
                             q_block=qb, k_block=kb)
    torch.cuda.synchronize()
    for a, b in zip(fused, composed):
        assert torch.equal(a, b)
    _check_qk(fused, ref, cfg.N)


def test_fused_producer_flux_workload(sage):
    """FLUX joint shape from pre-norm Q and K: fused quantiser bit-exact in
    full; attention on every 16th query row within the oracle bar."""
    cfg = synth.config(1)
    _log(f"[producer] workload {cfg.name} B{cfg.B} N{cfg.N} H{cfg.H} D{cfg.D}")
    q, k, v = synth.make_qkv(cfg)
    wq, wk, rope = _consts(cfg)
    yq, bq = oracle.norm_rope(q, wq, rope.numpy())
    yk, bk = oracle.norm_rope(k, wk, rope.numpy())
    _log(f"  rows with a possibly inexact fp64 sum of squares: Q {bq}, K {bk}")
    ref, ref_v = oracle.quant_qk(yq, yk), oracle.quant_v(v)
    assert ref["inexact"] == 0
    qk = sage.norm_rope_quant_qk(q.cuda(), k.cuda(), wq.cuda(), wk.cuda(), rope.cuda())
    vq = sage.quant_v(v.cuda())
    out = sage.attn_fwd(*qk[:4], *vq, N=cfg.N)
    torch.cuda.synchronize()
    _check_qk(qk, ref, cfg.N)
    rows = synth.query_subset(cfg.N, every=16)
    got = out.float().cpu()[:, rows].permute(0, 2, 1, 3).double().numpy()
    _log(f"  rows {rows.size}/{cfg.N}")
    check_attention(got, oracle.attn_tiled(ref, ref_v, rows=rows), ref_v["v_mean"], log=_log)
