"""GPU parity of one rank's share under sequence parallelism ("FLUX 3 Action"
SGLang page, §3.1 Multi-GPU: the joint sequence is split and K/V are
gathered): sage_quant_q on the rank's token shard of Q, then
sage_attn_fwd_shard of those queries against the quantised K/V of the whole
sequence, through the C ABI.

Bar: the shard's Q codes and scales bit-exact against the oracle's quantiser on
the shard and bit-identical to the matching rows of the whole-sequence
sage_quant_qk_ex; the shard's attention bit-identical to the matching rows of
the whole-sequence sage_attn_fwd_ex (same key loop and roundings) and within
5e-3 relative L2 of the oracle's tiled attention on those rows.
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


def _shards(N, P):
    """P contiguous token shards of a multiple of 64 tokens each (the last one
    takes the rest): the shard starts stay on Q-block and key-tile bounds."""
    size = math.ceil(N / P / 64) * 64
    return [(a, min(N, a + size)) for a in range(0, N, size)]


def _rows_gathered(out_nhd, rows):
    return out_nhd.float().cpu()[:, rows].permute(0, 2, 1, 3).double().numpy()


@pytest.mark.parametrize("q_block", [32, 1])
@pytest.mark.parametrize("cfg", [synth.config(0), synth.custom(2, 777, 3, 128, tag=701),
                                 synth.custom(1, 130, 2, 64, tag=702)],
                         ids=lambda c: f"{c.name}-B{c.B}N{c.N}H{c.H}D{c.D}")
def test_quant_q_alone(sage, cfg, q_block):
    """sage_quant_q == the Q half of sage_quant_qk_ex == the oracle, bit for bit,
    on the whole sequence and on a token shard read in place from Q."""
    _log(f"[shard] quant_q {cfg.name} B{cfg.B} N{cfg.N} H{cfg.H} D{cfg.D} q_block {q_block}")
    q, k, _ = synth.make_qkv(cfg)
    qd, kd = q.cuda(), k.cuda()
    full = sage.quant_qk(qd, kd, q_block=q_block)
    alone = sage.quant_q(qd, q_block=q_block)
    torch.cuda.synchronize()
    assert torch.equal(alone[0], full[0]) and torch.equal(alone[1], full[1])
    ref = oracle.quant_qk(q, k, q_block=q_block)
    N, nq = cfg.N, math.ceil(cfg.N / q_block)
    np.testing.assert_array_equal(alone[0].cpu()[:, :, :N].numpy(), ref["q_i8"])
    np.testing.assert_array_equal(alone[1].cpu()[:, :, :nq].numpy().view(np.uint32),
                                  ref["q_scale"].view(np.uint32))
    if N > 64:
        a, b = 64, N  # a shard starting on a block bound, read as a strided view
        sh = sage.quant_q(qd[:, a:b], q_block=q_block)
        torch.cuda.synchronize()
        rs = oracle.quant_qk(q[:, a:b].contiguous(), k[:, a:b].contiguous(), q_block=q_block)
        np.testing.assert_array_equal(sh[0].cpu()[:, :, :b - a].numpy(), rs["q_i8"])
        np.testing.assert_array_equal(sh[0].cpu()[:, :, :b - a].numpy(),
                                      full[0].cpu()[:, :, a:b].numpy())
        assert torch.all(sh[0][:, :, b - a:] == 0)


def _check_shards(sage, cfg, P, q_block=32, k_block=64, oracle_rows=None, exact_full=True):
    q, k, v = synth.make_qkv(cfg)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    qk = sage.quant_qk(qd, kd, q_block=q_block, k_block=k_block)
    vq = sage.quant_v(vd)
    full = sage.attn_fwd(*qk[:4], *vq, N=cfg.N)
    torch.cuda.synchronize()
    ref_qk = ref_v = None
    for (a, b) in _shards(cfg.N, P):
        q_i8, q_scale = sage.quant_q(qd[:, a:b], q_block=q_block)
        out = sage.attn_fwd_shard(q_i8, q_scale, b - a, qk[2], qk[3], *vq, Nk=cfg.N)
        torch.cuda.synchronize()
        same = torch.equal(out.view(torch.int16), full[:, a:b].view(torch.int16))
        _log(f"  shard [{a}, {b}) of {cfg.N}: bit-identical to the whole-sequence rows: {same}")
        assert same
        if oracle_rows is not None:
            if ref_qk is None:
                ref_qk = oracle.quant_qk(q, k, q_block=q_block, k_block=k_block)
                ref_v = oracle.quant_v(v)
            loc = np.array([r for r in oracle_rows(b - a)], np.int32)
            got = _rows_gathered(out, loc)
            tiled = oracle.attn_tiled(ref_qk, ref_v, rows=(loc + a).astype(np.int32))
            _log(f"    rows {loc.size}")
            check_attention(got, tiled, ref_v["v_mean"], log=_log)


@pytest.mark.parametrize("qb,kb", [(32, 64), (1, 16)], ids=str)
@pytest.mark.parametrize("cfg,P", [(synth.config(0), 2), (synth.custom(2, 777, 3, 128, tag=703), 4),
                                   (synth.custom(1, 1000, 2, 64, tag=704), 3),
                                   (synth.custom(1, 100, 2, 128, tag=705), 2)],
                         ids=lambda x: f"{x.name}-N{x.N}" if hasattr(x, "name") else f"P{x}")
def test_shards_equal_whole_sequence_rows(sage, cfg, P, qb, kb):
    """Every shard's output equals the matching rows of the whole-sequence
    attention bit for bit; all rows checked against the oracle."""
    _log(f"[shard] {cfg.name} B{cfg.B} N{cfg.N} H{cfg.H} D{cfg.D} P{P} q_block {qb} k_block {kb}")
    _check_shards(sage, cfg, P, qb, kb, oracle_rows=lambda n: range(n))


def test_rank_share_long_t2v(sage):
    """Long T2V (B1 H40 N32760 D128) split 8 ways: the shards of 4096 tokens and
    the ragged last one (4088) against all 32760 keys; six sampled rows of every
    shard against the oracle."""
    cfg = synth.config(3)
    _log(f"[shard] rank share {cfg.name} B{cfg.B} N{cfg.N} H{cfg.H} D{cfg.D} P8")
    _check_shards(sage, cfg, 8, oracle_rows=lambda n: [0, 1, 31, 32, n // 2, n - 1])
