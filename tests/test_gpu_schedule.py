"""The attention's two key-step schedules (the compiler's order, and the MFMAs
spread through the softmax with the previous tile's P.V first) run the same
operations on the same values, so their outputs must be bit-identical: for
both workgroup sizes, both K block sizes, D 64 and 128, ragged and padded key
counts.  Each schedule's distance from the oracle is covered by the parity
tests, which run the default one."""
import sys

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


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


# Key-tile counts: 5 (N300: no steady group, so no deferred PV), 6 (N384 and the
# ragged N350: exactly one steady group, then the flush and the last steps),
# 13, 16 and 72 (several groups).
@pytest.mark.parametrize("shape", [(1, 300, 3, 64), (1, 384, 2, 128), (1, 350, 3, 64), (1, 1000, 2, 128),
                                   (2, 777, 5, 128), (1, 4608, 6, 128)],
                         ids=["N300-D64", "N384-D128", "N350-D64", "N1000-D128", "B2-N777", "N4608"])
@pytest.mark.parametrize("k_block", [64, 16])
@pytest.mark.parametrize("waves", [4, 8])
def test_schedules_bit_identical(sage, shape, k_block, waves):
    B, N, H, D = shape
    cfg = synth.custom(B, N, H, D, tag=500)
    _log(f"[schedule] B{B} N{N} H{H} D{D} k_block {k_block} waves {waves}")
    q, k, v = (t.cuda() for t in synth.make_qkv(cfg))
    qk = sage.quant_qk(q, k, k_block=k_block)
    vq = sage.quant_v(v)
    outs = []
    try:
        sage.sage_attn_tuning(waves)
        for sched in (1, 2):
            sage.sage_attn_schedule(sched)
            outs.append(sage.attn_fwd(*qk[:4], *vq, N))
        torch.cuda.synchronize()
    finally:
        sage.sage_attn_schedule(0)
        sage.sage_attn_tuning(0)
    a, b = (o.view(torch.int16) for o in outs)
    _log(f"  differing outputs: {int((a != b).sum())} of {a.numel()}")
    assert torch.isfinite(outs[0].float()).all()
    assert torch.equal(a, b)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("k_block", [64, 16])
@pytest.mark.parametrize("waves", [4, 8])
def test_forced_workgroup_size_against_oracle(sage, D, k_block, waves):
    """The default schedule under either workgroup size (forced) against the
    oracle's tiled attention, on a ragged key count with several steady groups
    (13 key tiles): the default shapes reach eight-wave workgroups only at D=128
    and with 64-token K blocks."""
    import oracle
    from tests.attn_bars import check_attention
    B, N, H = 1, 777, 2
    cfg = synth.custom(B, N, H, D, tag=510)
    _log(f"[oracle] B{B} N{N} H{H} D{D} k_block {k_block} waves {waves}")
    q, k, v = synth.make_qkv(cfg)
    ref_qk, ref_v = oracle.quant_qk(q, k, k_block=k_block), oracle.quant_v(v)
    qk = sage.quant_qk(q.cuda(), k.cuda(), k_block=k_block)
    vq = sage.quant_v(v.cuda())
    try:
        sage.sage_attn_tuning(waves)
        out = sage.attn_fwd(*qk[:4], *vq, N)
        torch.cuda.synchronize()
    finally:
        sage.sage_attn_tuning(0)
    got = out.float().cpu().permute(0, 2, 1, 3).double().numpy()
    tiled = oracle.attn_tiled(ref_qk, ref_v)
    check_attention(got, tiled, ref_v["v_mean"], log=_log)
