"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: bit-exact INT8 Q/K codes, FP8 V codes, all scales and means (padding
included); attention within relative L2 <= 5e-3 of the oracle's quantised
tiled path (also per (b, h), on the attention term O - v_mean, and with a
max-abs guard: tests/attn_bars.py) and <= 3e-2 of exact fp64 attention.  On
the tiny workload the method itself is ~3.6e-2 from exact attention (FP8
rounding of P and V), so there the exact-attention bar is a strict xfail: the
conflict shows in the results instead of passing.
"""
import hashlib
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
TOL_EXACT = 3e-2


def _log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def sage():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_attention_video_smooth_amd as s
    s.lib()  # raises if the library is missing
    return s


def _gpu_quant(sage, q, k, v, q_block=32, k_block=64):
    dev = torch.device("cuda")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    qk = sage.quant_qk(qd, kd, q_block=q_block, k_block=k_block)
    vq = sage.quant_v(vd)
    torch.cuda.synchronize()
    return qd, kd, vd, qk, vq


def _check_quant_bits(qk, vq, ref_qk, ref_v, N):
    q_i8, q_scale, k_i8, k_scale, k_mean = [t.cpu() for t in qk]
    v_fp8, v_scale, v_mean = [t.cpu() for t in vq]
    nq, nk = math.ceil(N / ref_qk.get("q_block", 32)), math.ceil(N / ref_qk.get("k_block", 64))
    np.testing.assert_array_equal(q_i8[:, :, :N].numpy(), ref_qk["q_i8"])
    np.testing.assert_array_equal(k_i8[:, :, :N].numpy(), ref_qk["k_i8"])
    assert torch.all(q_i8[:, :, N:] == 0) and torch.all(k_i8[:, :, N:] == 0)
    np.testing.assert_array_equal(q_scale[:, :, :nq].numpy().view(np.uint32), ref_qk["q_scale"].view(np.uint32))
    assert torch.all(q_scale[:, :, nq:] == 0)
    np.testing.assert_array_equal(k_scale[:, :, :nk].numpy().view(np.uint32), ref_qk["k_scale"].view(np.uint32))
    assert torch.all(k_scale[:, :, nk:] == 0)
    np.testing.assert_array_equal(k_mean.view(torch.int16).numpy().view(np.uint16), ref_qk["k_mean"])
    np.testing.assert_array_equal(v_fp8.numpy(), ref_v["v_fp8"])
    np.testing.assert_array_equal(v_scale.numpy().view(np.uint32), ref_v["v_scale"].view(np.uint32))
    np.testing.assert_array_equal(v_mean.numpy().view(np.uint32), ref_v["v_mean"].view(np.uint32))


def _rows_gathered(out_nhd, rows):
    # out [B,N,H,D] -> [B,H,len(rows),D] fp64
    return out_nhd.float().cpu()[:, rows].permute(0, 2, 1, 3).double().numpy()


def _tiled_by_heads(ref_qk, ref_v, rows, cfg, group=8):
    """The oracle's tiled attention, a group of heads per call (with a progress
    line per group: the long workload takes minutes on the host)."""
    parts = []
    for h0 in range(0, cfg.H, group):
        sl = slice(h0, min(cfg.H, h0 + group))
        sub_qk = {k2: (v2[:, sl] if isinstance(v2, np.ndarray) and v2.ndim >= 3 else v2)
                  for k2, v2 in ref_qk.items()}
        sub_v = {k2: (v2[:, sl] if isinstance(v2, np.ndarray) and v2.ndim >= 3 else v2)
                 for k2, v2 in ref_v.items()}
        parts.append(oracle.attn_tiled(sub_qk, sub_v, rows=rows))
        _log(f"  oracle heads {sl.start}..{sl.stop - 1} done")
    return np.concatenate(parts, axis=1)


SMALL = [
    synth.config(0),
    synth.custom(1, 1, 2, 64, tag=301),
    synth.custom(2, 63, 3, 64, tag=302),
    synth.custom(1, 65, 2, 128, tag=303),
    synth.custom(3, 200, 2, 128, tag=304),
    synth.custom(1, 777, 4, 128, tag=305),
    synth.custom(2, 1000, 1, 64, tag=306),
    # 640 heads: more heads than workgroups of one wave of the grid
    synth.custom(4, 100, 160, 64, tag=309),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: f"{c.name}-B{c.B}N{c.N}H{c.H}D{c.D}")
def test_small_shapes_full(sage, cfg):
    _log(f"[parity] {cfg.name} B{cfg.B} N{cfg.N} H{cfg.H} D{cfg.D}")
    q, k, v = synth.make_qkv(cfg)
    ref_qk, ref_v = oracle.quant_qk(q, k), oracle.quant_v(v)
    assert ref_qk["inexact"] == 0 and ref_v["bad"] == 0
    qd, kd, vd, qk, vq = _gpu_quant(sage, q, k, v)
    _check_quant_bits(qk, vq, ref_qk, ref_v, cfg.N)
    out = sage.attn_fwd(*qk[:4], *vq, N=cfg.N)
    torch.cuda.synchronize()
    got = _rows_gathered(out, np.arange(cfg.N))
    tiled = oracle.attn_tiled(ref_qk, ref_v)
    exact = oracle.attn_exact(q, k, v)
    e_or, e_ex, e_me = oracle.rel_l2(got, tiled), oracle.rel_l2(got, exact), oracle.rel_l2(tiled, exact)
    _log(f"  rel L2: gpu-vs-oracle {e_or:.3e}  gpu-vs-exact {e_ex:.3e}  oracle-vs-exact {e_me:.3e}")
    check_attention(got, tiled, vq[2].cpu().numpy(), log=_log)
    if cfg.N == 1:
        np.testing.assert_array_equal(got, exact.astype(np.float32).astype(np.float64))
    if cfg.name != "tiny":
        assert e_ex <= TOL_EXACT


@pytest.mark.xfail(strict=True, reason="method conflict: on the tiny workload (no V mean offset, N=256) "
                   "E4M3 rounding of both P and V puts the method itself ~3.6e-2 from exact fp64 "
                   "attention, above the 3e-2 bar; the oracle's quantised path is as far")
def test_tiny_exact_bar(sage):
    cfg = synth.config(0)
    q, k, v = synth.make_qkv(cfg)
    _, _, _, qk, vq = _gpu_quant(sage, q, k, v)
    out = sage.attn_fwd(*qk[:4], *vq, N=cfg.N)
    torch.cuda.synchronize()
    e_ex = oracle.rel_l2(_rows_gathered(out, np.arange(cfg.N)), oracle.attn_exact(q, k, v))
    _log(f"[parity] tiny gpu-vs-exact {e_ex:.3e} (bar {TOL_EXACT})")
    assert e_ex <= TOL_EXACT


WORKLOADS = [1, 2]


@pytest.mark.parametrize("idx", WORKLOADS)
def test_workload_quant_bits_and_attention(sage, idx):
    cfg = synth.config(idx)
    _log(f"[parity] workload {cfg.name} B{cfg.B} N{cfg.N} H{cfg.H} D{cfg.D}")
    q, k, v = synth.make_qkv(cfg)
    ref_qk, ref_v = oracle.quant_qk(q, k), oracle.quant_v(v)
    assert ref_qk["inexact"] == 0 and ref_v["bad"] == 0
    qd, kd, vd, qk, vq = _gpu_quant(sage, q, k, v)
    _check_quant_bits(qk, vq, ref_qk, ref_v, cfg.N)
    out = sage.attn_fwd(*qk[:4], *vq, N=cfg.N)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    # every query row against the oracle's tiled path
    got = _rows_gathered(out, np.arange(cfg.N))
    tiled = _tiled_by_heads(ref_qk, ref_v, None, cfg)
    check_attention(got, tiled, ref_v["v_mean"], log=_log, label=f"all {cfg.N} rows ")
    # every 8th 32-query block plus the last against exact fp64 attention
    rows = synth.query_subset(cfg.N, every=8)
    exact = oracle.attn_exact(q, k, v, rows=rows)
    e_ex = oracle.rel_l2(_rows_gathered(out, rows), exact)
    _log(f"  rows {rows.size}/{cfg.N}: gpu-vs-exact {e_ex:.3e}  "
         f"oracle-vs-exact {oracle.rel_l2(tiled[:, :, rows], exact):.3e}")
    assert e_ex <= TOL_EXACT


def test_long_workload_sampled(sage):
    """Long T2V shape (B1 H40 N32760 D128): quantised outputs bit-exact in full;
    attention on sampled query rows of every head."""
    cfg = synth.config(3)
    _log(f"[parity] workload {cfg.name} B{cfg.B} N{cfg.N} H{cfg.H} D{cfg.D}")
    q, k, v = synth.make_qkv(cfg)
    ref_qk, ref_v = oracle.quant_qk(q, k), oracle.quant_v(v)
    assert ref_qk["inexact"] == 0 and ref_v["bad"] == 0
    qd, kd, vd, qk, vq = _gpu_quant(sage, q, k, v)
    _check_quant_bits(qk, vq, ref_qk, ref_v, cfg.N)
    out = sage.attn_fwd(*qk[:4], *vq, N=cfg.N)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    # the stratified subset: every 8th 32-query block of every head plus the last
    rows = synth.query_subset(cfg.N, every=8)
    got = _rows_gathered(out, rows)
    tiled = _tiled_by_heads(ref_qk, ref_v, rows, cfg)
    check_attention(got, tiled, ref_v["v_mean"], log=_log, label=f"rows {rows.size}/{cfg.N} ")
    # exact fp64 attention on every 64th block plus the last
    rows_x = synth.query_subset(cfg.N, every=64)
    exact = oracle.attn_exact(q, k, v, rows=rows_x)
    sel = np.searchsorted(rows, rows_x)
    assert np.array_equal(rows[sel], rows_x)
    e_ex = oracle.rel_l2(got[:, :, sel], exact)
    _log(f"  rows {rows_x.size}/{cfg.N}: gpu-vs-exact {e_ex:.3e}")
    assert e_ex <= TOL_EXACT


def test_quant_long_bits(sage):
    """Standalone quant shape (B1 H40 N32760 D128, offsets N(0,4) on Q, K and V)."""
    cfg = synth.config(4)
    _log(f"[parity] workload {cfg.name} quant only")
    q, k, v = synth.make_qkv(cfg)
    ref_qk, ref_v = oracle.quant_qk(q, k), oracle.quant_v(v)
    assert ref_qk["inexact"] == 0 and ref_v["bad"] == 0
    qd, kd, vd, qk, vq = _gpu_quant(sage, q, k, v)
    _check_quant_bits(qk, vq, ref_qk, ref_v, cfg.N)


def test_strided_v_alias_and_strided_out(sage):
    """V read as a column slice of a wider projection output; output written into
    a wider buffer."""
    cfg = synth.custom(2, 300, 3, 128, tag=307)
    _log("[parity] strided V / out")
    q, k, v = synth.make_qkv(cfg)
    B, N, H, D = q.shape
    wide = torch.zeros(B, N, H * D + 256, dtype=torch.bfloat16)
    wide[:, :, 128:128 + H * D] = v.reshape(B, N, H * D)
    wide_d = wide.cuda()
    v_view = wide_d[:, :, 128:128 + H * D].view(B, N, H, D)
    vq = sage.quant_v(v_view)
    vq_ref = sage.quant_v(v.cuda())
    torch.cuda.synchronize()
    for a, b in zip(vq, vq_ref):
        assert torch.equal(a, b)
    ref_v = oracle.quant_v(wide[:, :, 128:128 + H * D].view(B, N, H, D))
    np.testing.assert_array_equal(vq[0].cpu().numpy(), ref_v["v_fp8"])
    qk = sage.quant_qk(q.cuda(), k.cuda())
    obuf = torch.zeros(B, N, H * D + 64, dtype=torch.bfloat16, device="cuda")
    o_view = obuf[:, :, 64:].view(B, N, H, D)
    sage.attn_fwd(*qk[:4], *vq, N=N, out=o_view)
    o_ref = sage.attn_fwd(*qk[:4], *vq, N=N)
    torch.cuda.synchronize()
    assert torch.equal(o_view, o_ref)
    assert torch.all(obuf[:, :, :64] == 0)


def test_determinism_sha256(sage):
    cfg = synth.config(2)
    _log("[parity] determinism x3")
    q, k, v = (t.cuda() for t in synth.make_qkv(cfg))
    digests = set()
    for _ in range(3):
        qk = sage.quant_qk(q, k)
        vq = sage.quant_v(v)
        out = sage.attn_fwd(*qk[:4], *vq, N=cfg.N)
        torch.cuda.synchronize()
        h = hashlib.sha256()
        for t in (*qk, *vq, out):
            h.update(t.contiguous().view(torch.uint8).cpu().numpy().tobytes())
        digests.add(h.hexdigest())
    assert len(digests) == 1


def test_sm_scale_argument(sage):
    cfg = synth.custom(1, 130, 2, 64, tag=308)
    q, k, v = synth.make_qkv(cfg)
    ref_qk, ref_v = oracle.quant_qk(q, k), oracle.quant_v(v)
    qk = sage.quant_qk(q.cuda(), k.cuda())
    vq = sage.quant_v(v.cuda())
    out = sage.attn_fwd(*qk[:4], *vq, N=cfg.N, sm_scale=0.05)
    torch.cuda.synchronize()
    got = _rows_gathered(out, np.arange(cfg.N))
    check_attention(got, oracle.attn_tiled(ref_qk, ref_v, sm_scale=0.05), ref_v["v_mean"], log=_log)


def test_errors_enqueue_nothing(sage):
    q = torch.zeros(1, 64, 2, 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sage.SageError) as e:
        sage.quant_qk(q, q)
    assert e.value.status == -3


def test_quant_single_long_head(sage):
    """One head of 270000 tokens at D=128: every statistics chunk is long and
    the quantised tensors span 33 MB per head."""
    cfg = synth.custom(1, 270000, 1, 128, tag=311)
    _log(f"[parity] long head B{cfg.B} N{cfg.N} H{cfg.H} D{cfg.D} quant only")
    q, k, v = synth.make_qkv(cfg)
    ref_qk, ref_v = oracle.quant_qk(q, k), oracle.quant_v(v)
    assert ref_qk["inexact"] == 0 and ref_v["bad"] == 0
    _, _, _, qk, vq = _gpu_quant(sage, q, k, v)
    _check_quant_bits(qk, vq, ref_qk, ref_v, cfg.N)


@pytest.mark.parametrize("k_block", [64, 16])
@pytest.mark.parametrize("D", [64, 128])
def test_degenerate_inputs(sage, D, k_block):
    """Zero and subnormal quantisation blocks (scale 0, codes 0 through the
    zero guard when 127/a or 448/a overflows), a head with constant K (all
    scores 0: uniform attention) and a constant V channel (scale 0: the output
    channel is bf16(v_mean) exactly)."""
    cfg = synth.custom(2, 200, 3, D, tag=312)
    _log(f"[parity] degenerate inputs B{cfg.B} N{cfg.N} H{cfg.H} D{D} k_block {k_block}")
    q, k, v = synth.make_qkv(cfg)
    tiny = torch.tensor(1e-40, dtype=torch.bfloat16)          # a bf16 subnormal
    assert 0 < float(tiny) < 1.2e-38
    q[:, 32:64] = 0                                           # a zero Q block, every head
    q[:, 64:96, 0] = tiny                                     # a subnormal Q block of head 0
    k[:, :, 2] = k[0, 0, 2]                                   # head 2: K constant over tokens
    v[:, :, 1, 7] = 2.5                                       # a constant V channel
    sign = torch.where(torch.arange(cfg.N) % 2 == 0, 1.0, -1.0).to(torch.bfloat16)
    v[:, :, 0, 3] = tiny * sign[None, :]                      # a V channel of +-subnormals
    ref_qk, ref_v = oracle.quant_qk(q, k, k_block=k_block), oracle.quant_v(v)
    assert ref_qk["inexact"] == 0 and ref_v["bad"] == 0
    assert np.all(ref_qk["q_scale"][:, :, 1] == 0) and np.all(ref_qk["q_scale"][:, 0, 2] == 0)
    assert np.all(ref_qk["k_scale"][:, 2] == 0)
    assert np.all(ref_v["v_scale"][:, 1, 7] == 0) and np.all(ref_v["v_scale"][:, 0, 3] == 0)
    qd, kd, vd, qk, vq = _gpu_quant(sage, q, k, v, k_block=k_block)
    _check_quant_bits(qk, vq, ref_qk, ref_v, cfg.N)
    out = sage.attn_fwd(*qk[:4], *vq, N=cfg.N)
    torch.cuda.synchronize()
    got = _rows_gathered(out, np.arange(cfg.N))
    tiled = oracle.attn_tiled(ref_qk, ref_v)
    check_attention(got, tiled, ref_v["v_mean"], log=_log)
    # the constant channel comes back as bf16(v_mean) in every row
    vm = torch.tensor(ref_v["v_mean"][:, 1, 7]).to(torch.bfloat16)
    col = out[:, :, 1, 7].cpu()
    assert torch.equal(col, vm[:, None].expand_as(col))
    # head 2 (constant K): every query sees the same uniform weights
    o2 = out[:, :, 2].float().cpu()
    assert torch.equal(o2, o2[:, :1].expand_as(o2))


GRAN_SHAPES = [
    synth.config(0),
    synth.custom(2, 63, 3, 64, tag=302),
    # N = 65 and 200: the last key tile holds 16-key blocks wholly beyond N
    synth.custom(1, 65, 2, 128, tag=303),
    synth.custom(3, 200, 2, 128, tag=304),
    synth.custom(1, 777, 4, 128, tag=305),
]
GRANS = [(1, 64), (32, 16), (1, 16)]


@pytest.mark.parametrize("qb,kb", GRANS, ids=lambda g: str(g))
@pytest.mark.parametrize("cfg", GRAN_SHAPES, ids=lambda c: f"{c.name}-B{c.B}N{c.N}H{c.H}D{c.D}")
def test_granularity_full(sage, cfg, qb, kb):
    """One Q scale per token (q_block 1) and/or four K scales per key tile
    (k_block 16): codes and scales bit-exact against the oracle at the same
    granularity, the other tensor identical to the default run, attention
    within the oracle bar."""
    _log(f"[parity] q_block {qb} k_block {kb} {cfg.name} B{cfg.B} N{cfg.N} H{cfg.H} D{cfg.D}")
    q, k, v = synth.make_qkv(cfg)
    ref_qk, ref_v = oracle.quant_qk(q, k, q_block=qb, k_block=kb), oracle.quant_v(v)
    assert ref_qk["inexact"] == 0 and ref_v["bad"] == 0
    qd, kd, vd, qk, vq = _gpu_quant(sage, q, k, v, q_block=qb, k_block=kb)
    assert qk[1].shape[-1] == qk[0].shape[2] // qb and qk[3].shape[-1] == qk[2].shape[2] // kb
    _check_quant_bits(qk, vq, ref_qk, ref_v, cfg.N)
    dflt = sage.quant_qk(qd, kd)
    torch.cuda.synchronize()
    same = ([0, 1] if qb == 32 else []) + ([2, 3] if kb == 64 else []) + [4]
    for i in same:
        assert torch.equal(qk[i], dflt[i])
    out = sage.attn_fwd(*qk[:4], *vq, N=cfg.N)
    torch.cuda.synchronize()
    got = _rows_gathered(out, np.arange(cfg.N))
    tiled = oracle.attn_tiled(ref_qk, ref_v)
    exact = oracle.attn_exact(q, k, v)
    e_or, e_ex = oracle.rel_l2(got, tiled), oracle.rel_l2(got, exact)
    e_dflt = oracle.rel_l2(oracle.attn_tiled(oracle.quant_qk(q, k), ref_v), exact)
    _log(f"  rel L2: gpu-vs-oracle {e_or:.3e}  gpu-vs-exact {e_ex:.3e}  "
         f"default-oracle-vs-exact {e_dflt:.3e}")
    check_attention(got, tiled, ref_v["v_mean"], log=_log)
    if cfg.name != "tiny":  # tiny: the method conflict recorded by test_tiny_exact_bar
        assert e_ex <= TOL_EXACT


@pytest.mark.parametrize("qb,kb", GRANS, ids=lambda g: str(g))
def test_granularity_workload_sampled(sage, qb, kb):
    """FLUX joint shape at the finer granularities: quantised outputs bit-exact
    in full, attention on every 8th 32-query block plus the last."""
    cfg = synth.config(1)
    _log(f"[parity] q_block {qb} k_block {kb} workload {cfg.name} B{cfg.B} N{cfg.N} H{cfg.H} D{cfg.D}")
    q, k, v = synth.make_qkv(cfg)
    ref_qk, ref_v = oracle.quant_qk(q, k, q_block=qb, k_block=kb), oracle.quant_v(v)
    qd, kd, vd, qk, vq = _gpu_quant(sage, q, k, v, q_block=qb, k_block=kb)
    _check_quant_bits(qk, vq, ref_qk, ref_v, cfg.N)
    out = sage.attn_fwd(*qk[:4], *vq, N=cfg.N)
    torch.cuda.synchronize()
    rows = synth.query_subset(cfg.N, every=8)
    got = _rows_gathered(out, rows)
    tiled = oracle.attn_tiled(ref_qk, ref_v, rows=rows)
    exact = oracle.attn_exact(q, k, v, rows=rows)
    e_ex = oracle.rel_l2(got, exact)
    _log(f"  rows {rows.size}/{cfg.N}: gpu-vs-exact {e_ex:.3e}")
    check_attention(got, tiled, ref_v["v_mean"], log=_log)
    assert e_ex <= TOL_EXACT


def test_plain_entry_points_equal_ex(sage):
    """sage_quant_qk / sage_attn_fwd are the q_block 32 case of the _ex calls,
    bit for bit."""
    cfg = synth.custom(2, 300, 3, 128, tag=313)
    q, k, v = (t.cuda() for t in synth.make_qkv(cfg))
    B, N, H, D = q.shape
    qk = sage.quant_qk(q, k)
    vq = sage.quant_v(v)
    out = sage.attn_fwd(*qk[:4], *vq, N=N)
    torch.cuda.synchronize()
    lib = sage.lib()
    plain = [torch.empty_like(t) for t in qk]
    ws = torch.zeros(lib.sage_quant_qk_workspace_size(B, N, H, D), dtype=torch.uint8, device="cuda")
    qs = [x for x in q.stride()[:3]]
    ks = [x for x in k.stride()[:3]]
    st = lib.sage_quant_qk(q.data_ptr(), *qs, k.data_ptr(), *ks, B, N, H, D,
                           *[t.data_ptr() for t in plain], ws.data_ptr(), ws.numel(),
                           torch.cuda.current_stream().cuda_stream)
    assert st == 0
    o2 = torch.empty_like(out)
    st = lib.sage_attn_fwd(*[t.data_ptr() for t in plain[:4]], *[t.data_ptr() for t in vq],
                           B, N, H, D, 0.0, o2.data_ptr(), *o2.stride()[:3],
                           torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    for a, b in zip(qk, plain):
        assert torch.equal(a, b)
    assert torch.equal(out, o2)


def _tiny_channel(N, tiny):
    """Token 0: tiny, tokens 1..N-2: +1, -1, ..., token N-1: 0 (N even): the
    exact sum is `tiny`; an fp64 running sum that meets +1 after it loses it."""
    col = np.zeros(N)
    col[0] = tiny
    col[1:N - 1] = np.where(np.arange(N - 2) % 2 == 0, 1.0, -1.0)
    return torch.from_numpy(col).to(torch.bfloat16)


@pytest.mark.parametrize("shape,tiny", [((1, 4608, 2, 64), 2.0 ** -100), ((1, 4608, 2, 64), 2.0 ** -133),
                                        ((2, 32768, 3, 128), 2.0 ** -100)],
                         ids=["N4608-2^-100", "N4608-2^-133", "N32768-2^-100"])
def test_channel_sum_exact_fallback(sage, shape, tiny):
    """Reading R3 for channels where plain fp64 accumulation is not exact: one
    K and one V channel hold a tiny bf16 value (normal or subnormal) among
    +-1 values, plus a channel of random values with one subnormal.  The GPU
    detects them and sums them exactly: means, scales and codes bit-exact."""
    B, N, H, D = shape
    cfg = synth.custom(B, N, H, D, tag=404)
    _log(f"[parity] exact channel sums B{B} N{N} H{H} D{D} tiny 2^{math.log2(tiny):.0f}")
    q, k, v = synth.make_qkv(cfg)
    col = _tiny_channel(N, tiny)
    k[B - 1, :, H - 1, 5] = col
    v[0, :, H - 1, 9] = col
    k[0, 7, 0, 3] = 1e-40  # a subnormal among N(0,1)-like values
    v[B - 1, N // 2, 0, 0] = -1e-40
    ref_qk, ref_v = oracle.quant_qk(q, k), oracle.quant_v(v)
    assert ref_qk["inexact"] == 2 and ref_v["inexact"] == 2 and ref_v["bad"] == 0
    _, _, _, qk, vq = _gpu_quant(sage, q, k, v)
    _check_quant_bits(qk, vq, ref_qk, ref_v, N)
    if tiny == 2.0 ** -100:
        assert ref_v["v_mean"][0, H - 1, 9] == np.float32(tiny / N) != 0


def test_channel_sum_exact_fallback_producer(sage):
    """The same for the fused QK RMSNorm + RoPE producer: a pre-norm K channel
    pair (4, 5) holding a tiny value at token 0 and +-1 values elsewhere gives
    producer outputs with a tiny value among O(1) ones; the fallback sums the
    producer's outputs exactly (recomputing them per token)."""
    from tests.test_gpu_producer import _check_qk, _consts
    cfg = synth.custom(1, 2048, 2, 128, tag=405)
    _log("[parity] exact channel sums behind the fused producer")
    q, k, _ = synth.make_qkv(cfg)
    col = _tiny_channel(cfg.N, 2.0 ** -100)
    k[0, :, 1, 4] = col
    k[0, :, 1, 5] = 0
    wq, wk, rope = _consts(cfg)
    yq, _ = oracle.norm_rope(q, wq, rope.numpy())
    yk, _ = oracle.norm_rope(k, wk, rope.numpy())
    ref = oracle.quant_qk(yq, yk)
    _log(f"  oracle channels with an inexact plain sum: {ref['inexact']}")
    assert ref["inexact"] >= 1
    qk = sage.norm_rope_quant_qk(q.cuda(), k.cuda(), wq.cuda(), wk.cuda(), rope.cuda())
    torch.cuda.synchronize()
    _check_qk(qk, ref, cfg.N)
