"""Host-only checks of the C ABI: the library loads, exports every function that
include/sage.h declares, and rejects bad arguments with the documented status
codes without touching a GPU (sage_validate_*)."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sage.h")


@pytest.fixture(scope="module")
def sage():
    import quantized_attention_video_smooth_amd as s
    if not os.path.exists(s.LIB_PATH):
        from quantized_attention_video_smooth_amd import build
        build.build()
    s.lib()
    return s


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(sage_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_exports_every_declared_symbol(sage):
    names = _declared_functions()
    assert {"sage_quant_qk", "sage_quant_v", "sage_attn_fwd"} <= set(names)
    for n in names:
        assert hasattr(sage.lib(), n), n


def test_layout_and_slot_map(sage):
    import ctypes
    buf = (ctypes.c_int32 * 4)()
    assert sage.lib().sage_get_layout(ctypes.addressof(buf)) == 0
    assert list(buf) == [32, 64, 64, 1]
    assert sage.lib().sage_get_layout(None) == -1
    slots = [sage.sage_v_slot(t) for t in range(64)]
    assert sorted(slots) == list(range(64))
    assert sage.sage_v_slot(64) == -1 and sage.sage_v_slot(-1) == -1
    import oracle
    assert slots == [oracle.v_slot(t) for t in range(64)]
    assert [sage.sage_padded_tokens(n) for n in (1, 64, 65, 3128, 32760)] == [64, 64, 128, 3136, 32768]


A = 1 << 20  # fake, 16-byte aligned "device" addresses spaced far apart


def _qk_args(B=1, N=100, H=2, D=64, **over):
    Np = (N + 63) // 64 * 64
    a = dict(q=A, q_sb=N * H * D, q_sn=H * D, q_sh=D, k=2 * A, k_sb=N * H * D, k_sn=H * D, k_sh=D,
             B=B, N=N, H=H, D=D, q_i8=3 * A, q_scale=4 * A, k_i8=5 * A, k_scale=6 * A,
             k_mean=7 * A, ws=8 * A, ws_bytes=1 << 40)
    a.update(over)
    return a


def _vqk(sage, a):
    return sage.lib().sage_validate_quant_qk(a["q"], a["q_sb"], a["q_sn"], a["q_sh"], a["k"], a["k_sb"],
                                             a["k_sn"], a["k_sh"], a["B"], a["N"], a["H"], a["D"],
                                             a["q_i8"], a["q_scale"], a["k_i8"], a["k_scale"],
                                             a["k_mean"], a["ws"], a["ws_bytes"])


def test_validate_quant_qk_status_codes(sage):
    assert _vqk(sage, _qk_args()) == 0
    assert _vqk(sage, _qk_args(q=None)) == -1
    assert _vqk(sage, _qk_args(ws=None)) == -1
    assert _vqk(sage, _qk_args(N=0)) == -2
    assert _vqk(sage, _qk_args(B=0)) == -2
    assert _vqk(sage, _qk_args(D=96)) == -3
    assert _vqk(sage, _qk_args(q_sn=-128)) == -4
    assert _vqk(sage, _qk_args(k_sn=132)) == -5
    assert _vqk(sage, _qk_args(q=A + 8)) == -5
    assert _vqk(sage, _qk_args(ws_bytes=16)) == -6
    assert _vqk(sage, _qk_args(k_i8=3 * A + 64)) == -7          # overlaps q_i8
    assert _vqk(sage, _qk_args(q_scale=A + 256)) == -7          # output inside input q
    assert _vqk(sage, _qk_args(N=1 << 20, H=64, D=128, B=1)) == -2  # >= 2^31 elements
    # size-1 dimensions may carry any stride
    assert _vqk(sage, _qk_args(B=1, q_sb=3, k_sb=0)) == 0


def test_validate_quant_v_status_codes(sage):
    lib = sage.lib()
    ok = (A, 100 * 2 * 64, 2 * 64, 64, 1, 100, 2, 64, 2 * A, 3 * A, 4 * A, 5 * A, 1 << 40)
    assert lib.sage_validate_quant_v(*ok) == 0
    bad = list(ok); bad[8] = None
    assert lib.sage_validate_quant_v(*bad) == -1
    bad = list(ok); bad[2] = 2 * 64 + 4  # token stride breaks alignment
    assert lib.sage_validate_quant_v(*bad) == -5
    bad = list(ok); bad[8] = A + 512     # v_fp8 inside the input
    assert lib.sage_validate_quant_v(*bad) == -7
    bad = list(ok); bad[12] = 8
    assert lib.sage_validate_quant_v(*bad) == -6
    bad = list(ok); bad[7] = 32
    assert lib.sage_validate_quant_v(*bad) == -3


def test_validate_attn_status_codes(sage):
    lib = sage.lib()
    ok = (A, 2 * A, 3 * A, 4 * A, 5 * A, 6 * A, 7 * A, 1, 100, 2, 128, 8 * A, 100 * 2 * 128, 2 * 128, 128)
    assert lib.sage_validate_attn_fwd(*ok) == 0
    bad = list(ok); bad[11] = 3 * A + 16   # out overlaps k_i8
    assert lib.sage_validate_attn_fwd(*bad) == -7
    bad = list(ok); bad[11] = None
    assert lib.sage_validate_attn_fwd(*bad) == -1
    bad = list(ok); bad[13] = 0          # N > 1 with zero token stride
    assert lib.sage_validate_attn_fwd(*bad) == -4


def test_workspace_sizes(sage):
    assert sage.sage_quant_qk_workspace_size(1, 100, 2, 96) == 0
    a = sage.sage_quant_qk_workspace_size(2, 4608, 24, 128)
    b = sage.sage_quant_v_workspace_size(2, 4608, 24, 128)
    assert 0 < a < b < 64 << 20
    assert a % 256 == 0 and b % 256 == 0


def test_ex_entry_points_granularity(sage):
    """The _ex calls accept q_block 32 or 1 and k_block 64 or 16, refuse
    anything else before any HIP call, and size the scale ranges by them."""
    lib = sage.lib()
    B, N, H, D = 1, 100, 2, 64
    Np = 128
    big = 1 << 40
    args = [big, 0, H * D, D, 2 * big, 0, H * D, D, B, N, H, D,
            3 * big, 4 * big, 5 * big, 6 * big, 7 * big, 8 * big, 1 << 30]
    for qb in (32, 1):
        for kb in (64, 16):
            assert lib.sage_validate_quant_qk_ex(*args, qb, kb) == 0
    for bad in (0, 2, 16, 64, -1):
        assert lib.sage_validate_quant_qk_ex(*args, bad, 64) == -3
        assert lib.sage_quant_qk_ex(*args, bad, 64, None) == -3
    for bad in (0, 1, 32, 128, -16):
        assert lib.sage_validate_quant_qk_ex(*args, 32, bad) == -3
        assert lib.sage_quant_qk_ex(*args, 32, bad, None) == -3
    # per-token q_scale is 32x longer: a q_scale placed just below k_i8 now overlaps it
    near = list(args)
    near[13] = 5 * big - B * H * Np * 4 // 32
    assert lib.sage_validate_quant_qk_ex(*near, 32, 64) == 0
    assert lib.sage_validate_quant_qk_ex(*near, 1, 64) == -7
    # 16-token k_scale is 4x longer: one placed just below k_mean now overlaps it
    near = list(args)
    near[15] = 7 * big - B * H * Np * 4 // 64
    assert lib.sage_validate_quant_qk_ex(*near, 32, 64) == 0
    assert lib.sage_validate_quant_qk_ex(*near, 32, 16) == -7
    aargs = [big, 2 * big, 3 * big, 4 * big, 5 * big, 6 * big, 7 * big, B, N, H, D,
             8 * big, N * H * D, H * D, D]
    assert lib.sage_validate_attn_fwd_ex(*aargs, 1, 16) == 0
    assert lib.sage_validate_attn_fwd_ex(*aargs, 8, 64) == -3
    assert lib.sage_validate_attn_fwd_ex(*aargs, 32, 32) == -3
    assert lib.sage_attn_fwd_ex(*aargs[:11], 0.0, *aargs[11:], 8, 64, None) == -3


def test_shard_entry_points_validation(sage):
    """sage_quant_q and sage_attn_fwd_shard: documented status codes before any
    HIP call; the Q and K/V ranges are sized by Nq and Nk separately."""
    lib = sage.lib()
    big = 1 << 40
    B, H, D = 1, 2, 64
    Nq, Nk = 100, 1000
    Npq, Npk = 128, 1024
    qargs = [big, 0, H * D, D, B, Nq, H, D, 2 * big, 3 * big]
    assert lib.sage_validate_quant_q(*qargs, 32) == 0
    assert lib.sage_validate_quant_q(*qargs, 1) == 0
    assert lib.sage_validate_quant_q(*qargs, 16) == -3
    assert lib.sage_quant_q(*qargs, 16, None) == -3
    bad = list(qargs); bad[8] = None
    assert lib.sage_validate_quant_q(*bad, 32) == -1
    bad = list(qargs); bad[7] = 96
    assert lib.sage_validate_quant_q(*bad, 32) == -3
    bad = list(qargs); bad[2] = 0                      # Nq > 1 with zero token stride
    assert lib.sage_validate_quant_q(*bad, 32) == -4
    bad = list(qargs); bad[9] = big + 8                # q_scale inside the input rows
    assert lib.sage_validate_quant_q(*bad, 32) == -7

    def aargs(nq=Nq, nk=Nk, out=8 * big, k_i8=3 * big):
        return [big, 2 * big, nq, k_i8, 4 * big, 5 * big, 6 * big, 7 * big, nk, B, H, D,
                out, nq * H * D, H * D, D]
    assert lib.sage_validate_attn_fwd_shard(*aargs(), 32, 64) == 0
    assert lib.sage_validate_attn_fwd_shard(*aargs(), 1, 16) == 0
    assert lib.sage_validate_attn_fwd_shard(*aargs(), 8, 64) == -3
    assert lib.sage_attn_fwd_shard(*aargs()[:12], 0.0, *aargs()[12:], 8, 64, None) == -3
    assert lib.sage_validate_attn_fwd_shard(*aargs(nq=0), 32, 64) == -2
    assert lib.sage_validate_attn_fwd_shard(*aargs(nk=0), 32, 64) == -2
    # an output placed right after the K codes of Nk keys is fine; one inside them is not
    k_bytes = B * H * Npk * D
    assert lib.sage_validate_attn_fwd_shard(*aargs(out=3 * big + k_bytes), 32, 64) == 0
    assert lib.sage_validate_attn_fwd_shard(*aargs(out=3 * big + k_bytes - 16), 32, 64) == -7
    # the output spans Nq rows only: right after it may start K
    o_bytes = (Nq - 1) * H * D * 2 + (H - 1) * D * 2 + D * 2
    assert lib.sage_validate_attn_fwd_shard(*aargs(out=8 * big, k_i8=8 * big + o_bytes), 32, 64) == 0
    # Nq == Nk is the self-attention check of sage_validate_attn_fwd_ex
    same = aargs(nq=Nk, nk=Nk)
    ex = [same[0], same[1], same[3], same[4], same[5], same[6], same[7], B, Nk, H, D, *same[12:]]
    assert lib.sage_validate_attn_fwd_ex(*ex, 32, 64) == lib.sage_validate_attn_fwd_shard(*same, 32, 64) == 0


def test_attn_launch_shape(sage):
    """Shallow grids (FLUX, B2 H24 N4608: 864 eight-wave workgroups, ~3.4 per
    CU) take four-wave workgroups; deep ones (B1 H40 N32760: 20 per CU) eight."""
    w, g = sage.sage_attn_launch_shape(2, 4608, 24, 128)
    assert (w, g) == (4, 2 * 24 * 36)
    w, g = sage.sage_attn_launch_shape(1, 32760, 40, 128)
    assert w == 8 and g == 40 * 128
    w, g = sage.sage_attn_launch_shape(1, 1, 1, 64)
    assert g % 8 == 0 and g >= 1
    with pytest.raises(sage.SageError) as e:
        sage.sage_attn_launch_shape(1, 10, 2, 96)
    assert e.value.status == -3
    assert sage.lib().sage_attn_launch_shape(1, 10, 2, 64, None, None) == -1


def test_benchmark_hooks(sage):
    """The process-wide benchmark hooks take exactly their documented values
    (schedule 0..2; waves 0, 4 or 8) and a forced workgroup size shows in the
    reported launch shape; both are reset afterwards."""
    lib = sage.lib()
    try:
        for v in (0, 1, 2):
            assert lib.sage_attn_schedule(v) == 0
        for v in (-1, 3, 100):
            assert lib.sage_attn_schedule(v) == -9  # SAGE_ERR_VALUE
        for v in (0, 4, 8):
            assert lib.sage_attn_tuning(v) == 0
        for v in (-1, 1, 2, 16):
            assert lib.sage_attn_tuning(v) == -9
        assert lib.sage_attn_tuning(8) == 0
        w, g = sage.sage_attn_launch_shape(2, 4608, 24, 128)
        assert (w, g) == (8, 2 * 24 * 18)
    finally:
        lib.sage_attn_schedule(0)
        lib.sage_attn_tuning(0)
    assert sage.sage_attn_launch_shape(2, 4608, 24, 128)[0] == 4


def test_binding_refuses_without_library(monkeypatch, tmp_path):
    import quantized_attention_video_smooth_amd as s
    monkeypatch.setattr(s, "_lib", None)
    monkeypatch.setattr(s, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        s.lib()


def test_norm_rope_validation(sage):
    """sage_validate_norm_rope / sage_norm_rope: every refusal happens on the
    host, before any HIP call."""
    lib = sage.lib()
    B, N, H, D = 2, 100, 3, 128
    big = 1 << 40
    x, w, rope, y = big, 2 * big, 3 * big, 4 * big
    good = [x, N * H * D, H * D, D, B, N, H, D, w, rope, 1e-6, y, N * H * D, H * D, D]
    assert lib.sage_validate_norm_rope(*good) == 0
    for i, code in ((0, -1), (8, -1), (9, -1), (11, -1)):
        bad = list(good)
        bad[i] = None
        assert lib.sage_validate_norm_rope(*bad) == code
    for eps in (-1e-6, float("nan"), float("inf")):
        bad = list(good)
        bad[10] = eps
        assert lib.sage_validate_norm_rope(*bad) == -9
        assert lib.sage_norm_rope(*bad, None) == -9
    bad = list(good)
    bad[9] = rope + 8                        # the table is read 16 bytes at a time
    assert lib.sage_validate_norm_rope(*bad) == -5
    bad = list(good)
    bad[8] = w + 2
    assert lib.sage_validate_norm_rope(*bad) == -5
    bad = list(good)
    bad[11] = rope + N * D * 4 - 16          # y starts inside the table
    assert lib.sage_validate_norm_rope(*bad) == -7
    bad = list(good)
    bad[11] = x + 64                         # y overlaps x
    assert lib.sage_validate_norm_rope(*bad) == -7
    bad = list(good)
    bad[7] = 96
    assert lib.sage_validate_norm_rope(*bad) == -3
    assert lib.sage_status_string(-9) != lib.sage_status_string(-100)


def test_norm_rope_quant_qk_validation(sage):
    lib = sage.lib()
    B, N, H, D = 1, 100, 2, 64
    big = 1 << 40
    qk = [big, 0, H * D, D, 2 * big, 0, H * D, D, B, N, H, D]
    consts = [9 * big, 10 * big, 11 * big, 1e-6]
    outs = [3 * big, 4 * big, 5 * big, 6 * big, 7 * big, 8 * big, 1 << 30]
    assert lib.sage_validate_norm_rope_quant_qk(*qk, *consts, *outs, 32, 64) == 0
    assert lib.sage_validate_norm_rope_quant_qk(*qk, *consts, *outs, 1, 16) == 0
    assert lib.sage_validate_norm_rope_quant_qk(*qk, *consts, *outs, 2, 64) == -3
    for i in range(3):
        c = list(consts)
        c[i] = None
        assert lib.sage_validate_norm_rope_quant_qk(*qk, *c, *outs, 32, 64) == -1
    c = list(consts)
    c[3] = -1.0
    assert lib.sage_validate_norm_rope_quant_qk(*qk, *c, *outs, 32, 64) == -9
    assert lib.sage_norm_rope_quant_qk(*qk, *c, *outs, 32, 64, None) == -9
    c = list(consts)
    c[2] = 7 * big + 64                      # the table overlaps k_mean's range
    assert lib.sage_validate_norm_rope_quant_qk(*qk, *c, *outs, 32, 64) == -7
    c = list(consts)
    c[0] = 9 * big + 4
    assert lib.sage_validate_norm_rope_quant_qk(*qk, *c, *outs, 32, 64) == -5


def test_norm_rope_quant_qk_workspace(sage):
    """The fused producer's workspace is the quantiser's plus one fp32 per K
    token row (rounded up to 256 bytes); a smaller one is refused."""
    lib = sage.lib()
    for B, N, H, D in ((1, 100, 2, 64), (2, 4608, 24, 128), (1, 32760, 40, 128)):
        Np = sage.sage_padded_tokens(N)
        base = lib.sage_quant_qk_workspace_size(B, N, H, D)
        extra = (B * H * Np * 4 + 255) // 256 * 256
        assert lib.sage_norm_rope_quant_qk_workspace_size(B, N, H, D) == base + extra
    assert lib.sage_norm_rope_quant_qk_workspace_size(1, 100, 2, 96) == 0
    B, N, H, D = 1, 100, 2, 64
    big = 1 << 40
    need = lib.sage_norm_rope_quant_qk_workspace_size(B, N, H, D)
    qk = [big, 0, H * D, D, 2 * big, 0, H * D, D, B, N, H, D]
    consts = [9 * big, 10 * big, 11 * big, 1e-6]
    outs = [3 * big, 4 * big, 5 * big, 6 * big, 7 * big, 8 * big]
    assert lib.sage_validate_norm_rope_quant_qk(*qk, *consts, *outs, need, 32, 64) == 0
    assert lib.sage_validate_norm_rope_quant_qk(*qk, *consts, *outs, need - 1, 32, 64) == -6
    assert lib.sage_validate_quant_qk_ex(*qk, *outs, lib.sage_quant_qk_workspace_size(B, N, H, D),
                                         32, 64) == 0


def test_projection_validation(sage):
    """sage_validate_quant_rows_fp8 / sage_validate_gemm_fp8_rowwise refuse bad
    arguments on the host, with the same codes the entry points return."""
    lib = sage.lib()
    big = 1 << 40
    M, K, N = 300, 3072, 512
    assert lib.sage_validate_quant_rows_fp8(big, K, M, K, 2 * big, 3 * big) == 0
    assert lib.sage_validate_quant_rows_fp8(big, K + 64, M, K, 2 * big, 3 * big) == 0
    assert lib.sage_validate_quant_rows_fp8(None, K, M, K, 2 * big, 3 * big) == -1
    assert lib.sage_validate_quant_rows_fp8(big, K, 0, K, 2 * big, 3 * big) == -2
    assert lib.sage_validate_quant_rows_fp8(big, K, M, 12, 2 * big, 3 * big) == -3
    assert lib.sage_validate_quant_rows_fp8(big, 32768, M, 32768, 2 * big, 3 * big) == -3
    assert lib.sage_validate_quant_rows_fp8(big, K - 8, M, K, 2 * big, 3 * big) == -4
    assert lib.sage_validate_quant_rows_fp8(big, K + 4, M, K, 2 * big, 3 * big) == -5
    assert lib.sage_validate_quant_rows_fp8(big + 8, K, M, K, 2 * big, 3 * big) == -5
    assert lib.sage_validate_quant_rows_fp8(big, K, M, K, big + 64, 3 * big) == -7
    assert lib.sage_quant_rows_fp8(big, K, M, 12, 2 * big, 3 * big, None) == -3
    g = [big, 2 * big, M, 3 * big, 4 * big, N, K, 5 * big, 6 * big, N]
    assert lib.sage_validate_gemm_fp8_rowwise(*g) == 0
    bad = list(g); bad[7] = None
    assert lib.sage_validate_gemm_fp8_rowwise(*bad) == 0          # no bias
    bad = list(g); bad[3] = None
    assert lib.sage_validate_gemm_fp8_rowwise(*bad) == -1
    bad = list(g); bad[6] = 3000
    assert lib.sage_validate_gemm_fp8_rowwise(*bad) == -3         # K % 128
    bad = list(g); bad[5] = 510; bad[9] = 512
    assert lib.sage_validate_gemm_fp8_rowwise(*bad) == -3         # N % 4
    bad = list(g); bad[9] = N - 4
    assert lib.sage_validate_gemm_fp8_rowwise(*bad) == -4         # ldo < N
    bad = list(g); bad[9] = N + 2
    assert lib.sage_validate_gemm_fp8_rowwise(*bad) == -5
    bad = list(g); bad[4] = 4 * big + 4                           # w_scale read as float4
    assert lib.sage_validate_gemm_fp8_rowwise(*bad) == -5
    bad = list(g); bad[8] = 3 * big + 1024                        # out inside w8
    assert lib.sage_validate_gemm_fp8_rowwise(*bad) == -7
    assert lib.sage_gemm_fp8_rowwise(*bad, None) == -7
    bad = list(g); bad[2] = (1 << 24) + 1
    assert lib.sage_validate_gemm_fp8_rowwise(*bad) == -2
