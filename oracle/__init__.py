"""CPU oracle for smoothed, quantised attention -- TEST INFRASTRUCTURE ONLY.

Only tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg
may import this package.  It wraps ``sage_oracle.c`` (plain C, fp64) through
ctypes and shares no code with the HIP path.

Every function follows one step of the method; see the header of
``sage_oracle.c`` for the passages and readings.  Pins live in
``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sage_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

BQ, BK = 32, 64


def build() -> str:
    """Compile the oracle (gcc, OpenMP, no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-std=c11", "-Wall", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int
_dbl = ctypes.c_double
_f32 = ctypes.c_float


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    sig = {
        "orc_bf16_value": ([ctypes.c_uint16], ctypes.c_float),
        "orc_bf16_round": ([ctypes.c_float], ctypes.c_uint16),
        "orc_e4m3_decode": ([ctypes.c_uint8], _dbl),
        "orc_e4m3_encode": ([_dbl], ctypes.c_uint8),
        "orc_i8_code": ([ctypes.c_float], _i32),
        "orc_v_slot": ([_i32], _i32),
        "orc_bf16_round_n": ([_vp, _vp, _i64], None),
        "orc_e4m3_encode_n": ([_vp, _vp, _i64], None),
        "orc_e4m3_decode_n": ([_vp, _vp, _i64], None),
        "orc_k_mean": ([_vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _vp], _i32),
        "orc_k_center": ([_vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _vp, _vp], None),
        "orc_quant_i8_blocks": ([_vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _i32, _vp, _vp], None),
        "orc_quant_qk": ([_vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32,
                          _i32, _i32, _vp, _vp, _vp, _vp, _vp], _i32),
        "orc_quant_v": ([_vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _vp], _i32),
        "orc_online_softmax_pv": ([_vp, _vp, _i32, _i32, _i32, _i32, _vp], None),
        "orc_attn_tiled": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _dbl, _i32,
                            _i32, _i32, _vp, _i32, _vp], None),
        "orc_attn_exact": ([_vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64,
                            _i32, _i32, _i32, _i32, _dbl, _vp, _i32, _vp], None),
        "orc_norm_rope": ([_vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _vp, _f32, _vp, _vp], _i32),
        "orc_quant_rows_e4m3": ([_vp, _i64, _i32, _i32, _vp, _vp], None),
        "orc_gemm_fp8_rowwise": ([_vp, _vp, _i32, _vp, _vp, _i32, _i32, _vp, _vp, _i32, _vp, _i32,
                                  _vp, _vp, _vp], None),
        "orc_fsum": ([_vp, _i64], _dbl),
        "orc_num_threads": ([], _i32),
        "orc_set_num_threads": ([_i32], None),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _bf16_view(t):
    """A bf16 torch CPU tensor [B, N, H, D] (any strides, d-stride 1) -> (uint16 base
    array keeping the storage alive, element strides (sb, sn, sh))."""
    import torch
    assert t.dtype == torch.bfloat16 and t.device.type == "cpu" and t.dim() == 4
    assert t.stride(3) == 1
    base = t.view(torch.int16).numpy()  # shares memory, keeps strides
    return base, t.stride(0), t.stride(1), t.stride(2)


def num_threads() -> int:
    return _load().orc_num_threads()


def set_num_threads(n: int) -> None:
    """Thread count of the oracle's OpenMP loops (for timing; results do not
    depend on it)."""
    _load().orc_set_num_threads(int(n))


# ---- codecs --------------------------------------------------------------

def bf16_round(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, dtype=np.uint16)
    _load().orc_bf16_round_n(_p(x), _p(y), x.size)
    return y


def fsum(x: np.ndarray) -> float:
    """Correctly rounded fp64 sum of the exact sum of x (the channel sums of
    reading R3 when plain fp64 accumulation is not provably exact)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    return float(_load().orc_fsum(_p(x), x.size))


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(x.shape, dtype=np.uint8)
    _load().orc_e4m3_encode_n(_p(x), _p(y), x.size)
    return y


def e4m3_decode(c: np.ndarray) -> np.ndarray:
    c = np.ascontiguousarray(c, dtype=np.uint8)
    y = np.empty(c.shape, dtype=np.float64)
    _load().orc_e4m3_decode_n(_p(c), _p(y), c.size)
    return y


def i8_code(x: float) -> int:
    return _load().orc_i8_code(x)


def v_slot(t: int) -> int:
    return _load().orc_v_slot(t)


# ---- quantisation ----------------------------------------------------------

def quant_qk(q, k, q_block: int = BQ, k_block: int = BK):
    """Fused steps 1-4.  Returns dict of numpy arrays:
    q_i8 / k_i8 [B,H,N,D] int8, q_scale [B,H,ceil(N/q_block)], k_scale [B,H,ceil(N/k_block)]
    fp32, k_mean [B,H,D] uint16 (bf16 bits), inexact (int: channels whose plain fp64 sum is not
    provably exact; their mean comes from the rounded exact sum),
    q_block, k_block.  q_block = 32 (the path's block granularity) or 1 (one scale per
    token); k_block = 64 (the key tile) or 16."""
    if q_block not in (1, BQ):
        raise ValueError("q_block must be 32 or 1")
    if k_block not in (16, BK):
        raise ValueError("k_block must be 64 or 16")
    B, N, H, D = q.shape
    qb, qsb, qsn, qsh = _bf16_view(q)
    kb, ksb, ksn, ksh = _bf16_view(k)
    out = dict(
        q_i8=np.empty((B, H, N, D), np.int8),
        q_scale=np.empty((B, H, math.ceil(N / q_block)), np.float32),
        k_i8=np.empty((B, H, N, D), np.int8),
        k_scale=np.empty((B, H, math.ceil(N / k_block)), np.float32),
        k_mean=np.empty((B, H, D), np.uint16),
    )
    bad = _load().orc_quant_qk(_p(qb), qsb, qsn, qsh, _p(kb), ksb, ksn, ksh, B, N, H, D, q_block,
                               k_block, _p(out["q_i8"]), _p(out["q_scale"]), _p(out["k_i8"]),
                               _p(out["k_scale"]), _p(out["k_mean"]))
    out["inexact"] = int(bad)
    out["q_block"] = q_block
    out["k_block"] = k_block
    return out


def norm_rope(x, weight, rope, eps: float = 1e-6):
    """QK RMSNorm + RoPE producer (orc_norm_rope).  x bf16 torch CPU [B,N,H,D]
    (any strides, d-stride 1), weight bf16 [D], rope fp32 [N, D/2, 2] (cos, sin).
    Returns (y bf16 torch tensor [B,N,H,D] contiguous, number of rows whose
    sum of squares is not provably exact)."""
    import torch
    B, N, H, D = x.shape
    xb, sb, sn, sh = _bf16_view(x)
    w = np.ascontiguousarray(weight.contiguous().view(torch.int16).numpy())
    assert w.shape == (D,)
    rope = np.ascontiguousarray(rope, dtype=np.float32)
    assert rope.shape == (N, D // 2, 2)
    y = torch.empty((B, N, H, D), dtype=torch.bfloat16)
    yb = y.view(torch.int16).numpy()
    bad = _load().orc_norm_rope(_p(xb), sb, sn, sh, B, N, H, D, _p(w), float(eps), _p(rope), _p(yb))
    return y, int(bad)


def quant_rows_e4m3(x):
    """Row-wise FP8 quantisation (orc_quant_rows_e4m3) of a bf16 torch CPU tensor
    [M, K] (any row stride, unit column stride).  Returns (codes uint8 [M, K],
    scales fp32 [M])."""
    import torch
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    M, K = x.shape
    base = x.view(torch.int16).numpy()
    codes = np.empty((M, K), np.uint8)
    scales = np.empty(M, np.float32)
    _load().orc_quant_rows_e4m3(_p(base), x.stride(0), M, K, _p(codes), _p(scales))
    return codes, scales


def gemm_fp8_rowwise(a, sa, b, sb, bias=None, rows=None, cols=None):
    """Scaled FP8 GEMM (orc_gemm_fp8_rowwise) on codes a [M, K], b [N, K] with
    row scales sa [M], sb [N] and optional bf16 torch bias [N].  Returns fp64
    (out, absum, blk) [len(rows), len(cols)]: the result and the two error
    magnitudes described in orc_gemm_fp8_rowwise."""
    import torch
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    M, K = a.shape
    N = b.shape[0]
    assert b.shape[1] == K
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    sb = np.ascontiguousarray(sb, dtype=np.float32)
    rows = np.ascontiguousarray(np.arange(M) if rows is None else rows, dtype=np.int32)
    cols = np.ascontiguousarray(np.arange(N) if cols is None else cols, dtype=np.int32)
    bb = None
    if bias is not None:
        bb = np.ascontiguousarray(bias.contiguous().view(torch.int16).numpy())
        assert bb.shape == (N,)
    out = np.empty((rows.size, cols.size), np.float64)
    absum = np.empty_like(out)
    blk = np.empty_like(out)
    _load().orc_gemm_fp8_rowwise(_p(a), _p(sa), M, _p(b), _p(sb), N, K, _p(bb) if bb is not None else None,
                                 _p(rows), rows.size, _p(cols), cols.size, _p(out), _p(absum), _p(blk))
    return out, absum, blk


def k_mean(k):
    B, N, H, D = k.shape
    kb, sb, sn, sh = _bf16_view(k)
    m = np.empty((B, H, D), np.uint16)
    bad = _load().orc_k_mean(_p(kb), sb, sn, sh, B, N, H, D, _p(m))
    return m, int(bad)


def k_center(k, mean: np.ndarray) -> np.ndarray:
    """bf16 bits of bf16(K - mean), contiguous [B,N,H,D]."""
    B, N, H, D = k.shape
    kb, sb, sn, sh = _bf16_view(k)
    mean = np.ascontiguousarray(mean, dtype=np.uint16)
    kc = np.empty((B, N, H, D), np.uint16)
    _load().orc_k_center(_p(kb), sb, sn, sh, B, N, H, D, _p(mean), _p(kc))
    return kc


def quant_i8_blocks(x_bits: np.ndarray, blk: int):
    """Per-block INT8 of a contiguous bf16-bits array [B,N,H,D]."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    B, N, H, D = x_bits.shape
    codes = np.empty((B, H, N, D), np.int8)
    scales = np.empty((B, H, math.ceil(N / blk)), np.float32)
    _load().orc_quant_i8_blocks(_p(x_bits), N * H * D, H * D, D, B, N, H, D, blk,
                                _p(codes), _p(scales))
    return codes, scales


def quant_v(v):
    """Steps 5-6.  Returns dict: v_fp8 [B,H,D,Np] uint8 (slot-permuted, zero pad),
    v_scale / v_mean [B,H,D] fp32, inexact (int: channels whose plain fp64 sum is
    not provably exact; their mean comes from the rounded exact sum), bad (int:
    channels where the min/max absmax identity failed, an oracle self-check)."""
    B, N, H, D = v.shape
    vb, sb, sn, sh = _bf16_view(v)
    Np = math.ceil(N / 64) * 64
    out = dict(
        v_fp8=np.empty((B, H, D, Np), np.uint8),
        v_scale=np.empty((B, H, D), np.float32),
        v_mean=np.empty((B, H, D), np.float32),
    )
    bad = _load().orc_quant_v(_p(vb), sb, sn, sh, B, N, H, D, _p(out["v_fp8"]),
                              _p(out["v_scale"]), _p(out["v_mean"]))
    out["inexact"] = int(bad) & 0xFFFFF
    out["bad"] = int(bad) >> 20
    return out


# ---- attention -------------------------------------------------------------

def online_softmax_pv(s: np.ndarray, vals: np.ndarray, bc: int, quant_p: bool) -> np.ndarray:
    s = np.ascontiguousarray(s, dtype=np.float64)
    vals = np.ascontiguousarray(vals, dtype=np.float64)
    n, dv = vals.shape
    assert s.shape == (n,)
    out = np.empty(dv, np.float64)
    _load().orc_online_softmax_pv(_p(s), _p(vals), n, dv, bc, int(bool(quant_p)), _p(out))
    return out


def _rows(N, rows):
    if rows is None:
        rows = np.arange(N, dtype=np.int32)
    return np.ascontiguousarray(rows, dtype=np.int32)


def attn_tiled(qk: dict, v: dict, sm_scale: float | None = None, rows=None, bc: int = BK):
    """Step 7 (quantised path, fp64).  Returns fp64 [B,H,len(rows),D]."""
    B, H, N, D = qk["q_i8"].shape
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    rows = _rows(N, rows)
    out = np.empty((B, H, rows.size, D), np.float64)
    arrs = [np.ascontiguousarray(qk["q_i8"]), np.ascontiguousarray(qk["q_scale"]),
            np.ascontiguousarray(qk["k_i8"]), np.ascontiguousarray(qk["k_scale"]),
            np.ascontiguousarray(v["v_fp8"]), np.ascontiguousarray(v["v_scale"]),
            np.ascontiguousarray(v["v_mean"])]
    _load().orc_attn_tiled(*[_p(a) for a in arrs], B, N, H, D, float(sm_scale), bc,
                           int(qk.get("q_block", BQ)), int(qk.get("k_block", BK)), _p(rows),
                           rows.size, _p(out))
    return out


def attn_exact(q, k, v, sm_scale: float | None = None, rows=None):
    """Step 8: exact fp64 softmax attention on the original bf16 inputs.
    Returns fp64 [B,H,len(rows),D]."""
    B, N, H, D = q.shape
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    rows = _rows(N, rows)
    qb, qsb, qsn, qsh = _bf16_view(q)
    kb, ksb, ksn, ksh = _bf16_view(k)
    vb, vsb, vsn, vsh = _bf16_view(v)
    out = np.empty((B, H, rows.size, D), np.float64)
    _load().orc_attn_exact(_p(qb), qsb, qsn, qsh, _p(kb), ksb, ksn, ksh, _p(vb), vsb, vsn, vsh,
                           B, N, H, D, float(sm_scale), _p(rows), rows.size, _p(out))
    return out


def rel_l2(x: np.ndarray, ref: np.ndarray) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm((x - ref).ravel()) / np.linalg.norm(ref.ravel()))
