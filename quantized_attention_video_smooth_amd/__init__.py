"""Python binding of libsage.so (smoothed, quantised attention on MI355X).

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI declared in include/sage.h.  torch provides device memory and
the current stream.  There is no fallback: if libsage.so is missing, importing
the raw functions raises.

Raw entry points keep the C names (sage_quant_qk, sage_quant_v,
sage_attn_fwd, ...) and take integers (pointers, strides, sizes).  The
tensor-level helpers quant_qk / quant_v / attn_fwd allocate outputs with
torch.empty on the input's device and call the raw entry points on
torch.cuda.current_stream().
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsage.so")

SAGE_OK = 0
BQ, BK, NPAD = 32, 64, 64


class SageError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None
_lock = threading.Lock()
_vp, _i64, _i32, _sz, _f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_float

_SIGS = {
    "sage_get_layout": ([_vp], _i32),
    "sage_padded_tokens": ([_i64], _i64),
    "sage_v_slot": ([_i32], _i32),
    "sage_quant_qk_workspace_size": ([_i32] * 4, _sz),
    "sage_quant_v_workspace_size": ([_i32] * 4, _sz),
    "sage_norm_rope_quant_qk_workspace_size": ([_i32] * 4, _sz),
    "sage_workspace_zero_bytes": ([], _sz),
    "sage_quant_qk_static": ([_vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32,
                              _vp, _vp, _vp, _vp, _vp, _vp], _i32),
    "sage_quant_qk": ([_vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32,
                       _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _i32),
    "sage_quant_v": ([_vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp], _i32),
    "sage_attn_fwd": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32,
                       _vp, _i64, _i64, _i64, _vp], _i32),
    "sage_validate_quant_qk": ([_vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32,
                                _vp, _vp, _vp, _vp, _vp, _vp, _sz], _i32),
    "sage_validate_quant_v": ([_vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz], _i32),
    "sage_validate_attn_fwd": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                _vp, _i64, _i64, _i64], _i32),
    "sage_attn_launch_shape": ([_i32, _i32, _i32, _i32, _vp, _vp], _i32),
    "sage_attn_tuning": ([_i32], _i32),
    "sage_attn_schedule": ([_i32], _i32),
    "sage_quant_qk_ex": ([_vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32,
                          _vp, _vp, _vp, _vp, _vp, _vp, _sz, _i32, _i32, _vp], _i32),
    "sage_attn_fwd_ex": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32,
                          _vp, _i64, _i64, _i64, _i32, _i32, _vp], _i32),
    "sage_validate_quant_qk_ex": ([_vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _i32, _i32, _i32,
                                   _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _i32, _i32], _i32),
    "sage_norm_rope": ([_vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _f32,
                        _vp, _i64, _i64, _i64, _vp], _i32),
    "sage_validate_norm_rope": ([_vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _f32,
                                 _vp, _i64, _i64, _i64], _i32),
    "sage_norm_rope_quant_qk": ([_vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _i32, _i32, _i32,
                                 _i32, _vp, _vp, _vp, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                 _i32, _i32, _vp], _i32),
    "sage_validate_norm_rope_quant_qk": ([_vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _i32,
                                          _i32, _i32, _i32, _vp, _vp, _vp, _f32, _vp, _vp, _vp,
                                          _vp, _vp, _vp, _sz, _i32, _i32], _i32),
    "sage_quant_rows_fp8": ([_vp, _i64, _i32, _i32, _vp, _vp, _vp], _i32),
    "sage_validate_quant_rows_fp8": ([_vp, _i64, _i32, _i32, _vp, _vp], _i32),
    "sage_gemm_fp8_rowwise": ([_vp, _vp, _i32, _vp, _vp, _i32, _i32, _vp, _vp, _i64, _vp], _i32),
    "sage_validate_gemm_fp8_rowwise": ([_vp, _vp, _i32, _vp, _vp, _i32, _i32, _vp, _vp, _i64], _i32),
    "sage_validate_attn_fwd_ex": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                   _vp, _i64, _i64, _i64, _i32, _i32], _i32),
    "sage_quant_q": ([_vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _i32, _vp], _i32),
    "sage_validate_quant_q": ([_vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _i32], _i32),
    "sage_attn_fwd_shard": ([_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32,
                             _vp, _i64, _i64, _i64, _i32, _i32, _vp], _i32),
    "sage_validate_attn_fwd_shard": ([_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                      _i32, _vp, _i64, _i64, _i64, _i32, _i32], _i32),
    "sage_status_string": ([_i32], ctypes.c_char_p),
}


def lib() -> ctypes.CDLL:
    """The loaded libsage.so (raises ImportError if it has not been built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise ImportError(
                        f"{LIB_PATH} is missing; build it with "
                        "`python -m quantized_attention_video_smooth_amd.build`")
                handle = ctypes.CDLL(LIB_PATH)
                for name, (args, res) in _SIGS.items():
                    f = getattr(handle, name)
                    f.argtypes = args
                    f.restype = res
                _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().sage_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != SAGE_OK:
        raise SageError(status, where)


# ---- raw C entry points (same names, integer arguments) ---------------------

def sage_quant_qk(*args) -> int:
    return lib().sage_quant_qk(*args)


def sage_quant_v(*args) -> int:
    return lib().sage_quant_v(*args)


def sage_attn_fwd(*args) -> int:
    return lib().sage_attn_fwd(*args)


def sage_quant_qk_ex(*args) -> int:
    return lib().sage_quant_qk_ex(*args)


def sage_attn_fwd_ex(*args) -> int:
    return lib().sage_attn_fwd_ex(*args)


def sage_quant_rows_fp8(*args) -> int:
    return lib().sage_quant_rows_fp8(*args)


def sage_quant_q(*args) -> int:
    return lib().sage_quant_q(*args)


def sage_attn_fwd_shard(*args) -> int:
    return lib().sage_attn_fwd_shard(*args)


def sage_gemm_fp8_rowwise(*args) -> int:
    return lib().sage_gemm_fp8_rowwise(*args)


def sage_norm_rope(*args) -> int:
    return lib().sage_norm_rope(*args)


def sage_norm_rope_quant_qk(*args) -> int:
    return lib().sage_norm_rope_quant_qk(*args)


def sage_attn_launch_shape(B: int, N: int, H: int, D: int) -> tuple:
    """(waves per workgroup, workgroups) of the attention launch for these sizes."""
    w, g = ctypes.c_int(0), ctypes.c_int(0)
    _check(lib().sage_attn_launch_shape(B, N, H, D, ctypes.byref(w), ctypes.byref(g)),
           "sage_attn_launch_shape")
    return w.value, g.value


def sage_attn_tuning(waves: int = 0) -> None:
    """Benchmark hook: forced attention workgroup size (0 automatic, 4 or 8
    waves), process-wide."""
    _check(lib().sage_attn_tuning(waves), "sage_attn_tuning")


def sage_attn_schedule(schedule: int = 0) -> None:
    """Benchmark hook: forced attention key-step schedule (0 default, i.e. 2;
    1 the compiler's order; 2 MFMAs spread through the softmax), process-wide."""
    _check(lib().sage_attn_schedule(schedule), "sage_attn_schedule")


def sage_padded_tokens(n: int) -> int:
    return lib().sage_padded_tokens(n)


def sage_v_slot(t: int) -> int:
    return lib().sage_v_slot(t)


def sage_quant_qk_workspace_size(B: int, N: int, H: int, D: int) -> int:
    return lib().sage_quant_qk_workspace_size(B, N, H, D)


def sage_quant_v_workspace_size(B: int, N: int, H: int, D: int) -> int:
    return lib().sage_quant_v_workspace_size(B, N, H, D)


def sage_norm_rope_quant_qk_workspace_size(B: int, N: int, H: int, D: int) -> int:
    return lib().sage_norm_rope_quant_qk_workspace_size(B, N, H, D)


# ---- tensor-level helpers ---------------------------------------------------

_workspaces: dict = {}


def workspace(device, nbytes: int):
    """A device scratch buffer of at least nbytes, cached per device; calls
    sharing it must be ordered (one stream).  Allocated zero-filled: the
    quantisers' workspaces begin with arrival counters that must be zero
    before the first call (each call leaves them zero)."""
    import torch
    key = str(device)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def _stream_ptr(stream) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _nhd(t, name):
    import torch
    if t.dtype != torch.bfloat16 or t.dim() != 4 or t.stride(3) != 1 or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA bf16 [B,N,H,D] tensor with unit stride over D")
    return t.stride(0), t.stride(1), t.stride(2)


def _producer_consts(w_list, rope, N, D):
    import torch
    for w in w_list:
        if w.dtype != torch.bfloat16 or tuple(w.shape) != (D,) or not w.is_cuda or not w.is_contiguous():
            raise ValueError("norm weights must be contiguous CUDA bf16 [D] tensors")
    if (rope.dtype != torch.float32 or tuple(rope.shape) != (N, D // 2, 2) or not rope.is_cuda
            or not rope.is_contiguous()):
        raise ValueError("rope must be a contiguous CUDA fp32 [N, D/2, 2] tensor of (cos, sin)")


def norm_rope(x, weight, rope, eps: float = 1e-6, out=None, stream=None):
    """QK RMSNorm + RoPE producer: x bf16 [B,N,H,D] -> bf16 [B,N,H,D] (or fills `out`).
    weight bf16 [D]; rope fp32 [N, D/2, 2] (cos, sin)."""
    import torch
    B, N, H, D = x.shape
    xs = _nhd(x, "x")
    _producer_consts([weight], rope, N, D)
    if out is None:
        out = torch.empty((B, N, H, D), dtype=torch.bfloat16, device=x.device)
    ys = _nhd(out, "out")
    _check(sage_norm_rope(x.data_ptr(), *xs, B, N, H, D, weight.data_ptr(), rope.data_ptr(),
                          float(eps), out.data_ptr(), *ys, _stream_ptr(stream)), "sage_norm_rope")
    return out


def norm_rope_quant_qk(q, k, wq, wk, rope, eps: float = 1e-6, stream=None, q_block: int = 32,
                       k_block: int = 64):
    """The producer fused into the quantiser: pre-norm q, k bf16 [B,N,H,D] -> the outputs of
    quant_qk(norm_rope(q, wq, rope), norm_rope(k, wk, rope)), without storing the bf16 tensors."""
    import torch
    B, N, H, D = q.shape
    if tuple(k.shape) != (B, N, H, D):
        raise ValueError("q and k must have the same shape")
    if q_block not in (1, BQ) or k_block not in (16, 64):
        raise ValueError("q_block must be 32 or 1 and k_block 64 or 16")
    qs, ks = _nhd(q, "q"), _nhd(k, "k")
    _producer_consts([wq, wk], rope, N, D)
    Np = sage_padded_tokens(N)
    dev = q.device
    q_i8 = torch.empty((B, H, Np, D), dtype=torch.int8, device=dev)
    q_scale = torch.empty((B, H, Np // q_block), dtype=torch.float32, device=dev)
    k_i8 = torch.empty((B, H, Np, D), dtype=torch.int8, device=dev)
    k_scale = torch.empty((B, H, Np // k_block), dtype=torch.float32, device=dev)
    k_mean = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
    need = sage_norm_rope_quant_qk_workspace_size(B, N, H, D)
    ws = workspace(dev, need)
    _check(sage_norm_rope_quant_qk(q.data_ptr(), *qs, k.data_ptr(), *ks, B, N, H, D,
                                   wq.data_ptr(), wk.data_ptr(), rope.data_ptr(), float(eps),
                                   q_i8.data_ptr(), q_scale.data_ptr(), k_i8.data_ptr(),
                                   k_scale.data_ptr(), k_mean.data_ptr(), ws.data_ptr(), ws.numel(),
                                   q_block, k_block, _stream_ptr(stream)),
           "sage_norm_rope_quant_qk")
    return q_i8, q_scale, k_i8, k_scale, k_mean


def quant_rows_fp8(x, stream=None):
    """Row-wise E4M3 quantisation: x bf16 [M, K] (row stride any multiple of 8, unit
    column stride) -> (codes uint8 [M, K], scales fp32 [M])."""
    import torch
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1 or not x.is_cuda:
        raise ValueError("x must be a CUDA bf16 [M, K] tensor with unit column stride")
    M, K = x.shape
    codes = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    scales = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check(sage_quant_rows_fp8(x.data_ptr(), x.stride(0), M, K, codes.data_ptr(), scales.data_ptr(),
                               _stream_ptr(stream)), "sage_quant_rows_fp8")
    return codes, scales


def gemm_fp8_rowwise(x8, x_scale, w8, w_scale, bias=None, out=None, stream=None):
    """Scaled FP8 GEMM: codes x8 [M, K], w8 [N, K] with row scales -> bf16 [M, N]
    (or fills `out`, which may be a column slice of a wider [M, *] buffer)."""
    import torch
    M, K = x8.shape
    N = w8.shape[0]
    for t, name in ((x8, "x8"), (w8, "w8")):
        if t.dtype != torch.uint8 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous CUDA uint8 tensor")
    if w8.shape[1] != K:
        raise ValueError("x8 and w8 must have the same K")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x8.device)
    if out.dtype != torch.bfloat16 or out.dim() != 2 or out.stride(1) != 1 or tuple(out.shape) != (M, N):
        raise ValueError("out must be a bf16 [M, N] view with unit column stride")
    _check(sage_gemm_fp8_rowwise(x8.data_ptr(), x_scale.data_ptr(), M, w8.data_ptr(), w_scale.data_ptr(),
                                 N, K, bias.data_ptr() if bias is not None else None, out.data_ptr(),
                                 out.stride(0), _stream_ptr(stream)), "sage_gemm_fp8_rowwise")
    return out


def quant_qk(q, k, stream=None, q_block: int = 32, k_block: int = 64):
    """K smoothing + INT8 K and INT8 Q.  Returns (q_i8 [B,H,Np,D], q_scale [B,H,Np/q_block],
    k_i8 [B,H,Np,D], k_scale [B,H,Np/k_block], k_mean [B,H,D] bf16).  q_block: 32 (one Q
    scale per 32-token block) or 1 (one per token); k_block: 64 or 16 tokens per K scale."""
    import torch
    B, N, H, D = q.shape
    if tuple(k.shape) != (B, N, H, D):
        raise ValueError("q and k must have the same shape")
    qs, ks = _nhd(q, "q"), _nhd(k, "k")
    Np = sage_padded_tokens(N)
    dev = q.device
    q_i8 = torch.empty((B, H, Np, D), dtype=torch.int8, device=dev)
    if q_block not in (1, BQ):
        raise ValueError("q_block must be 32 or 1")
    if k_block not in (16, 64):
        raise ValueError("k_block must be 64 or 16")
    q_scale = torch.empty((B, H, Np // q_block), dtype=torch.float32, device=dev)
    k_i8 = torch.empty((B, H, Np, D), dtype=torch.int8, device=dev)
    k_scale = torch.empty((B, H, Np // k_block), dtype=torch.float32, device=dev)
    k_mean = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
    need = sage_quant_qk_workspace_size(B, N, H, D)
    ws = workspace(dev, need)
    _check(sage_quant_qk_ex(q.data_ptr(), *qs, k.data_ptr(), *ks, B, N, H, D,
                            q_i8.data_ptr(), q_scale.data_ptr(), k_i8.data_ptr(), k_scale.data_ptr(),
                            k_mean.data_ptr(), ws.data_ptr(), ws.numel(), q_block, k_block,
                            _stream_ptr(stream)),
           "sage_quant_qk_ex")
    return q_i8, q_scale, k_i8, k_scale, k_mean


def quant_q(q, stream=None, q_block: int = 32):
    """INT8 Q alone (the Q half of quant_qk; e.g. one rank's token shard of Q).
    Returns (q_i8 [B,H,Np,D], q_scale [B,H,Np/q_block])."""
    import torch
    B, N, H, D = q.shape
    qs = _nhd(q, "q")
    if q_block not in (1, BQ):
        raise ValueError("q_block must be 32 or 1")
    Np = sage_padded_tokens(N)
    q_i8 = torch.empty((B, H, Np, D), dtype=torch.int8, device=q.device)
    q_scale = torch.empty((B, H, Np // q_block), dtype=torch.float32, device=q.device)
    _check(sage_quant_q(q.data_ptr(), *qs, B, N, H, D, q_i8.data_ptr(), q_scale.data_ptr(), q_block,
                        _stream_ptr(stream)),
           "sage_quant_q")
    return q_i8, q_scale


def quant_v(v, stream=None):
    """V smoothing + FP8 E4M3 V, transposed and slot-permuted.  Returns
    (v_fp8 [B,H,D,Np] uint8, v_scale [B,H,D], v_mean [B,H,D])."""
    import torch
    B, N, H, D = v.shape
    vs = _nhd(v, "v")
    Np = sage_padded_tokens(N)
    dev = v.device
    v_fp8 = torch.empty((B, H, D, Np), dtype=torch.uint8, device=dev)
    v_scale = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    v_mean = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    need = sage_quant_v_workspace_size(B, N, H, D)
    ws = workspace_v(dev, need)
    _check(sage_quant_v(v.data_ptr(), *vs, B, N, H, D, v_fp8.data_ptr(), v_scale.data_ptr(),
                        v_mean.data_ptr(), ws.data_ptr(), ws.numel(), _stream_ptr(stream)),
           "sage_quant_v")
    return v_fp8, v_scale, v_mean


_workspaces_v: dict = {}


def workspace_v(device, nbytes: int):
    """Separate cached workspace for sage_quant_v (zero-filled, as above)."""
    import torch
    key = str(device)
    ws = _workspaces_v.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces_v[key] = ws
    return ws


def attn_fwd(q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale, v_mean, N: int, sm_scale: float | None = None,
             out=None, stream=None):
    """Fused attention on the quantised operands; returns bf16 [B,N,H,D] (or fills `out`).
    The scale granularities follow the scale lengths: q_scale Np/32 or Np per head,
    k_scale Np/64 or Np/16."""
    import torch
    B, H, Np, D = q_i8.shape
    q_block = Np // q_scale.shape[-1]
    k_block = Np // k_scale.shape[-1]
    if out is None:
        out = torch.empty((B, N, H, D), dtype=torch.bfloat16, device=q_i8.device)
    os_ = _nhd(out, "out")
    _check(sage_attn_fwd_ex(q_i8.data_ptr(), q_scale.data_ptr(), k_i8.data_ptr(), k_scale.data_ptr(),
                            v_fp8.data_ptr(), v_scale.data_ptr(), v_mean.data_ptr(), B, N, H, D,
                            float(sm_scale) if sm_scale else 0.0, out.data_ptr(), *os_, q_block, k_block,
                            _stream_ptr(stream)),
           "sage_attn_fwd_ex")
    return out


def attn_fwd_shard(q_i8, q_scale, Nq: int, k_i8, k_scale, v_fp8, v_scale, v_mean, Nk: int,
                   sm_scale: float | None = None, out=None, stream=None):
    """Nq queries (quantised Q shard, e.g. from quant_q) against the Nk keys of the
    whole sequence (quantised K and V); returns bf16 [B,Nq,H,D] (or fills `out`).
    Scale granularities follow the scale lengths as in attn_fwd."""
    import torch
    B, H, Npq, D = q_i8.shape
    Npk = k_i8.shape[2]
    q_block = Npq // q_scale.shape[-1]
    k_block = Npk // k_scale.shape[-1]
    if out is None:
        out = torch.empty((B, Nq, H, D), dtype=torch.bfloat16, device=q_i8.device)
    os_ = _nhd(out, "out")
    _check(sage_attn_fwd_shard(q_i8.data_ptr(), q_scale.data_ptr(), Nq, k_i8.data_ptr(),
                               k_scale.data_ptr(), v_fp8.data_ptr(), v_scale.data_ptr(),
                               v_mean.data_ptr(), Nk, B, H, D, float(sm_scale) if sm_scale else 0.0,
                               out.data_ptr(), *os_, q_block, k_block, _stream_ptr(stream)),
           "sage_attn_fwd_shard")
    return out


def sage_attention(q, k, v, sm_scale: float | None = None, stream=None):
    """The whole path: quant_qk, quant_v, attn_fwd.  q, k, v bf16 [B,N,H,D]."""
    qk = quant_qk(q, k, stream)
    vq = quant_v(v, stream)
    return attn_fwd(qk[0], qk[1], qk[2], qk[3], *vq, N=q.shape[1], sm_scale=sm_scale, stream=stream)
