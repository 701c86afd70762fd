"""Seeded synthetic inputs shaped like the DiT attention workloads.

The generator draws standard normals from a counter-based stream (synth.c) and
maps them to per-tensor value distributions.  It holds none of the attention
method's arithmetic; the fp32 -> bf16 step is torch's own round-to-nearest-even
cast.  Both the HIP path and the CPU oracle consume these tensors.

Workloads (shapes from the FLUX.3 Action RTX 5090 report, §02 stage 03, and the
MiniMax H3 on DGX Spark page, "fixed workload"; distributions are the stated
synthetic recipe, N(mean, variance)):

  0 tiny         B1 H2  N256   D64   Q,K,V~N(0,1); K += off~N(0,4)
  1 flux_joint   B2 H24 N4608  D128  Q,K~N(0,1), 31 (h,d) outlier channels x8;
                                     K += off~N(0,3); V += off~N(0,1)
  2 video_early  B2 H24 N3128  D128  as flux_joint
  3 long_t2v     B1 H40 N32760 D128  Q,K~N(0,1); K += off~N(0,4); V += off~N(0,0.5)
  4 quant_long   B1 H40 N32760 D128  Q,K,V~N(0,1) + off~N(0,4) on each

Per-channel offsets and outlier multipliers are indexed by (h, d) and shared by
every batch entry and token.

Inputs of the QK RMSNorm + RoPE producer ("FLUX 3 Action" SGLang page, §1 and
the latency notes: a fused QK RMSNorm + RoPE over a 4-axis (t, h, w, l) RoPE):
the pre-norm Q and K are the tensors above; `norm_weight` draws the per-channel
weights 1 + 0.1 z (bf16); `rope_table` builds the cos / sin of each token's
rotation angles from a synthetic 4-axis position grid (the pages give neither
the axis sizes nor the frequencies; see the function).

Inputs of the row-wise FP8 projection (report §02 stage 02; SGLang page latency
notes): `proj_inputs` draws the activation X ~ N(0, 1), the weight
W ~ N(0, 1/K) and the bias ~ N(0, 0.01), all bf16.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

STREAM_Q, STREAM_K, STREAM_V = 1, 2, 3
STREAM_K_OFF, STREAM_V_OFF, STREAM_Q_OFF = 4, 5, 6
STREAM_OUTLIER = 7
STREAM_QW, STREAM_KW = 8, 9
STREAM_PX, STREAM_PW, STREAM_PB = 10, 11, 12


def build() -> str:
    """Compile synth.c into libsynth.so next to it (gcc, OpenMP)."""
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        u64, i64, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double
        vp = ctypes.c_void_p
        lib.synth_u64.argtypes = [u64, u64, u64, i64, i64, vp]
        lib.synth_normal_f64.argtypes = [u64, u64, u64, i64, i64, vp]
        lib.synth_fill_f32.argtypes = [u64, u64, u64, i64, dbl, vp, vp, i64, vp]
        for f in (lib.synth_u64, lib.synth_normal_f64, lib.synth_fill_f32):
            f.restype = None
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def draws_u64(seed: int, config: int, stream: int, count: int, start: int = 0) -> np.ndarray:
    out = np.empty(count, dtype=np.uint64)
    _load().synth_u64(seed, config, stream, start, count, _ptr(out))
    return out


def normals(seed: int, config: int, stream: int, count: int, start: int = 0) -> np.ndarray:
    out = np.empty(count, dtype=np.float64)
    _load().synth_normal_f64(seed, config, stream, start, count, _ptr(out))
    return out


@dataclass(frozen=True)
class Dist:
    """sigma * z * (8 on outlier channels) + offset[h,d],  offset ~ N(0, off_var)."""
    var: float = 1.0
    outliers: bool = False
    off_var: Optional[float] = None


@dataclass(frozen=True)
class Config:
    idx: int
    name: str
    B: int
    H: int
    N: int
    D: int
    q: Dist = field(default_factory=Dist)
    k: Dist = field(default_factory=Dist)
    v: Dist = field(default_factory=Dist)
    outlier_frac: float = 0.01
    outlier_mult: float = 8.0

    @property
    def shape(self):
        return (self.B, self.N, self.H, self.D)


_FLUX_Q = Dist(1.0, outliers=True)
_FLUX_K = Dist(1.0, outliers=True, off_var=3.0)
_FLUX_V = Dist(1.0, off_var=1.0)

CONFIGS = (
    Config(0, "tiny", 1, 2, 256, 64, q=Dist(1.0), k=Dist(1.0, off_var=4.0), v=Dist(1.0)),
    Config(1, "flux_joint", 2, 24, 4608, 128, q=_FLUX_Q, k=_FLUX_K, v=_FLUX_V),
    Config(2, "video_early", 2, 24, 3128, 128, q=_FLUX_Q, k=_FLUX_K, v=_FLUX_V),
    Config(3, "long_t2v", 1, 40, 32760, 128, q=Dist(1.0), k=Dist(1.0, off_var=4.0),
           v=Dist(1.0, off_var=0.5)),
    Config(4, "quant_long", 1, 40, 32760, 128, q=Dist(1.0, off_var=4.0),
           k=Dist(1.0, off_var=4.0), v=Dist(1.0, off_var=4.0)),
)


def config(idx_or_name) -> Config:
    for c in CONFIGS:
        if c.idx == idx_or_name or c.name == idx_or_name:
            return c
    raise KeyError(idx_or_name)


def custom(B: int, N: int, H: int, D: int, q: Dist = Dist(), k: Dist = Dist(1.0, off_var=4.0),
           v: Dist = Dist(1.0, off_var=1.0), tag: int = 100) -> Config:
    """An ad-hoc shape; `tag` keys the random streams (distinct from configs 0-4)."""
    return Config(tag, f"custom{tag}", B, H, N, D, q=q, k=k, v=v)


def outlier_channels(cfg: Config, seed: int = 0) -> np.ndarray:
    """round(frac * H * D) distinct flat (h*D + d) indices: those with the smallest draws."""
    n_chan = cfg.H * cfg.D
    n_out = int(round(cfg.outlier_frac * n_chan))
    r = draws_u64(seed, cfg.idx, STREAM_OUTLIER, n_chan)
    return np.sort(np.argsort(r, kind="stable")[:n_out])


def _channel_terms(cfg: Config, dist: Dist, off_stream: int, seed: int):
    n_chan = cfg.H * cfg.D
    scale = None
    if dist.outliers:
        scale = np.ones(n_chan, dtype=np.float64)
        scale[outlier_channels(cfg, seed)] = cfg.outlier_mult
    off = None
    if dist.off_var is not None:
        off = normals(seed, cfg.idx, off_stream, n_chan) * math.sqrt(dist.off_var)
    return scale, off


def fill_f32(cfg: Config, which: str, seed: int = 0) -> np.ndarray:
    """fp32 values of one tensor ('q', 'k' or 'v'), row-major [B, N, H, D]."""
    dist = {"q": cfg.q, "k": cfg.k, "v": cfg.v}[which]
    stream = {"q": STREAM_Q, "k": STREAM_K, "v": STREAM_V}[which]
    off_stream = {"q": STREAM_Q_OFF, "k": STREAM_K_OFF, "v": STREAM_V_OFF}[which]
    scale, off = _channel_terms(cfg, dist, off_stream, seed)
    count = cfg.B * cfg.N * cfg.H * cfg.D
    out = np.empty(count, dtype=np.float32)
    _load().synth_fill_f32(seed, cfg.idx, stream, count, math.sqrt(dist.var), _ptr(scale),
                           _ptr(off), cfg.H * cfg.D, _ptr(out))
    return out.reshape(cfg.shape)


def make_qkv(cfg, seed: int = 0, device=None):
    """(q, k, v) as bf16 torch tensors [B, N, H, D] (contiguous NHD)."""
    import torch
    if not isinstance(cfg, Config):
        cfg = config(cfg)
    out = []
    for which in ("q", "k", "v"):
        t = torch.from_numpy(fill_f32(cfg, which, seed))
        if device is not None:
            t = t.to(device)
        out.append(t.to(torch.bfloat16))
    return tuple(out)


def query_subset(N: int, every: int = 8, block: int = 32) -> np.ndarray:
    """Stratified query rows: every `every`-th block of `block` queries, plus the last
    (possibly partial) block.  Used where the oracle cannot afford all rows."""
    nblk = (N + block - 1) // block
    blocks = sorted(set(range(0, nblk, every)) | {nblk - 1})
    rows = [r for b in blocks for r in range(b * block, min(N, (b + 1) * block))]
    return np.asarray(rows, dtype=np.int32)


def norm_weight(cfg, which: str, seed: int = 0):
    """RMSNorm weight of the Q ('q') or K ('k') norm: bf16 torch tensor [D],
    1 + 0.1 z, shared by every head."""
    import torch
    if not isinstance(cfg, Config):
        cfg = config(cfg)
    stream = {"q": STREAM_QW, "k": STREAM_KW}[which]
    w = 1.0 + 0.1 * normals(seed, cfg.idx, stream, cfg.D)
    return torch.from_numpy(w.astype(np.float32)).to(torch.bfloat16)


def rope_positions(N: int) -> np.ndarray:
    """Synthetic 4-axis positions [N, 4] = (t, h, w, l) of a joint sequence: the
    first min(512, N // 8) tokens are text (t = h = w = 0, l = index), the rest
    are video latents on a t x 16 x 32 grid (l = 0)."""
    n_text = min(512, N // 8)
    pos = np.zeros((N, 4), np.int64)
    pos[:n_text, 3] = np.arange(n_text)
    j = np.arange(N - n_text)
    pos[n_text:, 0] = j // 512
    pos[n_text:, 1] = (j // 32) % 16
    pos[n_text:, 2] = j % 32
    return pos


def rope_table(N: int, D: int, theta: float = 10000.0) -> np.ndarray:
    """cos / sin of the rotation angles: fp32 [N, D/2, 2].  The D/2 channel pairs
    are split over the axes (t, h, w, l) as (1, 3, 3, 1) eighths; pair i of an
    axis with d pairs turns at pos * theta^(-i/d).  Angles and cos / sin are fp64,
    rounded once to fp32."""
    P = D // 2
    split = [P // 8, 3 * P // 8, 3 * P // 8, P // 8]
    pos = rope_positions(N).astype(np.float64)
    ang = np.empty((N, P), np.float64)
    c0 = 0
    for a, d in enumerate(split):
        freq = theta ** (-np.arange(d, dtype=np.float64) / d)
        ang[:, c0:c0 + d] = pos[:, a:a + 1] * freq[None, :]
        c0 += d
    out = np.empty((N, P, 2), np.float32)
    out[..., 0] = np.cos(ang)
    out[..., 1] = np.sin(ang)
    return out


PROJ_SHAPES = {
    # the V + MLP projection of a FLUX.3-Action-like joint block: tokens
    # B*N = 2*4608, hidden H*D = 24*128, outputs V (hidden) + MLP (4 hidden)
    "vmlp_proj": (2 * 4608, 3072, 3072 + 4 * 3072),
}


def proj_inputs(M: int, K: int, N: int, seed: int = 0, tag: int = 200):
    """(x [M, K], w [N, K], bias [N]) bf16 torch tensors; `tag` keys the streams."""
    import torch
    x = normals(seed, tag, STREAM_PX, M * K).reshape(M, K)
    w = normals(seed, tag, STREAM_PW, N * K).reshape(N, K) / math.sqrt(K)
    b = normals(seed, tag, STREAM_PB, N) * 0.1
    cast = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)
    return cast(x), cast(w), cast(b)
