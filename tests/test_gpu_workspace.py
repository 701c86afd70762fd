"""The quantisers' workspace contract, through the C ABI: one workspace,
zero-filled once, serves any sequence of calls ordered on one stream, whatever
their shapes, because every call leaves its arrival counters zero.  A sequence
of shapes with many, few and one statistics chunk per head, one of them with a
channel that takes the exact re-summation path, runs on one shared K/Q and one
shared V workspace; every call's codes, scales and means are bit-exact against
the oracle, and the counter region is zero after every call."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.test_gpu_parity import _check_quant_bits, _tiny_channel

pytestmark = pytest.mark.gpu

SHAPES = [(1, 4608, 3, 128), (2, 1000, 5, 64), (1, 300, 2, 128), (1, 2048, 2, 128), (1, 4608, 3, 128)]


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


def test_one_workspace_for_a_sequence_of_calls(sage):
    lib = sage.lib()
    dev = torch.device("cuda")
    s = torch.cuda.current_stream().cuda_stream
    zb = lib.sage_workspace_zero_bytes()
    n_qk = max(lib.sage_quant_qk_workspace_size(*sh) for sh in SHAPES)
    n_v = max(lib.sage_quant_v_workspace_size(*sh) for sh in SHAPES)
    ws_qk = torch.zeros(n_qk, dtype=torch.uint8, device=dev)
    ws_v = torch.zeros(n_v, dtype=torch.uint8, device=dev)
    for i, (B, N, H, D) in enumerate(SHAPES):
        cfg = synth.custom(B, N, H, D, tag=600 + i)
        q, k, v = synth.make_qkv(cfg)
        if i == 3:  # one K and one V channel on the exact re-summation path
            col = _tiny_channel(N, 2.0 ** -100)
            k[0, :, H - 1, 7] = col
            v[0, :, 0, 11] = col
        _log(f"[workspace] call {i}: B{B} N{N} H{H} D{D}")
        Np = sage.sage_padded_tokens(N)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        qk = [torch.empty((B, H, Np, D), dtype=torch.int8, device=dev),
              torch.empty((B, H, Np // 32), dtype=torch.float32, device=dev),
              torch.empty((B, H, Np, D), dtype=torch.int8, device=dev),
              torch.empty((B, H, Np // 64), dtype=torch.float32, device=dev),
              torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)]
        vq = [torch.empty((B, H, D, Np), dtype=torch.uint8, device=dev),
              torch.empty((B, H, D), dtype=torch.float32, device=dev),
              torch.empty((B, H, D), dtype=torch.float32, device=dev)]
        st = lib.sage_quant_qk(qd.data_ptr(), *qd.stride()[:3], kd.data_ptr(), *kd.stride()[:3], B, N, H, D,
                               *[t.data_ptr() for t in qk], ws_qk.data_ptr(), ws_qk.numel(), s)
        assert st == 0
        st = lib.sage_quant_v(vd.data_ptr(), *vd.stride()[:3], B, N, H, D, *[t.data_ptr() for t in vq],
                              ws_v.data_ptr(), ws_v.numel(), s)
        assert st == 0
        torch.cuda.synchronize()
        assert int(ws_qk[:zb].count_nonzero()) == 0 and int(ws_v[:zb].count_nonzero()) == 0
        ref_qk, ref_v = oracle.quant_qk(q, k), oracle.quant_v(v)
        if i == 3:
            assert ref_qk["inexact"] >= 1 and ref_v["inexact"] >= 1
        _check_quant_bits(qk, vq, ref_qk, ref_v, N)
