"""sage_quant_qk_static (the quantiser entry point that allocates nothing: its
workspace is a static device array in the library) against sage_quant_qk with
a caller workspace, bit for bit, on calls in a row, each smaller than the one
before (each finds the array holding the previous call's contents); and the
size limit, checked on the host before any launch.  Collected last: it must
pass after every other GPU test as well as alone."""
import sys

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

SAGE_ERR_WORKSPACE = -6


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


def _static_call(sage, q, k):
    B, N, H, D = q.shape
    Np = sage.sage_padded_tokens(N)
    dev = q.device
    outs = [torch.full((B, H, Np, D), 77, dtype=torch.int8, device=dev),
            torch.full((B, H, Np // 32), 7.0, dtype=torch.float32, device=dev),
            torch.full((B, H, Np, D), 77, dtype=torch.int8, device=dev),
            torch.full((B, H, Np // 64), 7.0, dtype=torch.float32, device=dev),
            torch.full((B, H, D), 7.0, dtype=torch.bfloat16, device=dev)]
    st = sage.lib().sage_quant_qk_static(q.data_ptr(), *q.stride()[:3], k.data_ptr(), *k.stride()[:3],
                                         B, N, H, D, *[t.data_ptr() for t in outs],
                                         torch.cuda.current_stream().cuda_stream)
    assert st == 0, f"sage_quant_qk_static returned {st}"
    return outs


def test_static_scratch_matches_workspace_path(sage):
    # first the larger call, then a smaller one: the second finds the array
    # holding the first call's contents
    for cfg in (synth.config(1), synth.custom(1, 200, 3, 128, tag=601), synth.config(0)):
        _log(f"[no-alloc] {cfg.name} B{cfg.B} N{cfg.N} H{cfg.H} D{cfg.D}")
        q, k, _ = synth.make_qkv(cfg, device="cuda")
        got = _static_call(sage, q, k)
        ref = sage.quant_qk(q, k)
        torch.cuda.synchronize()
        for name, a, b in zip(("q_i8", "q_scale", "k_i8", "k_scale", "k_mean"), got, ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), name


def test_static_scratch_size_limit(sage):
    # 20000 heads: one statistics chunk each, a 51 MB workspace > 16 MiB
    B, N, H, D = 1, 64, 20000, 128
    assert sage.sage_quant_qk_workspace_size(B, N, H, D) > 16 << 20
    q = torch.zeros((B, N, H, D), dtype=torch.bfloat16, device="cuda")
    Np = 64
    outs = [torch.empty((B, H, Np, D), dtype=torch.int8, device="cuda"),
            torch.empty((B, H, Np // 32), dtype=torch.float32, device="cuda"),
            torch.empty((B, H, Np, D), dtype=torch.int8, device="cuda"),
            torch.empty((B, H, Np // 64), dtype=torch.float32, device="cuda"),
            torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")]
    st = sage.lib().sage_quant_qk_static(q.data_ptr(), *q.stride()[:3], q.data_ptr(), *q.stride()[:3],
                                         B, N, H, D, *[t.data_ptr() for t in outs],
                                         torch.cuda.current_stream().cuda_stream)
    assert st == SAGE_ERR_WORKSPACE
