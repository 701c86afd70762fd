"""The path captured in a HIP graph (torch.cuda.CUDAGraph around the C-ABI
calls, with sage_quant_v forked to a second stream and joined back): every
replay, with eager work and synchronisations of the program's own in between,
is bit-identical to the eager result.  The library allocates nothing and
records no memset, so a capture holds only its kernels."""
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


@pytest.mark.parametrize("cfg", [synth.custom(1, 777, 4, 128, tag=801), synth.config(1)],
                         ids=lambda c: f"{c.name}-B{c.B}N{c.N}H{c.H}D{c.D}")
def test_graph_replays_match_eager(sage, cfg):
    _log(f"[graph] {cfg.name} B{cfg.B} N{cfg.N} H{cfg.H} D{cfg.D}")
    lib = sage.lib()
    B, N, H, D = cfg.B, cfg.N, cfg.H, cfg.D
    Np = sage.sage_padded_tokens(N)
    dev = torch.device("cuda")
    q, k, v = (t.to(dev) for t in synth.make_qkv(cfg))
    eager_qk = sage.quant_qk(q, k)
    eager_v = sage.quant_v(v)
    eager_out = sage.attn_fwd(*eager_qk[:4], *eager_v, N=N)
    torch.cuda.synchronize()

    q_i8 = torch.empty((B, H, Np, D), dtype=torch.int8, device=dev)
    q_scale = torch.empty((B, H, Np // 32), dtype=torch.float32, device=dev)
    k_i8 = torch.empty_like(q_i8)
    k_scale = torch.empty((B, H, Np // 64), dtype=torch.float32, device=dev)
    k_mean = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
    v_fp8 = torch.empty((B, H, D, Np), dtype=torch.uint8, device=dev)
    v_scale = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    v_mean = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    out = torch.empty((B, N, H, D), dtype=torch.bfloat16, device=dev)
    ws_qk = torch.zeros(sage.sage_quant_qk_workspace_size(B, N, H, D), dtype=torch.uint8, device=dev)
    ws_v = torch.zeros(sage.sage_quant_v_workspace_size(B, N, H, D), dtype=torch.uint8, device=dev)
    qs, ks, vs, os_ = q.stride()[:3], k.stride()[:3], v.stride()[:3], out.stride()[:3]

    g = torch.cuda.CUDAGraph()
    cap, side = torch.cuda.Stream(), torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=cap):
        cp, sp = int(cap.cuda_stream), int(side.cuda_stream)
        side.wait_stream(cap)
        st = lib.sage_quant_v(v.data_ptr(), *vs, B, N, H, D, v_fp8.data_ptr(), v_scale.data_ptr(),
                              v_mean.data_ptr(), ws_v.data_ptr(), ws_v.numel(), sp)
        st |= lib.sage_quant_qk(q.data_ptr(), *qs, k.data_ptr(), *ks, B, N, H, D, q_i8.data_ptr(),
                                q_scale.data_ptr(), k_i8.data_ptr(), k_scale.data_ptr(),
                                k_mean.data_ptr(), ws_qk.data_ptr(), ws_qk.numel(), cp)
        cap.wait_stream(side)
        st |= lib.sage_attn_fwd(q_i8.data_ptr(), q_scale.data_ptr(), k_i8.data_ptr(),
                                k_scale.data_ptr(), v_fp8.data_ptr(), v_scale.data_ptr(),
                                v_mean.data_ptr(), B, N, H, D, 0.0, out.data_ptr(), *os_, cp)
    assert st == 0
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (q_i8, k_i8, v_fp8, out):
            t.zero_()  # eager work between replays; the replay must rewrite every output
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        # eager library work between replays, on other buffers
        sage.attn_fwd(*eager_qk[:4], *eager_v, N=N)
        torch.cuda.synchronize()
        for got, want in ((q_i8, eager_qk[0]), (q_scale, eager_qk[1]), (k_i8, eager_qk[2]),
                          (k_scale, eager_qk[3]), (k_mean, eager_qk[4]), (v_fp8, eager_v[0]),
                          (v_scale, eager_v[1]), (v_mean, eager_v[2])):
            assert torch.equal(got, want), rep
        same = torch.equal(out.view(torch.int16), eager_out.view(torch.int16))
        _log(f"  replay {rep}: every output bit-identical to eager: {same}")
        assert same
