"""GPU parity of the row-wise FP8 projection (report §02 stage 02; SGLang page
latency notes) through the C ABI: sage_quant_rows_fp8 bit-exact against the
oracle's row quantiser; sage_gemm_fp8_rowwise against the oracle's fp64 scaled
GEMM on the same codes, element by element within
    ulp_bf16(|ref|) + 2^-10 * blk + 2^-20 * absum.
One bf16 rounding of the result; the matrix cores' accumulation, which adds
each 64-product block to the running value keeping a fixed number of bits
below the larger of the two (measured on gfx950 for v_mfma_f32_32x32x64_f8f6f4:
error <= 2^-10.8 x max(|running value|, largest product) per instruction;
blk sums that magnitude over the blocks with exact partial sums); and the fp32
scale and bias operations, relative to the magnitude sum absum."""
import sys

import numpy as np
import pytest
import torch

import oracle
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


def _ulp_bf16(v):
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def _check_gemm(got, ref, absum, blk):
    got = got.double().numpy()
    tol = _ulp_bf16(ref) + 2.0 ** -10 * blk + 2.0 ** -20 * absum
    err = np.abs(got - ref)
    bad = err > tol
    assert not bad.any(), f"{bad.sum()} entries out of bound; worst {(err / tol).max():.2f} x tol"
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


@pytest.mark.parametrize("M,K", [(1, 8), (37, 256), (300, 3072), (5, 16384)])
def test_quant_rows_bits(sage, M, K):
    _log(f"[proj] quant rows M{M} K{K}")
    x, _, _ = synth.proj_inputs(M, K, 4, tag=610 + M)
    x[min(2, M - 1)] = 0                          # a zero row
    wide = torch.zeros(M, K + 64, dtype=torch.bfloat16)
    wide[:, 32:32 + K] = x                        # rows read from a wider buffer
    xv = wide.cuda()[:, 32:32 + K]
    codes, scales = sage.quant_rows_fp8(xv)
    torch.cuda.synchronize()
    rc, rs = oracle.quant_rows_e4m3(x)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)
    np.testing.assert_array_equal(scales.cpu().numpy().view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("M,K,N,with_bias", [(37, 128, 28, True), (300, 384, 260, False),
                                              (513, 1024, 516, True), (256, 256, 256, True),
                                              (70, 16384, 132, True)])
def test_gemm_small_full(sage, M, K, N, with_bias):
    """Ragged M and N (partial 256-blocks on both sides), K up to its limit of
    16384 (256 k-stages), every entry checked."""
    _log(f"[proj] gemm M{M} K{K} N{N} bias {with_bias}")
    x, w, b = synth.proj_inputs(M, K, N, tag=620 + M)
    xc, xs = sage.quant_rows_fp8(x.cuda())
    wc, ws = sage.quant_rows_fp8(w.cuda())
    bias = b.cuda() if with_bias else None
    out = sage.gemm_fp8_rowwise(xc, xs, wc, ws, bias=bias)
    torch.cuda.synchronize()
    ref, absum, blk = oracle.gemm_fp8_rowwise(xc.cpu().numpy(), xs.cpu().numpy(), wc.cpu().numpy(),
                                              ws.cpu().numpy(), bias=b if with_bias else None)
    e = _check_gemm(out.cpu(), ref, absum, blk)
    _log(f"  rel L2 vs fp64 oracle {e:.3e}")
    assert e < 4e-3


@pytest.mark.parametrize("N,extra,off", [(200, 128, 64), (200, 132, 4), (196, 132, 68)],
                         ids=["ldo%8=0,16B-aligned", "ldo%8=4,8B-aligned", "N%8=4,ldo%8=0,8B-aligned"])
def test_gemm_into_a_column_slice(sage, N, extra, off):
    """The output written into columns [off, off+N) of a wider buffer (row
    pitch N + extra elements): equal to the contiguous output, the rest of the
    buffer untouched.  Covers 16-byte row stores and the 8-byte ones used when
    the pitch or the base allows no more."""
    M, K = 130, 256
    _log(f"[proj] column slice N{N} pitch {N + extra} offset {off}")
    x, w, b = synth.proj_inputs(M, K, N, tag=630)
    xc, xs = sage.quant_rows_fp8(x.cuda())
    wc, ws = sage.quant_rows_fp8(w.cuda())
    buf = torch.full((M, N + extra), 7.0, dtype=torch.bfloat16, device="cuda")
    view = buf[:, off:off + N]
    sage.gemm_fp8_rowwise(xc, xs, wc, ws, bias=b.cuda(), out=view)
    ref_out = sage.gemm_fp8_rowwise(xc, xs, wc, ws, bias=b.cuda())
    torch.cuda.synchronize()
    assert torch.equal(view, ref_out)
    assert torch.all(buf[:, :off] == 7) and torch.all(buf[:, off + N:] == 7)


def test_vmlp_projection_sampled_and_v_alias(sage):
    """V + MLP projection of a FLUX-like block (M 9216, K 3072, N 15360): the
    GEMM on sampled entries against the oracle, and sage_quant_v reading the V
    part of the output in place (bit-identical to quantising a copy)."""
    M, K, N = synth.PROJ_SHAPES["vmlp_proj"]
    _log(f"[proj] vmlp M{M} K{K} N{N}")
    x, w, b = synth.proj_inputs(M, K, N)
    xc, xs = sage.quant_rows_fp8(x.cuda())
    wc, ws = sage.quant_rows_fp8(w.cuda())
    out = sage.gemm_fp8_rowwise(xc, xs, wc, ws, bias=b.cuda())
    torch.cuda.synchronize()
    rc, rs = oracle.quant_rows_e4m3(x)
    np.testing.assert_array_equal(xc.cpu().numpy(), rc)
    wcc = wc.cpu().numpy()
    np.testing.assert_array_equal(wcc, oracle.quant_rows_e4m3(w)[0])
    rows = np.unique(np.concatenate([np.arange(0, M, 97), [M - 1, 255, 256]])).astype(np.int32)
    cols = np.unique(np.concatenate([np.arange(0, N, 61), [N - 1, 255, 256, 3071, 3072]])).astype(np.int32)
    ref, absum, blk = oracle.gemm_fp8_rowwise(rc, rs, wcc, ws.cpu().numpy(), bias=b, rows=rows, cols=cols)
    got = out.cpu()[rows][:, cols]
    e = _check_gemm(got, ref, absum, blk)
    _log(f"  {rows.size} x {cols.size} entries, rel L2 vs fp64 oracle {e:.3e}")
    # V = the first H*D = 3072 output columns, read as [B, N, H, D] with token stride 15360
    B, Ntok, H, D = 2, 4608, 24, 128
    v_view = out.view(B, Ntok, N)[:, :, :H * D].view(B, Ntok, H, D)
    vq_alias = sage.quant_v(v_view)
    vq_copy = sage.quant_v(v_view.contiguous())
    torch.cuda.synchronize()
    for a, c in zip(vq_alias, vq_copy):
        assert torch.equal(a, c)
