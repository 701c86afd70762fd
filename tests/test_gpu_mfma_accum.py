"""The FP8 matrix-core instruction that both the attention's P.V and the
row-wise FP8 GEMM accumulate with (v_mfma_f32_32x32x64_f8f6f4, E4M3 operands,
fp32 accumulator), run on host-chosen operands and compared with the exact
fp64 sum.

The FP8 GEMM's per-element tolerance and the attention's distance from the
oracle both rest on how this instruction sums its 64 products: not as an
fp32-exact sum, but within 2^-10 * max(|C|, largest |product|) of the exact
value (the constant of the GEMM's per-element bound; the worst case measured
over the full E4M3 range is about 2^-10.8).  This test holds that model (and
the operand layout the kernels use) to the hardware, with zero and with random
C.
"""
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

BOUND = 2.0 ** -10


def _log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import mfma_probe
    return mfma_probe.load()


def _e4m3_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] ^= 0x01  # no NaN codes
    return c


def _decode(codes):
    return torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()


def _operands(a_codes, b_codes):
    """Per-wave matrices from the per-lane bytes: A [W, 32, 64], B [W, 64, 32]."""
    W = a_codes.shape[0]
    av = _decode(a_codes)  # [W, 64 lanes, 32 bytes]
    bv = _decode(b_codes)
    A = np.empty((W, 32, 64))
    Bm = np.empty((W, 64, 32))
    for l in range(64):
        A[:, l % 32, 32 * (l // 32):32 * (l // 32) + 32] = av[:, l]
        Bm[:, 32 * (l // 32):32 * (l // 32) + 32, l % 32] = bv[:, l]
    return A, Bm


def _cd_index():
    """(row, col) of register i of lane l in the 32 x 32 accumulator."""
    rows = np.empty((64, 16), np.int64)
    cols = np.empty((64, 16), np.int64)
    for l in range(64):
        for i in range(16):
            rows[l, i] = 8 * (i // 4) + 4 * (l // 32) + i % 4
            cols[l, i] = l % 32
    return rows, cols


def _run(probe, a_codes, b_codes, c_lanes):
    dev = torch.device("cuda")
    W = a_codes.shape[0]
    a = torch.from_numpy(a_codes).to(dev)
    b = torch.from_numpy(b_codes).to(dev)
    c = torch.from_numpy(c_lanes.astype(np.float32)).to(dev)
    d = torch.empty_like(c)
    s = torch.cuda.current_stream().cuda_stream
    st = probe.probe_mfma_f8(a.data_ptr(), b.data_ptr(), c.data_ptr(), d.data_ptr(), W, s)
    assert st == 0
    torch.cuda.synchronize()
    return d.cpu().double().numpy()


def _check(d_lanes, c_lanes, A, Bm, label):
    rows, cols = _cd_index()
    W = A.shape[0]
    C = np.zeros((W, 32, 32))
    D = np.zeros((W, 32, 32))
    C[:, rows, cols] = c_lanes
    D[:, rows, cols] = d_lanes
    exact = C + np.einsum("wmk,wkn->wmn", A, Bm)
    prod_max = np.zeros((W, 32, 32))
    for k in range(64):
        prod_max = np.maximum(prod_max, np.abs(A[:, :, k, None]) * np.abs(Bm[:, None, k, :]))
    scale = np.maximum(np.abs(C), prod_max)
    err = np.abs(D - exact)
    ratio = np.where(scale > 0, err / np.where(scale > 0, scale, 1.0), err)
    rounded = np.float32(exact).astype(np.float64)
    _log(f"  {label}: {D.size} results, max |D - exact| / max(|C|, max|prod|) = 2^{np.log2(ratio.max() + 1e-300):.2f}"
         f" (bound 2^-10); {np.mean(D != rounded) * 100:.1f}% differ from fp32(exact)")
    assert np.isfinite(D).all()
    assert (ratio <= BOUND).all()


@pytest.mark.parametrize("c_kind", ["zero", "random"])
def test_fp8_mfma_accumulation_bound(probe, c_kind):
    rng = np.random.default_rng(7 if c_kind == "zero" else 8)
    W = 4096
    a_codes = _e4m3_codes(rng, (W, 64, 32))
    b_codes = _e4m3_codes(rng, (W, 64, 32))
    if c_kind == "zero":
        c_lanes = np.zeros((W, 64, 16))
    else:
        c_lanes = rng.standard_normal((W, 64, 16)) * np.exp2(rng.integers(-8, 17, size=(W, 64, 16)))
        c_lanes = c_lanes.astype(np.float32).astype(np.float64)
    A, Bm = _operands(a_codes, b_codes)
    d = _run(probe, a_codes, b_codes, c_lanes)
    _check(d, c_lanes, A, Bm, f"C {c_kind}")


@pytest.mark.parametrize("c_kind", ["zero", "offset", "random"])
def test_int8_mfma_is_exact(probe, c_kind):
    """v_mfma_i32_32x32x32_i8 (the attention's Q K^T): D = C + A B exactly in
    int32, for a zero C, the constant 0x4B400000 and random C."""
    rng = np.random.default_rng(20)
    W = 1024
    a_codes = rng.integers(-127, 128, size=(W, 64, 16), dtype=np.int8)
    b_codes = rng.integers(-127, 128, size=(W, 64, 16), dtype=np.int8)
    if c_kind == "zero":
        c_lanes = np.zeros((W, 64, 16), np.int32)
    elif c_kind == "offset":
        c_lanes = np.full((W, 64, 16), 0x4B400000, np.int32)
    else:
        c_lanes = rng.integers(-2 ** 30, 2 ** 30, size=(W, 64, 16), dtype=np.int32)
    A = np.zeros((W, 32, 32), np.int64)
    Bm = np.zeros((W, 32, 32), np.int64)
    for l in range(64):
        A[:, l % 32, 16 * (l // 32):16 * (l // 32) + 16] = a_codes[:, l]
        Bm[:, 16 * (l // 32):16 * (l // 32) + 16, l % 32] = b_codes[:, l]
    rows, cols = _cd_index()
    C = np.zeros((W, 32, 32), np.int64)
    C[:, rows, cols] = c_lanes
    exact = C + np.einsum("wmk,wkn->wmn", A, Bm)
    dev = torch.device("cuda")
    a = torch.from_numpy(a_codes).to(dev)
    b = torch.from_numpy(b_codes).to(dev)
    c = torch.from_numpy(c_lanes).to(dev)
    d = torch.empty_like(c)
    assert probe.probe_mfma_i8(a.data_ptr(), b.data_ptr(), c.data_ptr(), d.data_ptr(), W,
                               torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    D = np.zeros((W, 32, 32), np.int64)
    D[:, rows, cols] = d.cpu().numpy()
    _log(f"  int8 MFMA, C {c_kind}: {np.count_nonzero(D != exact)} of {D.size} results differ from C + A B")
    assert np.array_equal(D, exact)
