"""Pins for the oracle's codecs (bf16, E4M3FN, INT8) against library casts,
exhaustive enumeration and brute-force nearest-even search.

The E4M3 layout (1 sign, 4 exponent, 3 mantissa bits) is the one stated in the
A10 FLUX.1 article, §1.1; the library cross-check is torch's float8_e4m3fn.
"""
import numpy as np
import pytest
import torch

import oracle


def _f32_bits(n, rng):
    bits = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    return x[np.isfinite(x)]


def _torch_bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_round_matches_torch_random_bits():
    rng = np.random.default_rng(0)
    x = _f32_bits(2_000_000, rng)
    np.testing.assert_array_equal(oracle.bf16_round(x), _torch_bf16_bits(x))


def test_bf16_round_ties_to_even():
    # low 16 bits exactly one half of a bf16 ulp: must go to the even neighbour
    upper = np.arange(0, 0x7F7F, 7, dtype=np.uint32)
    bits = (upper << 16) | 0x8000
    x = bits.view(np.float32)
    got = oracle.bf16_round(x)
    want = np.where(upper & 1, upper + 1, upper).astype(np.uint16)
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(got, _torch_bf16_bits(x))
    # just above / below the tie
    np.testing.assert_array_equal(oracle.bf16_round(((upper << 16) | 0x8001).view(np.float32)), (upper + 1).astype(np.uint16))
    np.testing.assert_array_equal(oracle.bf16_round(((upper << 16) | 0x7FFF).view(np.float32)), upper.astype(np.uint16))


def test_bf16_roundtrip_all_patterns():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = (h.astype(np.uint32) << 16).view(np.float32)
    finite = np.isfinite(vals) | np.isinf(vals)
    np.testing.assert_array_equal(oracle.bf16_round(vals[finite]), h[finite])
    assert all(oracle._load().orc_bf16_value(int(i)) == vals[i] for i in (0, 1, 0x3F80, 0x8000, 0x7F7F, 0xFF7F))


def _torch_e4m3_values():
    codes = torch.arange(256, dtype=torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_decode_all_codes_matches_torch():
    want = _torch_e4m3_values()
    got = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    np.testing.assert_array_equal(got[ok], want[ok])
    # layout facts: 1 sign, 4 exponent, 3 mantissa bits; max finite 448; NaN only at S.1111.111
    assert np.nanmax(got) == 448.0 and np.nanmin(got) == -448.0
    assert np.isnan(got).sum() == 2 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def _finite_pos_values():
    v = _torch_e4m3_values()[:0x7F]  # codes 0x00..0x7E, increasing
    assert np.all(np.diff(v) > 0)
    return v


def _brute_e4m3(x: float) -> int:
    """Nearest finite code by exhaustive search; ties to the even code; saturate."""
    vals = _finite_pos_values()
    a = abs(x)
    sign = 0x80 if np.signbit(x) else 0
    if a >= vals[-1]:
        return sign | 0x7E
    d = np.abs(vals - a)
    best = np.flatnonzero(d == d.min())
    if best.size == 2:  # exact midpoint -> even code
        c = int(best[0] if best[0] % 2 == 0 else best[1])
    else:
        c = int(best[0])
    return sign | c


def test_e4m3_encode_midpoints_and_exact_values():
    vals = _finite_pos_values()
    mids = (vals[:-1] + vals[1:]) / 2
    probe = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                            [448.0, 449.0, 463.99, 464.0, 500.0, 1e30, 1e-30, 2.0**-10, 2.0**-10 * 1.0001]])
    probe = np.concatenate([probe, -probe, [0.0, -0.0]])
    got = oracle.e4m3_encode(probe)
    want = np.array([_brute_e4m3(float(x)) for x in probe], np.uint8)
    np.testing.assert_array_equal(got, want)


def test_e4m3_encode_matches_torch_random():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(400_000) * 100.0,
        rng.standard_normal(200_000) * 0.01,
        rng.uniform(-448, 448, 200_000),
        rng.uniform(-2**-6, 2**-6, 100_000),
    ]).astype(np.float32)
    got = oracle.e4m3_encode(x.astype(np.float64))
    want = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got, want)


def test_e4m3_encode_sign_of_zero():
    assert oracle.e4m3_encode(np.array([0.0]))[0] == 0x00
    assert oracle.e4m3_encode(np.array([-0.0]))[0] == 0x80
    assert oracle.e4m3_encode(np.array([-1e-9]))[0] == 0x80  # rounds to -0


def test_i8_code_rne_and_clamp():
    for x, want in [(0.5, 0), (1.5, 2), (2.5, 2), (-0.5, 0), (-1.5, -2), (126.5, 126), (127.4, 127),
                    (127.5, 127), (300.0, 127), (-128.0, -127), (-127.5, -127), (0.49999997, 0)]:
        assert oracle.i8_code(x) == want, x
    rng = np.random.default_rng(2)
    xs = (rng.standard_normal(20000) * 80).astype(np.float32)
    got = np.array([oracle.i8_code(float(x)) for x in xs])
    np.testing.assert_array_equal(got, np.clip(np.rint(xs), -127, 127))


def test_v_slot_is_bijection_on_64():
    slots = [oracle.v_slot(t) for t in range(64)]
    assert sorted(slots) == list(range(64))


def test_golden_layout_fixture():
    """The E4M3 layout fixture (page-stated bit split) agrees with the decoder:
    4 exponent bits give 16 binades of 8 mantissa steps each."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "e4m3_layout.txt")
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    table = {r[0]: tuple(int(x) for x in r[1:]) for r in rows[1:]}
    s, e, m = table["e4m3"]
    assert s + e + m == 8
    vals = oracle.e4m3_decode(np.arange(1 << (e + m), dtype=np.uint8))
    finite = vals[~np.isnan(vals)]
    assert finite.size == (1 << (e + m)) - 1
    # within each normal binade the step is constant: 2^m values per binade
    for be in range(1, 1 << e):
        seg = oracle.e4m3_decode(np.arange(be << m, (be + 1) << m, dtype=np.uint8))
        seg = seg[~np.isnan(seg)]
        assert np.allclose(np.diff(seg), seg[0] / (1 << m))
