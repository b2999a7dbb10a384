"""Pins of the oracle's element formats against the format definitions and library routines.

E2M1 table and maximum: Megatron-Core "core.inference.moe.flashinfer_nvfp4" module data
(FLOAT4_E2M1_MAX = 6.0).  E4M3 maximum: same module (FLOAT8_E4M3_MAX = 448.0); the scale type is
torch.float8_e4m3fn (alphamoe_nvfp4_aligned_moe page), so torch's own float8_e4m3fn conversion is
an independent routine to check decoding and in-range rounding against.  BF16 rounding is checked
against torch's float32 -> bfloat16 conversion.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.formats import E4M3_TABLE


def test_e2m1_table_and_max():
    vals = oracle.e2m1_decode(np.arange(16))
    expect = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(vals[:8]) == expect
    assert list(vals[8:]) == [-v for v in expect]
    assert np.signbit(vals[8])                      # code 0x8 is -0
    assert vals.max() == oracle.FLOAT4_E2M1_MAX == 6.0
    # Format definition written independently: s.e1e0.m, bias 1, one mantissa bit.
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        mag = m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)
        assert vals[c] == (-mag if s else mag)


def test_e4m3_decode_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_decode(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert sorted(np.nonzero(nan)[0].tolist()) == [0x7F, 0xFF]
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.nanmax(got) == oracle.FLOAT8_E4M3_MAX == 448.0
    assert got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6 and got[0x38] == 1.0
    assert np.all(np.diff(E4M3_TABLE[:0x7F]) > 0)   # code order == value order


def _f32_sweep():
    """Every float32 in [2**-12, 480] on a fine stride, plus all E4M3 midpoints +- 1 ulp."""
    lo = np.float32(2.0 ** -12).view(np.int32)
    hi = np.float32(480.0).view(np.int32)
    dense = np.arange(lo, hi, 97, dtype=np.int32).view(np.float32)
    g = E4M3_TABLE[:0x7F]
    mids = ((g[1:] + g[:-1]) / 2).astype(np.float32)      # exact in float32
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)), g.astype(np.float32)])
    return np.concatenate([dense, near, np.array([0.0, 2.0 ** -10, 447.99, 448.0], np.float32)])


def test_e4m3_encode_matches_torch_in_range():
    v = _f32_sweep()
    v = v[v <= 448.0]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode(v)
    assert np.array_equal(ref, got)


def test_e4m3_encode_saturates():
    v = np.array([448.0, 449.0, 463.99, 464.0, 1000.0, 3.0e38], dtype=np.float32)
    assert list(oracle.e4m3_encode(v)) == [0x7E] * 6


E2M1_MIDPOINTS = [  # (midpoint, code it rounds to): ties go to the even code
    (0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)]


def test_e2m1_encode_ties_and_neighbours():
    for mid, code in E2M1_MIDPOINTS:
        m = np.float32(mid)
        below = np.nextafter(m, np.float32(0))
        above = np.nextafter(m, np.float32(100))
        assert oracle.e2m1_encode(np.array([m]))[0] == code
        assert oracle.e2m1_encode(np.array([-m]))[0] == code | 8
        lo_code = oracle.e2m1_encode(np.array([below]))[0]
        hi_code = oracle.e2m1_encode(np.array([above]))[0]
        # just below the midpoint: the lower neighbour; just above: the upper one
        assert oracle.e2m1_decode([lo_code])[0] < mid < oracle.e2m1_decode([hi_code])[0]


def test_e2m1_encode_brute_force_nearest():
    """Dense sweep: the chosen value is a nearest grid value; saturation above 6; sign copy."""
    rng = np.random.default_rng(0)
    y = np.concatenate([rng.uniform(-8, 8, 200000), np.linspace(-7, 7, 28001)]).astype(np.float32)
    codes = oracle.e2m1_encode(y)
    vals = oracle.e2m1_decode(codes)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    dist = np.abs(np.abs(y.astype(np.float64))[:, None] - grid[None, :]).min(axis=1)
    sat = np.abs(y) > 6
    assert np.all(np.abs(np.abs(y[~sat]) - np.abs(vals[~sat])) == dist[~sat])
    assert np.all(np.abs(vals[sat]) == 6)
    assert np.array_equal(np.signbit(y), (codes & 8) != 0)
    assert oracle.e2m1_encode(np.array([-0.0], np.float32))[0] == 8
    assert oracle.e2m1_encode(np.array([-1e-30], np.float32))[0] == 8


def test_bf16_rounding_matches_torch_for_float32():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, 300000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    x = x[np.abs(x) < 3.0e38]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_to_bf16(x.astype(np.float64))
    assert np.array_equal(ref, got)


def test_bf16_rounding_float64_ties():
    q = 2.0 ** -7                                    # BF16 spacing in [1, 2)
    assert oracle.round_to_bf16(np.array([1 + q / 2]))[0] == 1.0            # tie -> even
    assert oracle.round_to_bf16(np.array([1 + 3 * q / 2]))[0] == 1 + 2 * q  # tie -> even
    assert oracle.round_to_bf16(np.array([1 + q / 2 + 2.0 ** -40]))[0] == 1 + q
    assert oracle.round_to_bf16(np.array([1 + q / 2 - 2.0 ** -40]))[0] == 1.0
    assert oracle.round_to_bf16(np.array([2.0 ** -133 * 1.5]))[0] == 2.0 ** -132   # subnormal tie
    bits = oracle.f64_to_bf16_bits(np.array([1.0, -2.0, 2.0 ** -24]))
    assert list(bits) == [0x3F80, 0xC000, 0x3380]


@pytest.mark.parametrize("v", [0.0, -0.0, 1.5, -3.0e-20])
def test_bf16_bits_round_trip(v):
    b = oracle.f64_to_bf16_bits(np.array([v]))
    back = oracle.bf16_bits_to_f32(b)[0]
    assert back == np.float32(oracle.round_to_bf16(np.array([v]))[0])
    assert np.signbit(back) == np.signbit(v)
