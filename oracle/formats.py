"""Element formats used by NVFP4: E2M1 values, E4M3 (FN) block scales, BF16.

Test infrastructure (see the package docstring): plain table-driven code, float64 throughout.
"""

import numpy as np

# Megatron-Core "core.inference.moe.flashinfer_nvfp4", module data: the three format constants.
NVFP4_BLOCK_SIZE = 16
FLOAT4_E2M1_MAX = 6.0
FLOAT8_E4M3_MAX = 448.0

# E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit.  Code s.e1e0.m has magnitude
# m*0.5 when e == 0 and (1 + m/2) * 2**(e-1) otherwise.  Written out by magnitude code 0..7.
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def e2m1_decode(codes):
    """4-bit E2M1 codes (0..15, any integer array) -> float64 values (sign bit 3)."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def _e4m3_value(code):
    """One E4M3FN code -> float (NaN for S.1111.111).  Bias 7, 3 mantissa bits, no infinities."""
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 0xF and m == 7:
        return float("nan")
    if e == 0:
        v = (m / 8.0) * 2.0 ** -6
    else:
        v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes):
    """uint8 E4M3FN codes -> float64 values."""
    return E4M3_TABLE[np.asarray(codes).astype(np.int64) & 0xFF]


# Non-negative finite E4M3 values in code order 0x00..0x7E; the table is increasing.
_E4M3_POS = E4M3_TABLE[:0x7F].copy()


def _nearest_on_grid(mag, grid):
    """Index of the nearest grid value for each non-negative magnitude, ties to the even index.

    ``grid`` is increasing and its index is the code, so "even index" is "even code".  Values
    above the last grid point map to the last one (saturation).
    """
    mag = np.asarray(mag, dtype=np.float64)
    hi = np.searchsorted(grid, mag, side="left")          # first grid value >= mag
    hi = np.clip(hi, 0, len(grid) - 1)
    lo = np.clip(hi - 1, 0, len(grid) - 1)
    d_lo = mag - grid[lo]                                   # exact: few significant bits each
    d_hi = grid[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(mag >= grid[-1], len(grid) - 1, idx)
    return idx.astype(np.int64)


def e4m3_encode(v):
    """Non-negative finite float32 values -> E4M3FN codes (uint8).

    The pages name the scale type (torch.float8_e4m3fn on the alphamoe_nvfp4_aligned_moe page)
    but not its rounding; reading taken: round to nearest on the E4M3 grid (subnormal step
    2**-9), ties to the even code, saturating at FLOAT8_E4M3_MAX = 448.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(~np.isfinite(v)) or np.any(v < 0):
        raise ValueError("e4m3_encode expects finite non-negative values")
    return _nearest_on_grid(v, _E4M3_POS).astype(np.uint8)


def e2m1_encode(y):
    """float32 values -> 4-bit E2M1 codes (uint8, 0..15).

    Reading taken (the pages are silent): magnitude rounds to the nearest of the eight E2M1
    magnitudes with ties to the even code, saturating at FLOAT4_E2M1_MAX = 6; the sign bit is
    the IEEE sign bit of the input, so -0.0 and tiny negatives give code 0x8.
    """
    y = np.asarray(y, dtype=np.float32)
    if np.any(~np.isfinite(y)):
        raise ValueError("e2m1_encode expects finite values")
    code = _nearest_on_grid(np.abs(y.astype(np.float64)), E2M1_MAGNITUDES)
    code = code | np.where(np.signbit(y), 8, 0)
    return code.astype(np.uint8)


def bf16_bits_to_f32(bits):
    """uint16 BF16 bit patterns -> float32 values (exact)."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def round_to_bf16(x):
    """Round float64 values to the nearest BF16 value, ties to even; returns float64.

    BF16 keeps 8 significant bits and the float32 exponent range; below 2**-126 the spacing is
    2**-133 (subnormals).  Written as: quantum = 2**max(e-8, -133) where |x| = m*2**e with
    0.5 <= m < 1, then rint (round half to even) of x/quantum.  Infinities and NaN pass through.
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0)
    _, e = np.frexp(x[fin])
    qexp = np.maximum(e - 8, -133)
    out[fin] = np.ldexp(np.rint(np.ldexp(x[fin], -qexp)), qexp)
    # Values past the largest BF16 (0x7F7F) overflow to infinity.
    big = np.abs(out) > np.ldexp(255.0, 120)
    out[big & fin] = np.copysign(np.inf, x[big & fin])
    return out


def f64_to_bf16_bits(x):
    """Round float64 to BF16 (as round_to_bf16) and return the uint16 bit patterns."""
    r = round_to_bf16(x).astype(np.float32)   # exact: a BF16 value is a float32 value
    return (r.view(np.uint32) >> 16).astype(np.uint16)
