"""MXFP4 and MXFP8: E2M1 or E4M3 values with one E8M0 (power-of-two) scale per 32 values.

Test infrastructure (see the package docstring).

What the pages fix: FrostLowLatencyConfig, FP4 weight-only paragraph: MXFP4 weights keep
canonical E2M1 payloads with E8M0 scales per 32 K values and are dequantized in FP32; the vLLM
flashinfer_utils page: UE8M0 block scales, 127 encoding 1.0.  The packing (two E2M1 per byte, the
even value in the low nibble) is the one of NVFP4.

Reading taken for the quantization recipe, which the pages do not spell out (the OCP
microscaling one): per block of 32 values with amax = max |x|,
* amax == 0: scale code 0 (2**-127), every element code 0 (0x8 for a negative zero);
* otherwise the shared exponent X = floor(log2(amax)) - 2 (2 = the exponent of the largest E2M1
  magnitude, 6 = 1.5 * 2**2), clamped to [-127, 127]; scale code X + 127;
* element codes e2m1_encode(fl32(x * 2**-X)) (exact power-of-two scaling; round to nearest,
  ties to even, saturating at 6).
A dequantized element is e2m1(code) * 2**(scale code - 127); code 255 (NaN) is never produced.

MXFP8 (FrostLowLatencyConfig, MX paragraph: MXFP4 or MXFP8 weights run with MXFP8 inputs): E4M3
elements (bias 7, largest magnitude 448 = 1.75 * 2**8) with one E8M0 scale per 32 values.
Reading taken for its quantization (the same OCP microscaling recipe, with the element format's
largest exponent 8 in place of E2M1's 2): amax == 0 gives scale code 0 and zero codes (0x80 for a
negative zero); otherwise X = floor(log2(amax)) - 8 clamped to [-127, 127], scale code X + 127,
and element codes are E4M3 of x * 2**-X (exact power-of-two scaling), rounded to the nearest E4M3
value with ties to the even code and saturating at 448, the sign bit copied from the input.
"""

import numpy as np

from .formats import _E4M3_POS, _nearest_on_grid, e2m1_decode, e2m1_encode, e4m3_decode
from .quant import unpack_codes

MX_BLOCK_SIZE = 32


def e8m0_decode(codes):
    """UE8M0 codes -> float64 scales 2**(code - 127); code 255 is NaN."""
    c = np.asarray(codes).astype(np.int64)
    v = np.ldexp(1.0, c - 127)
    return np.where(c == 255, np.nan, v)


def quantize_mxfp4(x):
    """float32 [R, C] (C % 32 == 0) -> (q uint8 [R, C/2], sf uint8 [R, C/32])."""
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    if C % MX_BLOCK_SIZE:
        raise ValueError("columns must be a multiple of 32")
    if np.any(~np.isfinite(x)):
        raise ValueError("non-finite input")
    blocks = x.reshape(R, C // MX_BLOCK_SIZE, MX_BLOCK_SIZE)
    amax = np.abs(blocks).max(axis=2).astype(np.float64)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))).astype(np.int64)
    X = np.clip(e - 2, -127, 127)
    code = np.where(amax > 0, X + 127, 0).astype(np.uint8)
    Xe = np.where(amax > 0, X, 0)
    scaled = (blocks.astype(np.float64) * np.ldexp(1.0, -Xe)[..., None]).astype(np.float32)
    codes = e2m1_encode(scaled).reshape(R, C)
    q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return q, code


def dequantize_mxfp4(q, sf):
    """(q [R, C/2], sf [R, C/32]) -> float64 [R, C]."""
    v = e2m1_decode(unpack_codes(q))
    return v * np.repeat(e8m0_decode(sf), MX_BLOCK_SIZE, axis=1)


E4M3_EMAX = 8          # exponent of the largest E4M3 magnitude, 448 = 1.75 * 2**8


def _mx_shared_exponent(blocks, emax):
    """Per-block shared exponent X = floor(log2 amax) - emax (clamped to [-127, 127]) and scale
    code (0 for an all-zero block, whose X is taken as 0 for the element step)."""
    amax = np.abs(blocks).max(axis=2).astype(np.float64)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))).astype(np.int64)
    X = np.clip(e - emax, -127, 127)
    code = np.where(amax > 0, X + 127, 0).astype(np.uint8)
    return np.where(amax > 0, X, 0), code


def quantize_mxfp8(x):
    """float32 [R, C] (C % 32 == 0) -> (q uint8 [R, C] E4M3FN codes, sf uint8 [R, C/32] E8M0)."""
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    if C % MX_BLOCK_SIZE:
        raise ValueError("columns must be a multiple of 32")
    if np.any(~np.isfinite(x)):
        raise ValueError("non-finite input")
    blocks = x.reshape(R, C // MX_BLOCK_SIZE, MX_BLOCK_SIZE)
    Xe, code = _mx_shared_exponent(blocks, E4M3_EMAX)
    scaled = (blocks.astype(np.float64) * np.ldexp(1.0, -Xe)[..., None]).reshape(R, C)
    mag = _nearest_on_grid(np.abs(scaled), _E4M3_POS)
    q = (mag | np.where(np.signbit(x.reshape(R, C)), 0x80, 0)).astype(np.uint8)
    return q, code


def dequantize_mxfp8(q, sf):
    """(q [R, C] E4M3 codes, sf [R, C/32]) -> float64 [R, C]."""
    return e4m3_decode(q) * np.repeat(e8m0_decode(sf), MX_BLOCK_SIZE, axis=1)


def mx_dot(a_int, a_exp, w_int, w_exp):
    """Exact products of MX operands, summed exactly and rounded once to float64.

    a_int [R, C] and w_int [N, C]: integer element values (the element times a power of two that
    makes it an integer), a_exp [R, C/32] and w_exp [N, C/32]: the power of two that each 32-value
    block's integers carry (its E8M0 scale times the element's integer step).  Per block the sum
    is an exact int64; the blocks are then added exactly: in float64 when every block term is a
    multiple of the smallest block unit and the total stays below 2**53 units, else with
    math.fsum (the correctly rounded sum).  Returns float64 [R, N].
    """
    import math

    R, C = a_int.shape
    N = w_int.shape[0]
    nb = C // MX_BLOCK_SIZE
    S = np.einsum("rbk,nbk->rnb", a_int.reshape(R, nb, MX_BLOCK_SIZE).astype(np.int64),
                  w_int.reshape(N, nb, MX_BLOCK_SIZE).astype(np.int64))
    e = a_exp.astype(np.int64)[:, None, :] + w_exp.astype(np.int64)[None, :, :]
    emin = e.min(axis=2, keepdims=True)
    big = int(np.abs(S).max(initial=0)).bit_length()
    spread = (e - emin).max(axis=2)
    ok = spread + big + int(nb).bit_length() <= 53
    units = S.astype(np.float64) * np.ldexp(1.0, e - emin)          # exact integers
    out = np.ldexp(units.sum(axis=2), emin[..., 0])
    if not np.all(ok):
        terms = S.astype(np.float64) * np.ldexp(1.0, e)
        for r, n in zip(*np.nonzero(~ok)):
            out[r, n] = math.fsum(terms[r, n])
    return out


def mxfp8_int(q, sf):
    """MXFP8 operand as (integers [R, C], block exponents [R, C/32]): E4M3 values are multiples of
    2**-9, so value = int * 2**(scale - 127 - 9)."""
    v = e4m3_decode(q)
    n = np.rint(v * 512.0).astype(np.int64)
    return n, sf.astype(np.int64) - 127 - 9


def mxfp4_int(q, sf):
    """MXFP4 operand as (integers [R, C], block exponents [R, C/32]): E2M1 values are multiples
    of 1/2, so value = int * 2**(scale - 127 - 1)."""
    v = e2m1_decode(unpack_codes(q))
    n = np.rint(v * 2.0).astype(np.int64)
    return n, sf.astype(np.int64) - 127 - 1
