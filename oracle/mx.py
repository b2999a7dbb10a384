"""MXFP4: E2M1 values with one E8M0 (power-of-two) scale per 32 consecutive values.

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
"""

import numpy as np

from .formats import e2m1_decode, e2m1_encode
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
