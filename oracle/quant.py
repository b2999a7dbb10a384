"""NVFP4 quantization: packed E2M1 values, linear E4M3 scales per 16 values, one FP32 scale.

Test infrastructure (see the package docstring).

The steps follow the pages' description of the format:
* blocks of NVFP4_BLOCK_SIZE = 16 consecutive values along a row, each with one E4M3 scale,
  stored in row order without swizzling (alphamoe_nvfp4_aligned_moe page, layout paragraph);
* one FP32 scale per token (Megatron-Core flashinfer_nvfp4 module text, and
  quantize_routed_nvfp4_input), one per weight matrix of each expert (the same module,
  _global_encode_scale), or a fixed global scale of one for the BF16 intermediate
  (CudnnGroupedGemmNvfp4Config page, permutation bullet);
* the FP32 scale handed back is the *decode* scale, one per token (vLLM flashinfer_utils,
  quantize_nvfp4_per_token_input);
* packing: two E2M1 per byte, even logical value in the low nibble (alphamoe page).

Readings taken where the pages are silent (every FP32 step rounds to nearest even, as numpy
float32 arithmetic does; no fused multiply-add):
1. encode scale  s_enc = fl32(FLOAT8_E4M3_MAX * FLOAT4_E2M1_MAX / amax) = fl32(2688 / amax) over
   the row (per-row) or the group of rows (per-group); s_enc = 1 when amax == 0.  A row or group
   with 0 < amax < 2**-106 (about 1.2e-32) is outside the contract, like non-finite input: there
   s_enc / sfv can overflow float32 for the smallest block scales.  Fixed mode uses s_enc = c.
   The decode scale returned is fl32(1 / s_enc).
2. block scale  v = fl32(fl32(bmax * s_enc) / 6), code sf = e4m3_encode(v), value sfv.
3. element  inv = 0 if sfv == 0 else fl32(s_enc / sfv);  code = e2m1_encode(fl32(x * inv)).
A dequantized element is e2m1(code) * sfv * s_dec.
"""

import numpy as np

from .formats import (
    FLOAT4_E2M1_MAX,
    FLOAT8_E4M3_MAX,
    NVFP4_BLOCK_SIZE,
    e2m1_decode,
    e2m1_encode,
    e4m3_decode,
    e4m3_encode,
)

SCALE_PER_ROW = 0
SCALE_PER_GROUP = 1
SCALE_FIXED = 2

_F32_MAX = np.float32(np.finfo(np.float32).max)


def _encode_scale(amax):
    """Step 1: FP32 encode scale from an FP32 amax (array)."""
    amax = np.asarray(amax, dtype=np.float32)
    if np.any((amax > 0) & (amax < np.float32(2.0 ** -106))):
        raise ValueError("0 < amax < 2**-106 is outside the quantizer's contract")
    num = np.float32(FLOAT8_E4M3_MAX) * np.float32(FLOAT4_E2M1_MAX)     # 2688, exact
    with np.errstate(divide="ignore", over="ignore"):
        s = num / np.where(amax == 0, np.float32(1), amax)               # float32 division
    s = np.where(amax == 0, np.float32(1), s)
    s = np.where(np.isinf(s), _F32_MAX, s).astype(np.float32)
    return s


def quantize_rows(x, s_enc):
    """Steps 2-3 for a float32 matrix x [R, C] with one float32 encode scale per row [R].

    Returns (q uint8 [R, C/2], sf uint8 [R, C/16]).
    """
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    if C % NVFP4_BLOCK_SIZE:
        raise ValueError("columns must be a multiple of 16")
    s_enc = np.asarray(s_enc, dtype=np.float32).reshape(R, 1, 1)
    blocks = x.reshape(R, C // NVFP4_BLOCK_SIZE, NVFP4_BLOCK_SIZE)
    bmax = np.max(np.abs(blocks), axis=2, keepdims=True)                     # exact
    v = (bmax * s_enc).astype(np.float32) / np.float32(FLOAT4_E2M1_MAX)      # two fp32 roundings
    sf = e4m3_encode(v.astype(np.float32).reshape(R, -1))                    # [R, C/16]
    sfv = e4m3_decode(sf).astype(np.float32).reshape(R, -1, 1)               # exact
    with np.errstate(divide="ignore", invalid="ignore"):
        inv = np.where(sfv == 0, np.float32(0), s_enc / np.where(sfv == 0, np.float32(1), sfv))
    inv = inv.astype(np.float32)
    y = (blocks * inv).astype(np.float32)                                    # fp32 rounding
    codes = e2m1_encode(y.reshape(R, C))
    q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)           # even value low
    return q, sf


def quantize_nvfp4(x, mode=SCALE_PER_ROW, group_rows=None, fixed_encode_scale=1.0):
    """Quantize a float32 (or BF16-valued) matrix x [R, C] to NVFP4.

    mode SCALE_PER_ROW: one scale per row; returns dec_scale [R].
    mode SCALE_PER_GROUP: one scale per group of ``group_rows`` consecutive rows (one expert
        matrix); returns dec_scale [R // group_rows].
    mode SCALE_FIXED: encode scale ``fixed_encode_scale``; returns dec_scale [1].
    Returns (q uint8 [R, C/2], sf uint8 [R, C/16], dec_scale float32).
    """
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input is outside the quantizer's contract")
    R, C = x.shape
    if mode == SCALE_PER_ROW:
        amax = np.max(np.abs(x), axis=1) if C else np.zeros(R, np.float32)
        s_enc = _encode_scale(amax)
        s_row = s_enc
    elif mode == SCALE_PER_GROUP:
        if not group_rows or R % group_rows:
            raise ValueError("rows must be a whole number of groups")
        amax = np.max(np.abs(x.reshape(R // group_rows, -1)), axis=1)
        s_enc = _encode_scale(amax)
        s_row = np.repeat(s_enc, group_rows)
    elif mode == SCALE_FIXED:
        s_enc = np.array([fixed_encode_scale], dtype=np.float32)
        s_row = np.full(R, s_enc[0], dtype=np.float32)
    else:
        raise ValueError("unknown scale mode")
    dec = (np.float32(1) / s_enc).astype(np.float32)
    q, sf = quantize_rows(x, s_row)
    return q, sf, dec


def unpack_codes(q):
    """Packed bytes [R, C/2] -> E2M1 codes [R, C] (even value from the low nibble)."""
    q = np.asarray(q, dtype=np.uint8)
    R, Ch = q.shape
    codes = np.empty((R, 2 * Ch), dtype=np.uint8)
    codes[:, 0::2] = q & 0xF
    codes[:, 1::2] = q >> 4
    return codes


def dequantize_nvfp4(q, sf, dec_scale_rows=None):
    """Packed NVFP4 -> float64 values e2m1(code) * sfv [* dec_scale per row]."""
    codes = unpack_codes(q)
    R, C = codes.shape
    vals = e2m1_decode(codes) * np.repeat(e4m3_decode(sf), NVFP4_BLOCK_SIZE, axis=1)
    if dec_scale_rows is not None:
        vals = vals * np.asarray(dec_scale_rows, dtype=np.float64).reshape(R, 1)
    return vals


def dequantize_int(q, sf):
    """Packed NVFP4 -> int64 n with e2m1(code) * sfv == n * 2**-10 exactly.

    2*e2m1 magnitude is an integer in {0,1,2,3,4,6,8,12} and every E4M3 value is a multiple of
    2**-9 (its subnormal step), so their product is an integer times 2**-10, |n| < 2**22.
    """
    codes = unpack_codes(q).astype(np.int64)
    two_v = np.array([0, 1, 2, 3, 4, 6, 8, 12], dtype=np.int64)[codes & 7]
    two_v = np.where((codes & 8) != 0, -two_v, two_v)
    sfv = e4m3_decode(sf)
    if np.any(np.isnan(sfv)):
        raise ValueError("NaN block scale")
    sf_int = np.rint(sfv * 512.0).astype(np.int64)                   # exact integers
    return two_v * np.repeat(sf_int, NVFP4_BLOCK_SIZE, axis=1)
